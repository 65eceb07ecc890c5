// Host-side flattening of a candidate tree given as paths of head ranks
// (Medusa paper digest, Method 2-4: the tree is a static preset of top-index
// paths; each node attends to its ancestors only and sits at depth = path
// length).  Node order: root, then (depth, lexicographic path) -- parents
// always precede children, which the acceptance propagation relies on.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <vector>

#include "medusa_verify.h"
#include "internal.hpp"

namespace {
struct PathLess {
  bool operator()(const std::vector<int32_t>& a, const std::vector<int32_t>& b) const {
    if (a.size() != b.size()) return a.size() < b.size();
    return a < b;
  }
};
}  // namespace

extern "C" MV_API int mv_tree_compile(const int32_t* paths, const int32_t* path_len,
                                      int32_t n_paths, int32_t max_len, int32_t topk,
                                      int32_t cap_nodes, int32_t mask_words, int32_t* parent,
                                      int32_t* depth_of, int32_t* rank, uint64_t* anc,
                                      int32_t* T_out) {
  if (n_paths < 0 || max_len < 1 || topk < 1 || (n_paths > 0 && (!paths || !path_len)) ||
      !parent || !depth_of || !rank || !anc || !T_out)
    return mv::fail(MV_EINVAL, "mv_tree_compile: null pointer or bad scalar");
  const int T = n_paths + 1;
  if (T > MV_MAX_T) return mv::fail(MV_ETREE, "mv_tree_compile: %d nodes > %d", T, MV_MAX_T);
  if (cap_nodes < T) return mv::fail(MV_EINVAL, "mv_tree_compile: cap_nodes %d < T %d", cap_nodes, T);
  if (mask_words * 64 < T)
    return mv::fail(MV_EINVAL, "mv_tree_compile: mask_words %d too small for T %d", mask_words, T);

  std::map<std::vector<int32_t>, int, PathLess> index;
  std::vector<std::vector<int32_t>> ps(n_paths);
  for (int p = 0; p < n_paths; ++p) {
    const int len = path_len[p];
    if (len < 1 || len > max_len || len > MV_MAX_T - 1)
      return mv::fail(MV_ETREE, "mv_tree_compile: path %d has length %d", p, len);
    ps[p].assign(paths + (size_t)p * max_len, paths + (size_t)p * max_len + len);
    for (int32_t r : ps[p])
      if (r < 0 || r >= topk)
        return mv::fail(MV_ETREE, "mv_tree_compile: path %d has rank %d outside [0,%d)", p, r, topk);
    if (index.count(ps[p])) return mv::fail(MV_ETREE, "mv_tree_compile: duplicate path %d", p);
    index[ps[p]] = 0;
  }
  for (int p = 0; p < n_paths; ++p) {
    if (ps[p].size() > 1) {
      std::vector<int32_t> pre(ps[p].begin(), ps[p].end() - 1);
      if (!index.count(pre))
        return mv::fail(MV_ETREE, "mv_tree_compile: path %d lacks its parent (not prefix-closed)", p);
    }
  }
  // map is ordered by (length, lexicographic): assign node indices 1..
  int v = 1;
  for (auto& kv : index) kv.second = v++;
  std::vector<int32_t> par(T), dep(T), rk(T);
  par[0] = -1;
  dep[0] = 0;
  rk[0] = 0;
  std::vector<std::vector<int32_t>> byidx(T);
  for (auto& kv : index) {
    const int node = kv.second;
    byidx[node] = kv.first;
    dep[node] = (int32_t)kv.first.size();
    rk[node] = kv.first.back();
    if (kv.first.size() == 1) {
      par[node] = 0;
    } else {
      std::vector<int32_t> pre(kv.first.begin(), kv.first.end() - 1);
      par[node] = index[pre];
    }
  }
  for (int i = 0; i < T; ++i) {
    parent[i] = par[i];
    depth_of[i] = dep[i];
    rank[i] = rk[i];
    uint64_t* w = anc + (size_t)i * mask_words;
    for (int j = 0; j < mask_words; ++j) w[j] = 0;
    for (int a = i; a >= 0; a = par[a]) w[a >> 6] |= 1ull << (a & 63);
  }
  *T_out = T;
  return MV_OK;
}
