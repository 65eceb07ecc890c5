// Calibrated sparse-tree construction (Medusa paper digest, Method 4
// "Optimized sparse tree", paper section 2.3.3; Pitfalls: heads taken as
// independent).  A node with rank path (i_1..i_k) is estimated to be
// accepted with probability a[0][i_1] * ... * a[k-1][i_k]; the expected
// acceptance length of a tree is the sum of its nodes' estimates; the tree
// grows from the root by repeatedly taking the connected node with the
// highest estimate.  Ties go to the lexicographically smaller rank path.
// Host code: a binary heap over the frontier (children of chosen nodes).
#include <stdint.h>
#include <math.h>

#include <algorithm>
#include <queue>
#include <vector>

#include "medusa_verify.h"
#include "internal.hpp"

using mv::fail;

namespace {
struct Node {
  double value;                 // product of accuracies, left to right along the path
  std::vector<int32_t> path;
};
// heap order: the top is the highest value, then the smaller path
struct Worse {
  bool operator()(const Node& a, const Node& b) const {
    if (a.value != b.value) return a.value < b.value;
    return std::lexicographical_compare(b.path.begin(), b.path.end(), a.path.begin(),
                                        a.path.end());
  }
};
bool depth_then_path(const std::vector<int32_t>& a, const std::vector<int32_t>& b) {
  if (a.size() != b.size()) return a.size() < b.size();
  return a < b;
}
int check_acc(const double* acc, int32_t K, int32_t s) {
  if (!acc) return fail(MV_EINVAL, "acc is NULL");
  if (K < 1 || K > MV_MAX_DEPTH || s < 1 || s > MV_MAX_TOPK)
    return fail(MV_EINVAL, "accuracy table %dx%d outside [1,%d]x[1,%d]", K, s, MV_MAX_DEPTH,
                MV_MAX_TOPK);
  for (int i = 0; i < K * s; ++i)
    if (!(acc[i] >= 0.0 && acc[i] <= 1.0))
      return fail(MV_EINVAL, "accuracy a[%d][%d] = %g outside [0, 1]", i / s, i % s, acc[i]);
  return MV_OK;
}
}  // namespace

extern "C" {

MV_API int mv_tree_build_sparse(const double* acc, int32_t K, int32_t s, int32_t n_nodes,
                                int32_t max_depth, int32_t* paths, int32_t* path_len,
                                int32_t* n_out, double* expected_len) {
  int rc = check_acc(acc, K, s);
  if (rc) return rc;
  if (n_nodes < 0 || n_nodes > MV_MAX_T - 1)
    return fail(MV_EINVAL, "n_nodes=%d outside [0,%d]", n_nodes, MV_MAX_T - 1);
  if (max_depth < 1 || max_depth > MV_MAX_DEPTH) return fail(MV_EINVAL, "max_depth=%d", max_depth);
  if ((n_nodes > 0 && (!paths || !path_len)) || !n_out)
    return fail(MV_EINVAL, "mv_tree_build_sparse: NULL output");
  const int depth = std::min<int>(max_depth, K);
  std::priority_queue<Node, std::vector<Node>, Worse> frontier;
  for (int i = 0; i < s; ++i) frontier.push(Node{acc[i], {i}});
  std::vector<Node> chosen;
  while ((int)chosen.size() < n_nodes && !frontier.empty()) {
    Node best = frontier.top();
    frontier.pop();
    if ((int)best.path.size() < depth) {
      const double* row = acc + (size_t)best.path.size() * s;
      for (int i = 0; i < s; ++i) {
        Node c{best.value * row[i], best.path};
        c.path.push_back(i);
        frontier.push(std::move(c));
      }
    }
    chosen.push_back(std::move(best));
  }
  std::sort(chosen.begin(), chosen.end(),
            [](const Node& a, const Node& b) { return depth_then_path(a.path, b.path); });
  double sum = 0.0;
  for (size_t v = 0; v < chosen.size(); ++v) {
    const Node& nd = chosen[v];
    for (int j = 0; j < max_depth; ++j)
      paths[v * max_depth + j] = j < (int)nd.path.size() ? nd.path[j] : -1;
    path_len[v] = (int32_t)nd.path.size();
  }
  // the sum in the returned (flattened) order
  for (const Node& nd : chosen) sum += nd.value;
  *n_out = (int32_t)chosen.size();
  if (expected_len) *expected_len = sum;
  return MV_OK;
}

MV_API int mv_tree_expected_length(const double* acc, int32_t K, int32_t s, const int32_t* paths,
                                   const int32_t* path_len, int32_t n_paths, int32_t ld,
                                   double* out) {
  int rc = check_acc(acc, K, s);
  if (rc) return rc;
  if (n_paths < 0 || (n_paths > 0 && (!paths || !path_len)) || !out || ld < 1)
    return fail(MV_EINVAL, "mv_tree_expected_length: bad arguments");
  double sum = 0.0;
  for (int v = 0; v < n_paths; ++v) {
    const int len = path_len[v];
    if (len < 1 || len > K || len > ld) return fail(MV_ETREE, "path %d has length %d", v, len);
    double val = 1.0;
    for (int j = 0; j < len; ++j) {
      const int r = paths[(size_t)v * ld + j];
      if (r < 0 || r >= s) return fail(MV_ETREE, "path %d has rank %d at depth %d", v, r, j + 1);
      val = val * acc[(size_t)j * s + r];
    }
    sum += val;
  }
  *out = sum;
  return MV_OK;
}

}  // extern "C"
