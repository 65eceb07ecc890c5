// Host-only entry points of the library (tree flattening, calibrated sparse
// tree, expected acceptance length) driven through valid and invalid inputs,
// built with the address and undefined-behaviour sanitizers by
// tests/test_host_sanitizers.py.  Exit status 0 iff every call returned what
// it should and the outputs satisfy the tree invariants; the sanitizers abort
// on any memory or UB error.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "medusa_verify.h"

// the error-text buffer lives in the device-side translation unit of the
// library; this harness links only the host sources
namespace mv {
char* last_error_buf() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace mv

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

struct Paths {
  std::vector<int32_t> flat, len;
  int max_len = 1;
};

static Paths make(const std::vector<std::vector<int32_t>>& ps) {
  Paths p;
  for (auto& x : ps) p.max_len = std::max<int>(p.max_len, (int)x.size());
  p.flat.assign(std::max<size_t>(ps.size(), 1) * p.max_len, 0);
  p.len.assign(std::max<size_t>(ps.size(), 1), 0);
  for (size_t i = 0; i < ps.size(); ++i) {
    for (size_t j = 0; j < ps[i].size(); ++j) p.flat[i * p.max_len + j] = ps[i][j];
    p.len[i] = (int32_t)ps[i].size();
  }
  return p;
}

// compile and check: parents precede children, depth = parent depth + 1,
// ancestor words = own bit | parent's words, nothing past T
static int compile(const std::vector<std::vector<int32_t>>& ps, int topk, int mw_extra = 0) {
  Paths p = make(ps);
  const int n = (int)ps.size(), T = n + 1, mw = (T + 63) / 64 + mw_extra;
  std::vector<int32_t> par(T), dep(T), rk(T);
  std::vector<uint64_t> anc((size_t)T * mw);
  int32_t Tout = -1;
  const int rc = mv_tree_compile(p.flat.data(), p.len.data(), n, p.max_len, topk, T, mw,
                                 par.data(), dep.data(), rk.data(), anc.data(), &Tout);
  if (rc != MV_OK) return rc;
  CHECK(Tout == T);
  CHECK(par[0] == -1 && dep[0] == 0);
  for (int v = 0; v < T; ++v) {
    const uint64_t* w = &anc[(size_t)v * mw];
    CHECK((w[v >> 6] >> (v & 63)) & 1);
    if (v > 0) {
      CHECK(par[v] >= 0 && par[v] < v);
      CHECK(dep[v] == dep[par[v]] + 1);
      CHECK(rk[v] >= 0 && rk[v] < topk);
      const uint64_t* pw = &anc[(size_t)par[v] * mw];
      for (int j = 0; j < mw; ++j) {
        const uint64_t own = (j == (v >> 6)) ? (1ull << (v & 63)) : 0ull;
        CHECK(w[j] == (pw[j] | own));
      }
    }
    for (int a = T; a < mw * 64; ++a) CHECK(!((w[a >> 6] >> (a & 63)) & 1));
  }
  return rc;
}

static std::vector<std::vector<int32_t>> cartesian(const std::vector<int>& widths, int limit) {
  std::vector<std::vector<int32_t>> out, level{{}};
  for (int w : widths) {
    std::vector<std::vector<int32_t>> next;
    for (auto& p : level)
      for (int r = 0; r < w; ++r) {
        auto c = p;
        c.push_back(r);
        next.push_back(c);
      }
    for (auto& c : next)
      if ((int)out.size() < limit) out.push_back(c);
    level = next;
  }
  return out;
}

int main() {
  // valid trees: Cartesian (2,2,2), a 255-candidate truncated (4,4,4,4)
  // (four mask words), a root-only tree, a chain deeper than any head count
  CHECK(compile(cartesian({2, 2, 2}, 1000), 2) == MV_OK);
  CHECK(compile(cartesian({4, 4, 4, 4}, 255), 4) == MV_OK);
  CHECK(compile(cartesian({4, 4, 4, 4}, 255), 4, 1) == MV_OK);   // spare mask word
  CHECK(compile({}, 1) == MV_OK);
  {
    std::vector<std::vector<int32_t>> chain;
    for (int k = 1; k < 200; ++k) chain.push_back(std::vector<int32_t>(k, 0));
    CHECK(compile(chain, 1) == MV_OK);
  }
  // invalid trees: not prefix-closed, duplicate, rank >= topk, negative
  // rank, too many nodes
  CHECK(compile({{0, 1}}, 2) == MV_ETREE);
  CHECK(compile({{0}, {0}}, 2) == MV_ETREE);
  CHECK(compile({{0}, {3}}, 2) == MV_ETREE);
  CHECK(compile({{0}, {-1}}, 2) == MV_ETREE);
  CHECK(compile(cartesian({4, 4, 4, 4, 4}, 300), 4) == MV_ETREE);
  {
    // an empty path (length 0), capacities too small, NULL outputs
    Paths p = make({{0}, {1}});
    p.len[1] = 0;
    std::vector<int32_t> a(3), b(3), c(3);
    std::vector<uint64_t> m(3);
    int32_t T = 0;
    CHECK(mv_tree_compile(p.flat.data(), p.len.data(), 2, p.max_len, 2, 3, 1, a.data(), b.data(),
                          c.data(), m.data(), &T) == MV_ETREE);
    p = make({{0}, {1}});
    CHECK(mv_tree_compile(p.flat.data(), p.len.data(), 2, p.max_len, 2, 2, 1, a.data(), b.data(),
                          c.data(), m.data(), &T) == MV_EINVAL);
    CHECK(mv_tree_compile(p.flat.data(), p.len.data(), 2, p.max_len, 2, 3, 0, a.data(), b.data(),
                          c.data(), m.data(), &T) == MV_EINVAL);
    CHECK(mv_tree_compile(p.flat.data(), p.len.data(), 2, p.max_len, 2, 3, 1, nullptr, b.data(),
                          c.data(), m.data(), &T) == MV_EINVAL);
    CHECK(mv_tree_compile(nullptr, nullptr, 2, p.max_len, 2, 3, 1, a.data(), b.data(), c.data(),
                          m.data(), &T) == MV_EINVAL);
    CHECK(mv_tree_compile(p.flat.data(), p.len.data(), -1, p.max_len, 2, 3, 1, a.data(),
                          b.data(), c.data(), m.data(), &T) == MV_EINVAL);
  }

  // calibrated sparse tree and its expected length
  {
    const int K = 5, s = 10, n = 255, depth = 5;
    std::vector<double> acc(K * s);
    for (int k = 0; k < K; ++k)
      for (int i = 0; i < s; ++i) acc[k * s + i] = 0.6 / (k + 1) * pow(0.5, i);
    std::vector<int32_t> paths((size_t)n * depth, -7), len(n, -7);
    int32_t nout = -1;
    double e = -1.0;
    CHECK(mv_tree_build_sparse(acc.data(), K, s, n, depth, paths.data(), len.data(), &nout, &e) ==
          MV_OK);
    CHECK(nout == n && e > 0.0);
    std::vector<std::vector<int32_t>> ps;
    for (int v = 0; v < nout; ++v) {
      CHECK(len[v] >= 1 && len[v] <= depth);
      ps.emplace_back(paths.begin() + (size_t)v * depth, paths.begin() + (size_t)v * depth + len[v]);
    }
    CHECK(compile(ps, s) == MV_OK);                 // prefix-closed, valid ranks
    double e2 = -1.0;
    CHECK(mv_tree_expected_length(acc.data(), K, s, paths.data(), len.data(), nout, depth, &e2) ==
          MV_OK);
    CHECK(e2 == e);
    // a budget beyond the full tree stops when no node is left
    const int full = 2 + 4 + 8;                     // K = 3, s = 2: 2 + 4 + 8 nodes
    std::vector<int32_t> p2(100 * 3), l2(100);
    CHECK(mv_tree_build_sparse(acc.data(), 3, 2, 100, 3, p2.data(), l2.data(), &nout, nullptr) ==
          MV_OK);
    CHECK(nout == full);
    // invalid tables and sizes
    std::vector<double> bad = acc;
    bad[3] = NAN;
    CHECK(mv_tree_build_sparse(bad.data(), K, s, n, depth, paths.data(), len.data(), &nout, &e) ==
          MV_EINVAL);
    bad[3] = 1.5;
    CHECK(mv_tree_build_sparse(bad.data(), K, s, n, depth, paths.data(), len.data(), &nout, &e) ==
          MV_EINVAL);
    CHECK(mv_tree_build_sparse(acc.data(), K, s, MV_MAX_T, depth, paths.data(), len.data(), &nout,
                               &e) == MV_EINVAL);
    CHECK(mv_tree_build_sparse(acc.data(), MV_MAX_DEPTH + 1, s, n, depth, paths.data(), len.data(),
                               &nout, &e) == MV_EINVAL);
    CHECK(mv_tree_build_sparse(nullptr, K, s, n, depth, paths.data(), len.data(), &nout, &e) ==
          MV_EINVAL);
    // expected length of a path with a rank >= s, or longer than K
    std::vector<int32_t> q = {0, 11};
    std::vector<int32_t> ql = {2};
    CHECK(mv_tree_expected_length(acc.data(), K, s, q.data(), ql.data(), 1, 2, &e2) == MV_ETREE);
    std::vector<int32_t> q6(6, 0), ql6 = {6};
    CHECK(mv_tree_expected_length(acc.data(), K, s, q6.data(), ql6.data(), 1, 6, &e2) == MV_ETREE);
  }
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
