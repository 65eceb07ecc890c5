// Acceptance over the verified tree and selection of the next root.
//
// row_stats: one workgroup per tree row of V fp32 logits: argmax (lowest id
// among equal maxima) and, for typical acceptance, the row's tempered softmax
// normaliser and entropy in double precision:
//   q_i = exp((z_i - max)/temp) / S,  S = sum_i exp((z_i - max)/temp),
//   H = -sum_i q_i log(q_i + 1e-5).
// accept_finish: one workgroup per sequence: per-edge decisions (greedy:
// token == argmax of the parent row; typical: q_parent(token) >
// min(eps, delta * exp(-H_parent))), accepted-prefix propagation in node order
// (parents precede children), the deepest accepted node (typical: then the
// larger summed log-probability; then the lower index), its root path, the
// emitted tokens, the next root (argmax of the best row, or inverse-CDF
// sampling of its tempered softmax with the step's uniform draw) and the
// carried hidden state (that row of the final-normed hidden states).
#include "common.hpp"

namespace mvk {

__device__ __forceinline__ bool better_iv(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ logits, int V,
                                                        int mode, float temperature,
                                                        int32_t* __restrict__ amax,
                                                        double* __restrict__ stats) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  __shared__ double rd[4];
  const int row = blockIdx.x;
  const float* z = logits + (size_t)row * V;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float v = z[i];
    if (better_iv(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better_iv(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    rv[wave] = bv;
    ri[wave] = bi;
  }
  __syncthreads();
  float mx = rv[0];
  int mi = ri[0];
  for (int w = 1; w < 4; ++w)
    if (better_iv(rv[w], ri[w], mx, mi)) {
      mx = rv[w];
      mi = ri[w];
    }
  if (threadIdx.x == 0) amax[row] = mi;
  if (mode != MV_ACCEPT_TYPICAL) return;

  const double inv_t = 1.0 / (double)temperature;
  const double m = (double)mx;
  double S = 0.0;
  for (int i = threadIdx.x; i < V; i += 256) S += exp(((double)z[i] - m) * inv_t);
  S = warp_sum_d(S);
  __syncthreads();
  if (lane == 0) rd[wave] = S;
  __syncthreads();
  S = rd[0] + rd[1] + rd[2] + rd[3];
  double Hs = 0.0;
  for (int i = threadIdx.x; i < V; i += 256) {
    const double q = exp(((double)z[i] - m) * inv_t) / S;
    Hs += q * log(q + 1e-5);
  }
  Hs = warp_sum_d(Hs);
  __syncthreads();
  if (lane == 0) rd[wave] = Hs;
  __syncthreads();
  if (threadIdx.x == 0) {
    stats[(size_t)row * 3 + 0] = m;
    stats[(size_t)row * 3 + 1] = S;
    stats[(size_t)row * 3 + 2] = -(rd[0] + rd[1] + rd[2] + rd[3]);
  }
}

hipError_t launch_row_stats(const float* logits, int rows, int V, int mode, float temperature,
                            int32_t* argmax, double* stats, hipStream_t s) {
  hipLaunchKernelGGL(row_stats_kernel, dim3(rows), dim3(256), 0, s, logits, V, mode, temperature,
                     argmax, stats);
  return hipGetLastError();
}

#define MV_MAXT 256

// Inverse-CDF sample of softmax(z * inv_t) over ids in increasing order:
// the smallest id whose cumulative mass exceeds u (if rounding leaves none,
// the largest id of nonzero mass).  Whole workgroup (256 threads) calls it;
// each thread sums a contiguous chunk of ids, an exclusive prefix over the
// chunk sums locates the crossing.  Writes *out (and |cdf - u| to *margin).
__device__ void block_sample(const float* __restrict__ z, int V, int amax_id, double inv_t,
                             double u, int32_t* out, double* margin) {
  __shared__ double csum[256];
  __shared__ double s_total;
  __shared__ int s_found;
  const double m = (double)z[amax_id];
  const int chunk = (V + 255) / 256;
  const int c0 = threadIdx.x * chunk, c1 = min(V, c0 + chunk);
  double part = 0.0;
  for (int i = c0; i < c1; ++i) part += exp(((double)z[i] - m) * inv_t);
  csum[threadIdx.x] = part;
  if (threadIdx.x == 0) s_found = 0x7fffffff;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int t = 0; t < 256; ++t) {
      const double x = csum[t];
      csum[t] = tot;
      tot += x;
    }
    s_total = tot;
  }
  __syncthreads();
  const double S = s_total;
  double cum = csum[threadIdx.x];
  int found = -1;
  double mg = INFINITY;
  if (cum / S <= u) {
    for (int i = c0; i < c1; ++i) {
      const double prev = cum / S;
      cum += exp(((double)z[i] - m) * inv_t);
      if (cum / S > u) {
        found = i;
        mg = fmin(cum / S - u, u - prev);
        break;
      }
    }
  }
  if (found >= 0) atomicMin(&s_found, found);
  __syncthreads();
  if (found >= 0 && found == s_found) {
    *out = found;
    if (margin) *margin = mg;
  }
  if (threadIdx.x == 0 && s_found == 0x7fffffff) {
    int last = V - 1;
    while (last > 0 && exp(((double)z[last] - m) * inv_t) == 0.0) --last;
    *out = last;
    if (margin) *margin = 0.0;
  }
  __syncthreads();
}


__global__ __launch_bounds__(256) void accept_finish_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ amax,
    const double* __restrict__ stats, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ depth_of, const int32_t* __restrict__ tok, int T, int V, int depth,
    int mode, int root_mode, float temperature, float eps, float delta, const double* __restrict__ u,
    const int32_t* __restrict__ u_index, int u_stride, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ best_out, int32_t* __restrict__ next_root,
    int32_t* __restrict__ emitted, double* __restrict__ margin, const u16* __restrict__ hn,
    u16* __restrict__ h_last, int d) {
  __shared__ unsigned char pass[MV_MAXT], ok[MV_MAXT];
  __shared__ double lq[MV_MAXT], score[MV_MAXT];
  __shared__ int s_best;
  const int b = blockIdx.x;
  const int32_t* par = parent + (size_t)b * T;
  const int32_t* dep = depth_of + (size_t)b * T;
  const int32_t* tk = tok + (size_t)b * T;
  const int row0 = b * T;
  const double inv_t = 1.0 / (double)temperature;

  // per-edge decisions
  for (int v = threadIdx.x; v < T; v += 256) {
    if (v == 0) {
      pass[0] = 1;
      lq[0] = 0.0;
      if (margin) margin[(size_t)b * (T + 1)] = INFINITY;
      continue;
    }
    const int p = par[v];
    if (mode == MV_ACCEPT_GREEDY) {
      pass[v] = tk[v] == amax[row0 + p];
      lq[v] = 0.0;
    } else {
      const double* st = stats + (size_t)(row0 + p) * 3;
      const double zt = (double)logits[(size_t)(row0 + p) * V + tk[v]];
      const double lqv = (zt - st[0]) * inv_t - log(st[1]);
      const double q = exp(lqv);
      const double thr = fmin((double)eps, (double)delta * exp(-st[2]));
      pass[v] = q > thr;
      lq[v] = lqv;
      if (margin) margin[(size_t)b * (T + 1) + v] = thr != 0.0 ? (q - thr) / thr : INFINITY;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ok[0] = 1;
    score[0] = 0.0;
    int best = 0;
    for (int v = 1; v < T; ++v) {
      const int p = par[v];
      ok[v] = ok[p] && pass[v];
      score[v] = score[p] + lq[v];
      if (ok[v]) {
        if (dep[v] > dep[best] ||
            (dep[v] == dep[best] && mode == MV_ACCEPT_TYPICAL && score[v] > score[best]))
          best = v;
      }
    }
    // root path
    int nodes[MV_MAX_DEPTH + 1];
    int cnt = 0;
    for (int v = best; v >= 0 && cnt <= MV_MAX_DEPTH; v = (v == 0 ? -1 : par[v])) nodes[cnt++] = v;
    const int L = cnt - 1;
    accept_len[b] = L;
    best_out[b] = best;
    for (int m = 0; m <= depth; ++m) {
      const int node = m <= L ? nodes[L - m] : -1;
      path[(size_t)b * (depth + 1) + m] = node;
      if (emitted) emitted[(size_t)b * (depth + 1) + m] = node >= 0 ? tk[node] : -1;
    }
    s_best = best;
  }
  __syncthreads();
  const int best = s_best;
  const int brow = row0 + best;

  // carried hidden state
  if (hn && h_last) {
    for (int c = threadIdx.x; c < d; c += 256) h_last[(size_t)b * d + c] = hn[(size_t)brow * d + c];
  }

  // next root
  if (root_mode == MV_ROOT_ARGMAX) {
    if (threadIdx.x == 0) next_root[b] = amax[brow];
    return;
  }
  const double ub = u[(size_t)(u_index ? u_index[0] : 0) * u_stride + b];
  block_sample(logits + (size_t)brow * V, V, amax[brow], inv_t, ub, next_root + b,
               margin ? margin + (size_t)b * (T + 1) + T : nullptr);
}

// Prefill: after a chain chunk, sequence b's last real row (cnt[b] - 1)
// supplies h_last and the first root; n[b] += cnt[b].  cnt[b] == 0: nothing.
__global__ __launch_bounds__(256) void prefill_select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ amax, const int32_t* __restrict__ cnt,
    int T, int V, int root_mode, float temperature, const double* __restrict__ u, int u_stride,
    int32_t* __restrict__ root, int32_t* __restrict__ n_prefix, const u16* __restrict__ hn,
    u16* __restrict__ h_last, int d) {
  const int b = blockIdx.x;
  const int c = cnt[b];
  if (c <= 0) return;
  const int row = b * T + c - 1;
  for (int i = threadIdx.x; i < d; i += 256) h_last[(size_t)b * d + i] = hn[(size_t)row * d + i];
  if (root_mode == MV_ROOT_ARGMAX) {
    if (threadIdx.x == 0) root[b] = amax[row];
  } else {
    block_sample(logits + (size_t)row * V, V, amax[row], 1.0 / (double)temperature,
                 u[(size_t)b], root + b, nullptr);
  }
  __syncthreads();
  if (threadIdx.x == 0) n_prefix[b] += c;
}

hipError_t launch_prefill_select(const float* logits, const int32_t* amax, const int32_t* cnt,
                                 int B, int T, int V, int root_mode, float temperature,
                                 const double* u, int32_t* root, int32_t* n_prefix, const u16* hn,
                                 u16* h_last, int d, hipStream_t s) {
  hipLaunchKernelGGL(prefill_select_kernel, dim3(B), dim3(256), 0, s, logits, amax, cnt, T, V,
                     root_mode, temperature, u, 0, root, n_prefix, hn, h_last, d);
  return hipGetLastError();
}

hipError_t launch_accept_finish(const float* logits, const int32_t* argmax, const double* stats,
                                const int32_t* parent, const int32_t* depth_of,
                                const int32_t* tok, int B, int T, int V, int depth, int mode,
                                int root_mode, float temperature, float eps, float delta,
                                const double* u, const int32_t* u_index, int u_stride,
                                int32_t* accept_len, int32_t* path, int32_t* best,
                                int32_t* next_root, int32_t* emitted, double* margin,
                                const u16* hn, u16* h_last, int d, hipStream_t s) {
  hipLaunchKernelGGL(accept_finish_kernel, dim3(B), dim3(256), 0, s, logits, argmax, stats,
                     parent, depth_of, tok, T, V, depth, mode, root_mode, temperature, eps, delta,
                     u, u_index, u_stride, accept_len, path, best, next_root, emitted, margin, hn,
                     h_last, d);
  return hipGetLastError();
}

}  // namespace mvk
