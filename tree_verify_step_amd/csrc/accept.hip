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
// All decision arithmetic (thresholds, probabilities, sums) is double.
#include "common.hpp"

namespace mvk {

__device__ __forceinline__ bool better_iv(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide (256 threads) argmax with lowest-index ties; result in all threads.
__device__ __forceinline__ void block_argmax(float& bv, int& bi) {
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
  bv = rv[0];
  bi = ri[0];
  for (int w = 1; w < 4; ++w)
    if (better_iv(rv[w], ri[w], bv, bi)) {
      bv = rv[w];
      bi = ri[w];
    }
  __syncthreads();
}

__device__ __forceinline__ double block_sum_d(double v) {
  __shared__ double rd[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = warp_sum_d(v);
  if (lane == 0) rd[wave] = v;
  __syncthreads();
  v = rd[0] + rd[1] + rd[2] + rd[3];
  __syncthreads();
  return v;
}

// h[c] = bf16(x[c] * rsqrt(mean(x^2) + 1e-5) * g[c]) for one row of width d
// (the final RMSNorm of the carried hidden state).  Whole workgroup calls it.
// Thread t owns columns 4t + 1024i .. +3; up to NORM_PASSES passes are held
// in registers, so the row is read once, and the gains (which do not depend
// on the row) can be requested before the row is known (norm_gains).
constexpr int NORM_PASSES = 8;                 // d <= 8192 on the register path
struct NormGains {
  uint2 g[NORM_PASSES];
};
__device__ __forceinline__ NormGains norm_gains(const u16* __restrict__ g, int d) {
  NormGains ng;
#pragma unroll
  for (int i = 0; i < NORM_PASSES; ++i) {
    const int c = threadIdx.x * 4 + i * 1024;
    ng.g[i] = (g && c < d && d <= NORM_PASSES * 1024) ? *reinterpret_cast<const uint2*>(g + c)
                                                      : uint2{0u, 0u};
  }
  return ng;
}
__device__ void block_norm_row(const float* __restrict__ xr, const u16* __restrict__ g,
                               const NormGains& ng, u16* __restrict__ h, int d) {
  __shared__ float rf[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool regs = d <= NORM_PASSES * 1024;
  float4 xv[NORM_PASSES];
  float sq = 0.f;
  if (regs) {
#pragma unroll
    for (int i = 0; i < NORM_PASSES; ++i) {
      const int c = threadIdx.x * 4 + i * 1024;
      xv[i] = c < d ? *reinterpret_cast<const float4*>(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < NORM_PASSES; ++i)
      sq += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
  } else {
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      sq += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  sq = warp_sum(sq);
  if (lane == 0) rf[wave] = sq;
  __syncthreads();
  sq = rf[0] + rf[1] + rf[2] + rf[3];
  __syncthreads();
  const float rs = 1.0f / sqrtf(sq / (float)d + 1e-5f);
  if (regs) {
#pragma unroll
    for (int i = 0; i < NORM_PASSES; ++i) {
      const int c = threadIdx.x * 4 + i * 1024;
      if (c >= d) continue;
      const uint2 gw = ng.g[i];
      const uint32_t lo = (uint32_t)f32_to_bf16(xv[i].x * rs * bf16lo(gw.x)) |
                          ((uint32_t)f32_to_bf16(xv[i].y * rs * bf16hi(gw.x)) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(xv[i].z * rs * bf16lo(gw.y)) |
                          ((uint32_t)f32_to_bf16(xv[i].w * rs * bf16hi(gw.y)) << 16);
      *reinterpret_cast<uint2*>(h + c) = uint2{lo, hi};
    }
  } else {
    for (int c = threadIdx.x; c < d; c += 256) h[c] = f32_to_bf16(xr[c] * rs * bf16_to_f32(g[c]));
  }
}

// Rows are read as float4 (V % 4 == 0), 4 independent loads in flight per
// thread per iteration.
__global__ __launch_bounds__(256) void row_stats_kernel(const float* __restrict__ logits, int V,
                                                        int mode, double temperature,
                                                        int32_t* __restrict__ amax,
                                                        double* __restrict__ stats) {
  const int row = blockIdx.x;
  const float4* z4 = reinterpret_cast<const float4*>(logits + (size_t)row * V);
  const int V4 = V >> 2;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 1024) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = (i0 + u * 256) * 4;
      if (better_iv(v[u].x, id, bv, bi)) { bv = v[u].x; bi = id; }
      if (better_iv(v[u].y, id + 1, bv, bi)) { bv = v[u].y; bi = id + 1; }
      if (better_iv(v[u].z, id + 2, bv, bi)) { bv = v[u].z; bi = id + 2; }
      if (better_iv(v[u].w, id + 3, bv, bi)) { bv = v[u].w; bi = id + 3; }
    }
  }
  block_argmax(bv, bi);
  if (threadIdx.x == 0) amax[row] = bi;
  if (mode != MV_ACCEPT_TYPICAL) return;

  const double inv_t = 1.0 / temperature;
  const double m = (double)bv;
  double S = 0.0;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 1024) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      S += exp(((double)v[u].x - m) * inv_t) + exp(((double)v[u].y - m) * inv_t) +
           exp(((double)v[u].z - m) * inv_t) + exp(((double)v[u].w - m) * inv_t);
  }
  S = block_sum_d(S);
  double Hs = 0.0;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 1024) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double q = exp(((double)e[j] - m) * inv_t) / S;
        Hs += q * log(q + 1e-5);
      }
    }
  }
  Hs = block_sum_d(Hs);
  if (threadIdx.x == 0) {
    stats[(size_t)row * 3 + 0] = m;
    stats[(size_t)row * 3 + 1] = S;
    stats[(size_t)row * 3 + 2] = -Hs;
  }
}

hipError_t launch_row_stats(const float* logits, int rows, int V, int mode, double temperature,
                            int32_t* argmax, double* stats, hipStream_t s) {
  hipLaunchKernelGGL(row_stats_kernel, dim3(rows), dim3(256), 0, s, logits, V, mode, temperature,
                     argmax, stats);
  return hipGetLastError();
}

#define MV_MAXT 256

// Inverse-CDF sample of softmax(z * inv_t) over ids in increasing order:
// the smallest id whose cumulative mass exceeds u (if rounding leaves none,
// the largest id of nonzero mass).  Whole workgroup (256 threads) calls it;
// each thread sums a contiguous chunk of ids (multiple of 4), an exclusive
// prefix over the chunk sums locates the crossing.  Writes *out (and
// |cdf - u| to *margin).
__device__ void block_sample(const float* __restrict__ z, int V, int amax_id, double inv_t,
                             double u, int32_t* out, double* margin) {
  __shared__ double csum[256];
  __shared__ double s_total;
  __shared__ int s_found;
  const double m = (double)z[amax_id];
  const int chunk = (((V + 255) / 256) + 3) & ~3;
  const int c0 = min(V, (int)threadIdx.x * chunk), c1 = min(V, c0 + chunk);
  double part = 0.0;
  for (int i = c0; i < c1; i += 4) {
    const float4 v = *reinterpret_cast<const float4*>(z + i);
    part += exp(((double)v.x - m) * inv_t) + exp(((double)v.y - m) * inv_t) +
            exp(((double)v.z - m) * inv_t) + exp(((double)v.w - m) * inv_t);
  }
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
  if (c0 < c1 && cum / S <= u) {
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
    const float* __restrict__ logits, const int32_t* __restrict__ amax_rows,
    unsigned long long* __restrict__ amax_key, const double* __restrict__ stats, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ depth_of, const int32_t* __restrict__ tok, int T, int V, int depth,
    int mode, int root_mode, double temperature, double eps, double delta,
    const double* __restrict__ u, const int32_t* __restrict__ u_index, int u_stride,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ path, int32_t* __restrict__ best_out,
    int32_t* __restrict__ next_root, int32_t* __restrict__ emitted, double* __restrict__ margin,
    const float* __restrict__ x, const u16* __restrict__ final_norm, u16* __restrict__ h_last,
    int d, int32_t* __restrict__ n_advance) {
  __shared__ unsigned char pass[MV_MAXT], ok[MV_MAXT];
  __shared__ double lq[MV_MAXT], score[MV_MAXT];
  __shared__ int par[MV_MAXT], dep[MV_MAXT], tk[MV_MAXT];   // the tree, staged for the walk
  __shared__ int amax[MV_MAXT];                              // argmax of each of the T rows
  __shared__ int s_best;
  const int b = blockIdx.x;
  const NormGains ng = norm_gains(x && h_last ? final_norm : nullptr, d);
  for (int v = threadIdx.x; v < T; v += 256) {
    par[v] = parent[(size_t)b * T + v];
    dep[v] = depth_of[(size_t)b * T + v];
    tk[v] = tok[(size_t)b * T + v];
    if (amax_key) {         // the LM head's atomic argmax keys; cleared for the next step
      const size_t r = (size_t)b * T + v;
      amax[v] = argmax_key_col(amax_key[r]);
      amax_key[r] = 0ull;
    } else {
      amax[v] = amax_rows[(size_t)b * T + v];
    }
  }
  __syncthreads();
  const int row0 = b * T;
  const double inv_t = 1.0 / temperature;

  // per-edge decisions, one node per thread
  for (int v = threadIdx.x; v < T; v += 256) {
    if (v == 0) {
      pass[0] = 1;
      lq[0] = 0.0;
      if (margin) margin[(size_t)b * (T + 1)] = INFINITY;
      continue;
    }
    const int p = par[v];
    if (mode == MV_ACCEPT_GREEDY) {
      pass[v] = tk[v] == amax[p];
      lq[v] = 0.0;
    } else {
      const double* st = stats + (size_t)(row0 + p) * 3;
      const double zt = (double)logits[(size_t)(row0 + p) * V + tk[v]];
      const double lqv = (zt - st[0]) * inv_t - log(st[1]);
      const double q = exp(lqv);
      const double thr = fmin(eps, delta * exp(-st[2]));
      pass[v] = q > thr;
      lq[v] = lqv;
      if (margin) margin[(size_t)b * (T + 1) + v] = thr != 0.0 ? (q - thr) / thr : INFINITY;
    }
  }
  __syncthreads();
  // every node walks its own ancestor chain (no dependence between nodes):
  // ok = all edges on the root path pass, score = sum of log q from the root
  // down; then the deepest ok node (typical: then the highest score), lowest
  // index among equals, by a block reduction
  {
    const bool typ = mode == MV_ACCEPT_TYPICAL;
    int bv = 0, bd = 0;                 // best node, its depth
    double bs = 0.0;                    // its score
    for (int v = threadIdx.x; v < T; v += 256) {
      int ch[MV_MAX_DEPTH + 1];
      int a = v;
#pragma unroll
      for (int i = 0; i <= MV_MAX_DEPTH; ++i) {
        ch[i] = a;
        if (a > 0) a = (par[a] >= 0 && par[a] < T) ? par[a] : 0;
      }
      bool okv = a == 0;                // reached the root within the depth limit
      double sc = 0.0;
#pragma unroll
      for (int i = MV_MAX_DEPTH; i >= 0; --i)
        if (ch[i] > 0) {
          okv = okv && pass[ch[i]];
          sc += lq[ch[i]];
        }
      ok[v] = okv;
      score[v] = sc;
      if (okv && (dep[v] > bd || (typ && dep[v] == bd && sc > bs))) {
        bv = v;
        bd = dep[v];
        bs = sc;
      }
    }
    // candidates of one thread come in index order, so ties already favour
    // the lower index; across threads compare explicitly
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int ov = __shfl_xor(bv, o, 64), od = __shfl_xor(bd, o, 64);
      const double os = __shfl_xor(bs, o, 64);
      if (od > bd || (od == bd && ((typ && os > bs) || ((!typ || os == bs) && ov < bv)))) {
        bv = ov;
        bd = od;
        bs = os;
      }
    }
    __shared__ int w_v[4], w_d[4];
    __shared__ double w_s[4];
    if ((threadIdx.x & 63) == 0) {
      w_v[threadIdx.x >> 6] = bv;
      w_d[threadIdx.x >> 6] = bd;
      w_s[threadIdx.x >> 6] = bs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < 4; ++w)
        if (w_d[w] > bd || (w_d[w] == bd && ((typ && w_s[w] > bs) || ((!typ || w_s[w] == bs) && w_v[w] < bv)))) {
          bv = w_v[w];
          bd = w_d[w];
          bs = w_s[w];
        }
      s_best = bv;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int best = s_best;
    int nodes[MV_MAX_DEPTH + 1];
    int cnt = 0;
    for (int v = best; v >= 0 && cnt <= MV_MAX_DEPTH; v = (v == 0 ? -1 : par[v])) nodes[cnt++] = v;
    const int L = cnt - 1;
    accept_len[b] = L;
    best_out[b] = best;
    if (n_advance) n_advance[b] += L + 1;       // the accepted tokens join the prefix
    for (int m = 0; m <= depth; ++m) {
      const int node = m <= L ? nodes[L - m] : -1;
      path[(size_t)b * (depth + 1) + m] = node;
      if (emitted) emitted[(size_t)b * (depth + 1) + m] = node >= 0 ? tk[node] : -1;
    }
  }
  __syncthreads();
  const int best = s_best;
  const int brow = row0 + best;

  if (x && h_last) block_norm_row(x + (size_t)brow * d, final_norm, ng, h_last + (size_t)b * d, d);
  if (root_mode == MV_ROOT_ARGMAX) {
    if (threadIdx.x == 0) next_root[b] = amax[best];
    return;
  }
  const double ub = u[(size_t)(u_index ? u_index[0] : 0) * u_stride + b];
  block_sample(logits + (size_t)brow * V, V, amax[best], inv_t, ub, next_root + b,
               margin ? margin + (size_t)b * (T + 1) + T : nullptr);
}

hipError_t launch_accept_finish(const float* logits, const int32_t* argmax, unsigned long long* amax_key,
                                const double* stats,
                                const int32_t* parent, const int32_t* depth_of,
                                const int32_t* tok, int B, int T, int V, int depth, int mode,
                                int root_mode, double temperature, double eps, double delta,
                                const double* u, const int32_t* u_index, int u_stride,
                                int32_t* accept_len, int32_t* path, int32_t* best,
                                int32_t* next_root, int32_t* emitted, double* margin,
                                const float* x, const u16* final_norm, u16* h_last, int d,
                                hipStream_t s, int32_t* n_advance) {
  hipLaunchKernelGGL(accept_finish_kernel, dim3(B), dim3(256), 0, s, logits, argmax, amax_key,
                     stats,
                     parent, depth_of, tok, T, V, depth, mode, root_mode, temperature, eps, delta,
                     u, u_index, u_stride, accept_len, path, best, next_root, emitted, margin, x,
                     final_norm, h_last, d, n_advance);
  return hipGetLastError();
}

// Prefill: after a chain chunk, sequence b's last real row (cnt[b] - 1)
// supplies h_last (its final RMSNorm) and the first root; n[b] += cnt[b].
// cnt[b] == 0: nothing.
__global__ __launch_bounds__(256) void prefill_select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ amax, const int32_t* __restrict__ cnt,
    int T, int V, int root_mode, double temperature, const double* __restrict__ u,
    int32_t* __restrict__ root, int32_t* __restrict__ n_prefix, const float* __restrict__ x,
    const u16* __restrict__ final_norm, u16* __restrict__ h_last, int d) {
  const int b = blockIdx.x;
  const int c = cnt[b];
  if (c <= 0) return;
  const int row = b * T + c - 1;
  block_norm_row(x + (size_t)row * d, final_norm, norm_gains(final_norm, d), h_last + (size_t)b * d, d);
  if (root_mode == MV_ROOT_ARGMAX) {
    if (threadIdx.x == 0) root[b] = amax[row];
  } else {
    block_sample(logits + (size_t)row * V, V, amax[row], 1.0 / temperature, u[(size_t)b], root + b,
                 nullptr);
  }
  __syncthreads();
  if (threadIdx.x == 0) n_prefix[b] += c;
}

hipError_t launch_prefill_select(const float* logits, const int32_t* amax, const int32_t* cnt,
                                 int B, int T, int V, int root_mode, double temperature,
                                 const double* u, int32_t* root, int32_t* n_prefix,
                                 const float* x, const u16* final_norm, u16* h_last, int d,
                                 hipStream_t s) {
  hipLaunchKernelGGL(prefill_select_kernel, dim3(B), dim3(256), 0, s, logits, amax, cnt, T, V,
                     root_mode, temperature, u, root, n_prefix, x, final_norm, h_last, d);
  return hipGetLastError();
}

}  // namespace mvk
