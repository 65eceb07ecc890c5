// Acceptance over the verified tree and selection of the next root.
//
// row_stats: one workgroup per tree row of V fp32 logits: argmax (lowest id
// among equal maxima) and, for typical acceptance, the row's tempered softmax
// normaliser and entropy in double precision:
//   q_i = exp((z_i - max)/temp) / S,  S = sum_i exp((z_i - max)/temp),
//   H = -sum_i q_i log(q_i + 1e-5).
// With e_i = exp((z_i - max)/temp) the entropy is evaluated as
//   H = log S - (1/S) sum_i e_i log(e_i + 1e-5 S),
// the same sum without a division per id.  H only enters the threshold
// through exp(-H), so its absolute error is what counts: a few ulps of
// log S + H, since the subtracted mean is log S - H.
// accept_finish: one workgroup per sequence: per-edge decisions (greedy:
// token == argmax of the parent row; typical: q_parent(token) >
// min(eps, delta * exp(-H_parent))), accepted-prefix propagation in node order
// (parents precede children), the deepest accepted node (typical: then the
// larger summed log-probability; then the lower index), its root path, the
// emitted tokens, the next root (argmax of the best row, or inverse-CDF
// sampling of its tempered softmax with the step's uniform draw) and the
// carried hidden state (that row of the final-normed hidden states).
// reject_accept: one workgroup per sequence walks the tree with the
// speculative-sampling correction (see the kernel).
// All decision arithmetic (thresholds, probabilities, sums) is double.
#include "common.hpp"

namespace mvk {

__device__ __forceinline__ bool better_iv(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide (NW waves) argmax with lowest-index ties; result in all threads.
template <int NW = 4>
__device__ __forceinline__ void block_argmax(float& bv, int& bi) {
  __shared__ float rv[NW];
  __shared__ int ri[NW];
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
  for (int w = 1; w < NW; ++w)
    if (better_iv(rv[w], ri[w], bv, bi)) {
      bv = rv[w];
      bi = ri[w];
    }
  __syncthreads();
}

template <int NW = 4>
__device__ __forceinline__ double block_sum_d(double v) {
  __shared__ double rd[NW];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = warp_sum_d(v);
  if (lane == 0) rd[wave] = v;
  __syncthreads();
  v = rd[0];
  for (int w = 1; w < NW; ++w) v += rd[w];
  __syncthreads();
  return v;
}

// Sum over a wave in a fixed order, the same value in every lane.
__device__ __forceinline__ double wave_total_d(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  return __shfl(v, 0, 64);
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

// Rows are read as float4 (V % 4 == 0) by 1024 threads (four waves per SIMD
// hide the double-precision exp latency), 4 independent loads in flight per
// thread per iteration.  Each wave-iteration covers one 256-id block (a lane
// takes 4 consecutive ids), so the pass that sums the tempered exponentials
// can also store each block's sum (bsum [rows][ceil(V/256)], optional) for
// the inverse-CDF draws.
constexpr int RS_NT = 1024, RS_NW = RS_NT / 64;
__global__ __launch_bounds__(RS_NT) void row_stats_kernel(const float* __restrict__ logits, int V,
                                                          int mode, double temperature,
                                                          int32_t* __restrict__ amax,
                                                          double* __restrict__ stats,
                                                          double* __restrict__ bsum) {
  const int row = blockIdx.x;
  const float4* z4 = reinterpret_cast<const float4*>(logits + (size_t)row * V);
  const int V4 = V >> 2;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 4 * RS_NT) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * RS_NT;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int id = (i0 + u * RS_NT) * 4;
      if (better_iv(v[u].x, id, bv, bi)) { bv = v[u].x; bi = id; }
      if (better_iv(v[u].y, id + 1, bv, bi)) { bv = v[u].y; bi = id + 1; }
      if (better_iv(v[u].z, id + 2, bv, bi)) { bv = v[u].z; bi = id + 2; }
      if (better_iv(v[u].w, id + 3, bv, bi)) { bv = v[u].w; bi = id + 3; }
    }
  }
  block_argmax<RS_NW>(bv, bi);
  // a row of NaNs has no maximum: id 0 keeps every later index in the row
  if (threadIdx.x == 0) amax[row] = (unsigned)bi < (unsigned)V ? bi : 0;
  if (mode == MV_ACCEPT_GREEDY) return;

  const double inv_t = 1.0 / temperature;
  const double m = (double)bv;
  const int nb = (V + 255) >> 8;
  const int lane = threadIdx.x & 63;
  double S = 0.0;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 4 * RS_NT) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * RS_NT;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const double part = (exp(((double)v[u].x - m) * inv_t) + exp(((double)v[u].y - m) * inv_t)) +
                          (exp(((double)v[u].z - m) * inv_t) + exp(((double)v[u].w - m) * inv_t));
      S += part;
      const int blk = (i0 + u * RS_NT) >> 6;          // the same for the whole wave
      if (bsum && blk < nb) {
        const double t = wave_total_d(part);
        if (lane == 0) bsum[(size_t)row * nb + blk] = t;
      }
    }
  }
  S = block_sum_d<RS_NW>(S);
  if (mode != MV_ACCEPT_TYPICAL) {            // rejection sampling: max and normaliser only
    if (threadIdx.x == 0) {
      stats[(size_t)row * 3 + 0] = m;
      stats[(size_t)row * 3 + 1] = S;
      stats[(size_t)row * 3 + 2] = 0.0;
    }
    return;
  }
  const double c = 1e-5 * S;
  double Hs = 0.0;
  for (int i0 = threadIdx.x; i0 < V4; i0 += 4 * RS_NT) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * RS_NT;
      v[u] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float z[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double e = exp(((double)z[j] - m) * inv_t);
        Hs += e * log(e + c);
      }
    }
  }
  Hs = block_sum_d<RS_NW>(Hs);
  if (threadIdx.x == 0) {
    stats[(size_t)row * 3 + 0] = m;
    stats[(size_t)row * 3 + 1] = S;
    stats[(size_t)row * 3 + 2] = log(S) - Hs / S;
  }
}

// The same statistics for rows of at most NT·J·4 logits, held in registers:
// thread t reads float4 pieces t + j·NT (j < J) once, and keeps the tempered
// exponentials of the normaliser pass for the entropy pass, which then costs
// a division and a log per id, not a second read and a second exp.  The
// per-thread sums run over j in the same order as the loop above.
template <int NT, int J>
__global__ __launch_bounds__(NT) void row_stats_regs_kernel(const float* __restrict__ logits,
                                                            int V, int mode, double temperature,
                                                            int32_t* __restrict__ amax,
                                                            double* __restrict__ stats,
                                                            double* __restrict__ bsum) {
  constexpr int NW = NT / 64;
  const int row = blockIdx.x;
  const float4* z4 = reinterpret_cast<const float4*>(logits + (size_t)row * V);
  const int V4 = V >> 2;
  float4 v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + j * NT;
    v[j] = i < V4 ? z4[i] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  float bv = -INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int id = (threadIdx.x + j * NT) * 4;
    if (better_iv(v[j].x, id, bv, bi)) { bv = v[j].x; bi = id; }
    if (better_iv(v[j].y, id + 1, bv, bi)) { bv = v[j].y; bi = id + 1; }
    if (better_iv(v[j].z, id + 2, bv, bi)) { bv = v[j].z; bi = id + 2; }
    if (better_iv(v[j].w, id + 3, bv, bi)) { bv = v[j].w; bi = id + 3; }
  }
  block_argmax<NW>(bv, bi);
  if (threadIdx.x == 0) amax[row] = (unsigned)bi < (unsigned)V ? bi : 0;
  if (mode == MV_ACCEPT_GREEDY) return;

  const double inv_t = 1.0 / temperature;
  const double m = (double)bv;
  const int nb = (V + 255) >> 8;
  const int lane = threadIdx.x & 63;
  double e[J][4];
  double S = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    e[j][0] = exp(((double)v[j].x - m) * inv_t);
    e[j][1] = exp(((double)v[j].y - m) * inv_t);
    e[j][2] = exp(((double)v[j].z - m) * inv_t);
    e[j][3] = exp(((double)v[j].w - m) * inv_t);
    const double part = (e[j][0] + e[j][1]) + (e[j][2] + e[j][3]);
    S += part;
    const int blk = (threadIdx.x + j * NT) >> 6;        // the same for the whole wave
    if (bsum && blk < nb) {
      const double t = wave_total_d(part);
      if (lane == 0) bsum[(size_t)row * nb + blk] = t;
    }
  }
  S = block_sum_d<NW>(S);
  if (mode != MV_ACCEPT_TYPICAL) {
    if (threadIdx.x == 0) {
      stats[(size_t)row * 3 + 0] = m;
      stats[(size_t)row * 3 + 1] = S;
      stats[(size_t)row * 3 + 2] = 0.0;
    }
    return;
  }
  const double c = 1e-5 * S;
  double Hs = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) Hs += e[j][k] * log(e[j][k] + c);
  Hs = block_sum_d<NW>(Hs);
  if (threadIdx.x == 0) {
    stats[(size_t)row * 3 + 0] = m;
    stats[(size_t)row * 3 + 1] = S;
    stats[(size_t)row * 3 + 2] = log(S) - Hs / S;
  }
}

constexpr int RSR_NT = 1024, RSR_J = 8;

hipError_t launch_row_stats(const float* logits, int rows, int V, int mode, double temperature,
                            int32_t* argmax, double* stats, hipStream_t s, double* bsum) {
  if ((V >> 2) <= RSR_NT * RSR_J)
    hipLaunchKernelGGL((row_stats_regs_kernel<RSR_NT, RSR_J>), dim3(rows), dim3(RSR_NT), 0, s,
                       logits, V, mode, temperature, argmax, stats, bsum);
  else
    hipLaunchKernelGGL(row_stats_kernel, dim3(rows), dim3(RS_NT), 0, s, logits, V, mode,
                       temperature, argmax, stats, bsum);
  return hipGetLastError();
}

#define MV_MAXT 256

// Weighted inverse-CDF draw over ids 0..V-1 (V % 4 == 0) with weights >= 0:
// the smallest id whose cumulative weight (id order) exceeds u times the
// total; if rounding leaves none, the largest id of nonzero weight.  The
// whole workgroup (256 threads) calls it.  w4(i0, w) fills the weights of
// ids i0..i0+3.  Three passes, all reads coalesced: each wave sums 256-id
// blocks (a lane takes 4 consecutive ids) into LDS; an exclusive scan of the
// block sums finds the block where the cumulative weight crosses; one wave
// rescans that block.  Returns false (writing nothing) when the total is 0.
#define MV_DRAW_MAXB (MV_MAX_VOCAB / 256)   // 256-id blocks
// pre (optional): the 256-id block sums of the same weights, computed
// elsewhere (row_stats); fix(bsum) lets thread 0 adjust them (removed ids).
struct NoFix {
  __device__ void operator()(double*) const {}
};
template <class W4, class Fix = NoFix>
__device__ __forceinline__ bool block_draw(int V, double u, W4 w4, int32_t* out, double* margin,
                                           const double* pre = nullptr, Fix fix = Fix()) {
  __shared__ double bsum[MV_DRAW_MAXB], bpre[MV_DRAW_MAXB];   // block sums, exclusive prefixes
  __shared__ double wtot[4];
  __shared__ int s_blk, s_last;
  __shared__ double s_total;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = (V + 255) >> 8;
  // pass 1: block sums, lane partials in id order, then a fixed-order wave sum
  constexpr int UB = 8;               // blocks per wave in flight
  if (pre)
    for (int b = tid; b < nb; b += 256) bsum[b] = pre[b];
  for (int b0 = wave; !pre && b0 < nb; b0 += 4 * UB) {
    double part[UB];
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int b = b0 + 4 * j;
      const int i0 = (b << 8) + 4 * lane;
      double w[4] = {0.0, 0.0, 0.0, 0.0};
      if (b < nb && i0 < V) w4(i0, w);
      part[j] = (w[0] + w[1]) + (w[2] + w[3]);
    }
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      double v = part[j];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      v = __shfl(v, 0, 64);
      const int b = b0 + 4 * j;
      if (lane == 0 && b < nb) bsum[b] = v;
    }
  }
  __syncthreads();
  if (tid == 0) {
    fix(bsum);
    s_blk = 0x7fffffff;
    s_last = -1;
  }
  __syncthreads();
  // pass 2: exclusive scan of the block sums (each thread a run of them)
  const int per = (nb + 255) >> 8;
  const int r0 = min(nb, tid * per), r1 = min(nb, r0 + per);
  double run = 0.0;
  for (int b = r0; b < r1; ++b) run += bsum[b];
  double inc = run;                  // inclusive scan over the threads
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int k = 0; k < wave; ++k) base += wtot[k];
  if (tid == 0) s_total = ((wtot[0] + wtot[1]) + wtot[2]) + wtot[3];
  __syncthreads();
  const double S = s_total;
  if (!(S > 0.0)) {
    __syncthreads();
    return false;
  }
  double cum = base + inc - run;     // exclusive prefix of this thread's run
  bool hit = false;
  for (int b = r0; b < r1; ++b) {
    bpre[b] = cum;
    const double nxt = cum + bsum[b];
    if (!hit && nxt / S > u) {       // crossing: cumulative / S > u
      atomicMin(&s_blk, b);
      hit = true;
    }
    cum = nxt;
  }
  for (int b = r1 - 1; b >= r0; --b)
    if (bsum[b] > 0.0) {
      atomicMax(&s_last, b);
      break;
    }
  __syncthreads();
  // pass 3: one wave resolves the id inside the block
  if (wave == 0) {
    const int blk = s_blk;
    if (blk != 0x7fffffff) {
      const double before = bpre[blk];   // cumulative weight before the block
      const int i0 = (blk << 8) + 4 * lane;
      double w[4] = {0.0, 0.0, 0.0, 0.0};
      if (i0 < V) w4(i0, w);
      const double lsum = (w[0] + w[1]) + (w[2] + w[3]);
      double linc = lsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(linc, o, 64);
        if (lane >= o) linc += t;
      }
      double c = before + (linc - lsum);
      int found = -1;
      double mg = INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double prev = c;
        c += w[j];
        if (found < 0 && i0 < V && c / S > u) {
          found = i0 + j;
          mg = fmin(c / S - u, u - prev / S);
        }
      }
      const unsigned long long hit = __ballot(found >= 0);
      if (hit) {
        const int first = __ffsll((long long)hit) - 1;
        if (lane == first) {
          *out = found;
          if (margin) *margin = mg;
        }
      } else if (lane == 0) {        // rounding between the two scans: the block's last nonzero id
        int last = -1;
        for (int i = min(V, (blk + 1) << 8) - 1; i >= (blk << 8) && last < 0; i -= 4) {
          double ww[4];
          w4(i - 3, ww);
#pragma unroll
          for (int j = 3; j >= 0; --j)
            if (last < 0 && ww[j] > 0.0) last = i - 3 + j;
        }
        *out = last >= 0 ? last : (blk << 8);
        if (margin) *margin = 0.0;
      }
    } else if (lane == 0) {          // no crossing: the largest id of nonzero weight
      const int lb = s_last;
      int last = 0;
      if (lb >= 0) {
        for (int i = min(V, (lb + 1) << 8) - 1; i >= (lb << 8); i -= 4) {
          double ww[4];
          w4(i - 3, ww);
          int hitj = -1;
#pragma unroll
          for (int j = 3; j >= 0; --j)
            if (hitj < 0 && ww[j] > 0.0) hitj = j;
          if (hitj >= 0) {
            last = i - 3 + hitj;
            break;
          }
        }
      }
      *out = last;
      if (margin) *margin = 0.0;
    }
  }
  __syncthreads();
  return true;
}

// Inverse-CDF sample of softmax(z * inv_t): block_draw over the unnormalised
// weights exp((z_i - max) * inv_t).  Writes *out (and |cdf - u| to *margin).
__device__ __forceinline__ void block_sample(const float* __restrict__ z, int V, int amax_id, double inv_t,
                             double u, int32_t* out, double* margin, const double* pre = nullptr) {
  const double m = (double)z[amax_id];
  auto w4 = [&](int i0, double (&w)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(z + i0);
    w[0] = exp(((double)v.x - m) * inv_t);
    w[1] = exp(((double)v.y - m) * inv_t);
    w[2] = exp(((double)v.z - m) * inv_t);
    w[3] = exp(((double)v.w - m) * inv_t);
  };
  // no mass in the given block sums: recompute them; none at all (cannot
  // happen for finite logits): the argmax
  if (!block_draw(V, u, w4, out, margin, pre) && !(pre && block_draw(V, u, w4, out, margin)) &&
      threadIdx.x == 0) {
    *out = amax_id;
    if (margin) *margin = 0.0;
  }
  __syncthreads();
}

// The step's capacity check: thread 0 reads the prefix length before this
// kernel moves it on (the same thread's later update is ordered after it).
__device__ __forceinline__ void step_guard(const StepGuard& g, const int32_t* n, int b) {
  if (g.status && n && threadIdx.x == 0) {
    const int n0 = n[b];
    if (n0 < 0 || n0 > g.cap - g.T) atomicOr(g.status, MV_STATUS_CAPACITY);
  }
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
    int d, int32_t* __restrict__ n_advance, const double* __restrict__ bsum, StepGuard guard) {
  __shared__ unsigned char pass[MV_MAXT], ok[MV_MAXT];
  __shared__ double lq[MV_MAXT], score[MV_MAXT];
  __shared__ int par[MV_MAXT], dep[MV_MAXT], tk[MV_MAXT];   // the tree, staged for the walk
  __shared__ int amax[MV_MAXT];                              // argmax of each of the T rows
  __shared__ int s_best;
  const int b = blockIdx.x;
  const NormGains ng = norm_gains(x && h_last ? final_norm : nullptr, d);
  step_guard(guard, n_advance, b);
  for (int v = threadIdx.x; v < T; v += 256) {
    par[v] = parent[(size_t)b * T + v];
    dep[v] = depth_of[(size_t)b * T + v];
    tk[v] = tok[(size_t)b * T + v];
    if (amax_key) {         // the LM head's atomic argmax keys; cleared for the next step
      const size_t r = (size_t)b * T + v;
      const int col = argmax_key_col(amax_key[r]);
      amax[v] = (unsigned)col < (unsigned)V ? col : 0;   // NaN rows: no maximum, id 0
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
    } else if ((unsigned)tk[v] >= (unsigned)V) {   // not a token: never accepted
      pass[v] = 0;
      lq[v] = -INFINITY;
      if (margin) margin[(size_t)b * (T + 1) + v] = -INFINITY;
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
               margin ? margin + (size_t)b * (T + 1) + T : nullptr,
               bsum ? bsum + (size_t)brow * ((V + 255) >> 8) : nullptr);
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
                                hipStream_t s, int32_t* n_advance, const double* bsum,
                                StepGuard guard) {
  hipLaunchKernelGGL(accept_finish_kernel, dim3(B), dim3(256), 0, s, logits, argmax, amax_key,
                     stats,
                     parent, depth_of, tok, T, V, depth, mode, root_mode, temperature, eps, delta,
                     u, u_index, u_stride, accept_len, path, best, next_root, emitted, margin, x,
                     final_norm, h_last, d, n_advance, bsum, guard);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Rejection-sampling acceptance (speculative sampling: the lecture note's
// section 二.3 and the speculative-decoding tutorial's Maths section).  A
// draft token x drawn from q is kept against the target p with probability
// min(1, p(x)/q(x)); a rejected one is replaced by a draw from the positive
// part of p - q, normalised.  Over a tree: at the current node (target p =
// softmax(logits/temperature) of its row) the children are tried in node
// order against the running residual r (p at first); a kept child becomes
// the current node; a rejection turns r into the correction's residual and
// the next sibling is tried; when none is kept (or at a leaf) the next root
// is drawn from r by inverse CDF.  Drafts: without draft logits a candidate
// is a point mass (top-s candidates are fixed), so x is kept with
// probability r(x) and a rejection removes x from r; with draft logits
// [B][depth][V] the children at depth k use q = softmax(draft[k-1] / temp).
// A residual with no mass left (rejection of probability 0 up to rounding)
// falls back to the node's p.  Draws: u[c] decides child c (kept iff
// u[c] < a), u[0] makes the final draw.
//
// The walk is sequential (one decision at a time) but every thread runs it
// in lockstep on the same shared values; the V-wide passes (draft row
// statistics, residual updates, the final draw) use the whole workgroup.

// A residual value written by another wave of this workgroup: read at
// device scope, past the compute unit's vector cache.
__device__ __forceinline__ double ld_resid(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void reject_accept_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ amax_rows,
    const double* __restrict__ stats, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ tok, int T, int V, int depth, double inv_t,
    const float* __restrict__ draft, const double* __restrict__ dstats,
    const double* __restrict__ u, const int32_t* __restrict__ u_index, long long u_stride,
    double* resid, int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
    int32_t* __restrict__ best_out, int32_t* __restrict__ next_root,
    int32_t* __restrict__ emitted, double* __restrict__ margin, const float* __restrict__ x,
    const u16* __restrict__ final_norm, u16* __restrict__ h_last, int d,
    int32_t* __restrict__ n_advance, const double* __restrict__ bsum, StepGuard guard) {
  // the tree and every per-candidate quantity the walk needs, in LDS
  __shared__ int par[MV_MAXT], tk[MV_MAXT];
  __shared__ int fch[MV_MAXT], nsib[MV_MAXT];   // first child, next sibling (T: none)
  __shared__ int dupp[MV_MAXT];                 // nearest earlier sibling with the same token
  __shared__ double mrow[MV_MAXT], srow[MV_MAXT];   // row max and normaliser
  __shared__ double esel[MV_MAXT];   // exp((z_parent[tok] - max) / temp) of each candidate
  __shared__ double qsel[MV_MAXT];   // draft probability of each candidate
  __shared__ double usel[MV_MAXT];   // the step's draws
  __shared__ int xs[MV_MAXT];        // tokens removed from the final residual
  __shared__ int s_nx;
  __shared__ int s_nodes[MV_MAX_DEPTH + 1];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const NormGains ng = norm_gains(x && h_last ? final_norm : nullptr, d);
  step_guard(guard, n_advance, b);
  const size_t row0 = (size_t)b * T;
  const double* ub = u + (size_t)(u_index ? u_index[0] : 0) * u_stride + row0;
  for (int v = tid; v < T; v += 256) {
    const int pv = parent[row0 + v];
    usel[v] = ub[v];
    par[v] = v > 0 && pv >= 0 && pv < v ? pv : -1;   // other parents: not in the tree
    tk[v] = tok[row0 + v];
    fch[v] = T;
    const size_t row = row0 + v;
    mrow[v] = (double)logits[row * V + amax_rows[row]];
    srow[v] = stats[row * 3 + 1];
  }
  if (margin)
    for (int v = tid; v <= T; v += 256) margin[row0 + b + v] = INFINITY;
  __syncthreads();
  for (int v = tid; v < T; v += 256) {
    const int pv = par[v];
    int ns = T, dp = -1;
    double e = 0.0, q = 0.0;
    if (pv >= 0) {
      atomicMin(&fch[pv], v);
      for (int c = v + 1; c < T && ns == T; ++c)
        if (par[c] == pv) ns = c;
      for (int c = v - 1; c > pv && dp < 0; --c)
        if (par[c] == pv && tk[c] == tk[v]) dp = c;
      const int xt = tk[v];
      if ((unsigned)xt < (unsigned)V) {       // other ids are never kept
        e = exp(((double)logits[(row0 + pv) * V + xt] - mrow[pv]) * inv_t);
        if (draft) {
          int k = 0;                           // depth of v
          for (int a = v; a > 0 && k <= MV_MAX_DEPTH; a = par[a]) ++k;
          if (k >= 1 && k <= depth) {
            const size_t dr = (size_t)b * depth + (k - 1);
            q = exp(((double)draft[dr * V + xt] - dstats[dr * 3]) * inv_t) / dstats[dr * 3 + 1];
          }
        }
      }
    }
    nsib[v] = ns;
    dupp[v] = dp;
    esel[v] = e;
    qsel[v] = q;
  }
  __syncthreads();
  double* R = draft ? resid + (size_t)b * 2 * V : nullptr;   // two residual buffers [2][V]
  const int max_len = min(depth, MV_MAX_DEPTH);
  if (tid == 0) s_nodes[0] = 0;
  int cur = 0, L = 0;
  for (;;) {
    const float* z = logits + (row0 + cur) * V;
    const double m = mrow[cur], S = srow[cur];
    auto e_of4 = [&](int i0, double (&w)[4]) {
      const float4 v = *reinterpret_cast<const float4*>(z + i0);
      w[0] = exp(((double)v.x - m) * inv_t);
      w[1] = exp(((double)v.y - m) * inv_t);
      w[2] = exp(((double)v.z - m) * inv_t);
      w[3] = exp(((double)v.w - m) * inv_t);
    };
    const int first = L < max_len ? fch[cur] : T;
    const float* zd = draft && first < T ? draft + ((size_t)b * depth + L) * V : nullptr;
    const double md = zd ? dstats[((size_t)b * depth + L) * 3] : 0.0;
    const double Sd = zd ? dstats[((size_t)b * depth + L) * 3 + 1] : 1.0;
    int rb = -1;              // draft: residual buffer in use (-1: r is p)
    double rs = 1.0;          // its total
    double ex_e = 0.0;        // point drafts: removed mass (units of S) ...
    int ex_from = cur + 1;    // ... of the rejected siblings from this node index on
    int acc = -1;
    for (int c = first; c < T; c = nsib[c]) {
      const bool valid = (unsigned)tk[c] < (unsigned)V;
      double a = 0.0;
      const bool seen = !valid || dupp[c] >= ex_from;
      if (!draft) {
        if (!seen) a = fmin(1.0, esel[c] / (S - ex_e));
      } else if (valid) {
        const double qx = qsel[c];
        const double rx = rb >= 0 ? ld_resid(R + (size_t)rb * V + tk[c]) / rs : esel[c] / S;
        a = qx > 0.0 ? fmin(1.0, rx / qx) : (rx > 0.0 ? 1.0 : 0.0);
      }
      const double uc = usel[c];
      if (margin && tid == 0) margin[row0 + b + c] = uc - a;
      if (uc < a) {
        acc = c;
        break;
      }
      if (!draft) {
        if (!seen) {
          if (S - ex_e - esel[c] > 0.0) {
            ex_e += esel[c];
          } else {            // nothing left: back to p
            ex_e = 0.0;
            ex_from = c + 1;
          }
        }
      } else {
        // r <- max(0, r - q) into the other buffer; each thread rewrites the
        // ids it wrote last time, so only the scalar reads above and the
        // final draw cross waves
        const int nb = rb == 0 ? 1 : 0;
        double part = 0.0;
        for (int i = tid; i < V; i += 256) {
          const double ri = rb >= 0 ? R[(size_t)rb * V + i] / rs : exp(((double)z[i] - m) * inv_t) / S;
          const double qi = exp(((double)zd[i] - md) * inv_t) / Sd;
          const double ni = fmax(ri - qi, 0.0);
          R[(size_t)nb * V + i] = ni;
          part += ni;
        }
        __threadfence();
        const double sum = block_sum_d(part);
        if (sum > 0.0) {
          rb = nb;
          rs = sum;
        } else {
          rb = -1;
          rs = 1.0;
        }
      }
    }
    if (acc >= 0) {
      cur = acc;
      ++L;
      if (tid == 0) s_nodes[L] = cur;
      // draft residuals: the next node's first rejection rewrites buffer 0,
      // which a slower wave may still be reading for the decision just taken
      // (every wave takes the same branch, so the barrier is uniform)
      if (draft) __syncthreads();
      continue;
    }
    // final draw from the residual at cur (the row's block sums, when
    // given, replace the first pass over the row)
    const double* pre = bsum ? bsum + (row0 + cur) * ((V + 255) >> 8) : nullptr;
    const double u0 = usel[0];
    double* mg = margin ? margin + row0 + b + T : nullptr;
    int32_t* out = next_root + b;
    if (!draft) {
      if (tid == 0) {
        int n = 0;
        for (int c = first; c < T; c = nsib[c])
          if (c >= ex_from && (unsigned)tk[c] < (unsigned)V && dupp[c] < ex_from) xs[n++] = tk[c];
        s_nx = n;
      }
      __syncthreads();
      const int nx = s_nx;
      auto w_res = [&](int i0, double (&w)[4]) {
        e_of4(i0, w);
        for (int j = 0; j < nx; ++j) {
          const int k = xs[j] - i0;
          if (k == 0) w[0] = 0.0;
          if (k == 1) w[1] = 0.0;
          if (k == 2) w[2] = 0.0;
          if (k == 3) w[3] = 0.0;
        }
      };
      auto fix = [&](double* bs) {            // take the removed ids out of their blocks
        for (int j = 0; j < nx; ++j) {
          const int k = xs[j];
          bs[k >> 8] = fmax(bs[k >> 8] - exp(((double)z[k] - m) * inv_t), 0.0);
        }
      };
      if (!(pre ? block_draw(V, u0, w_res, out, mg, pre, fix) : block_draw(V, u0, w_res, out, mg)))
        block_sample(z, V, amax_rows[row0 + cur], inv_t, u0, out, mg, pre);
    } else if (rb >= 0) {
      const double* Rb = R + (size_t)rb * V;
      auto w_r = [&](int i0, double (&w)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = ld_resid(Rb + i0 + j);
      };
      block_draw(V, u0, w_r, out, mg);
    } else {
      block_sample(z, V, amax_rows[row0 + cur], inv_t, u0, out, mg, pre);
    }
    break;
  }
  if (tid == 0) {
    accept_len[b] = L;
    best_out[b] = cur;
    if (n_advance) n_advance[b] += L + 1;
    for (int k = 0; k <= depth; ++k) {
      const int node = k <= L ? s_nodes[k] : -1;
      path[(size_t)b * (depth + 1) + k] = node;
      if (emitted) emitted[(size_t)b * (depth + 1) + k] = node >= 0 ? tk[node] : -1;
    }
  }
  if (x && h_last)
    block_norm_row(x + (row0 + cur) * d, final_norm, ng, h_last + (size_t)b * d, d);
}

hipError_t launch_reject_accept(const float* logits, const int32_t* argmax, const double* stats,
                                const int32_t* parent, const int32_t* tok, int B, int T, int V,
                                int depth, double temperature, const float* draft,
                                const double* dstats, const double* u, const int32_t* u_index,
                                long long u_stride, double* resid, int32_t* accept_len,
                                int32_t* path, int32_t* best, int32_t* next_root,
                                int32_t* emitted, double* margin, const float* x,
                                const u16* final_norm, u16* h_last, int d, hipStream_t s,
                                int32_t* n_advance, const double* bsum, StepGuard guard) {
  if (T > MV_MAXT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reject_accept_kernel, dim3(B), dim3(256), 0, s, logits, argmax, stats, parent,
                     tok, T, V, depth, 1.0 / temperature, draft, dstats, u, u_index, u_stride, resid,
                     accept_len, path, best, next_root, emitted, margin, x, final_norm, h_last, d,
                     n_advance, bsum, guard);
  return hipGetLastError();
}

// Prefill: after a chain chunk, sequence b's last real row (cnt[b] - 1)
// supplies h_last (its final RMSNorm) and the first root; n[b] += cnt[b].
// cnt[b] == 0: nothing.
__global__ __launch_bounds__(256) void prefill_select_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ amax, const int32_t* __restrict__ cnt,
    int T, int V, int root_mode, double temperature, const double* __restrict__ u, int u_bstride,
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
    block_sample(logits + (size_t)row * V, V, amax[row], 1.0 / temperature,
                 u[(size_t)b * u_bstride], root + b, nullptr);
  }
  __syncthreads();
  if (threadIdx.x == 0) n_prefix[b] += c;
}

hipError_t launch_prefill_select(const float* logits, const int32_t* amax, const int32_t* cnt,
                                 int B, int T, int V, int root_mode, double temperature,
                                 const double* u, int u_bstride, int32_t* root, int32_t* n_prefix,
                                 const float* x, const u16* final_norm, u16* h_last, int d,
                                 hipStream_t s) {
  hipLaunchKernelGGL(prefill_select_kernel, dim3(B), dim3(256), 0, s, logits, amax, cnt, T, V,
                     root_mode, temperature, u, u_bstride, root, n_prefix, x, final_norm, h_last, d);
  return hipGetLastError();
}

}  // namespace mvk
