// Medusa heads: u_k = h + SiLU(W1_k h), z_k = W2_k u_k, then each head's
// top-s candidates fill the tree (node of depth k and rank i gets head k's
// i-th candidate; the root gets the root token).
//
// At batch size B the heads are matrix-vector products over bf16 weights
// that are read exactly once, so they are HBM-bound GEMVs: each wave owns
// whole weight rows, its 64 lanes read 16 contiguous bytes each (a 1 KiB
// coalesced piece of a row per instruction), multiply by the fp32 input held
// in LDS and reduce across the wave.
#include "common.hpp"

namespace mvk {

constexpr int GEMV_RW = 2;            // rows per wave per iteration
constexpr int GEMV_ROWS_PER_WG = 64;  // 16 rows per wave

// mode 0: y = W1 x -> u[b][k][j] = h[b][j] + SiLU(y) (x = h, bf16 input)
// mode 1: y = W2 x -> z[b][k][j] = y             (x = u[b][k], fp32 input)
template <int MAXB>
__global__ __launch_bounds__(256) void heads_gemv_kernel(const u16* __restrict__ hb,
                                                         const float* __restrict__ uf,
                                                         const u16* __restrict__ W,
                                                         float* __restrict__ out, int B, int D,
                                                         int d, int rows, int mode) {
  extern __shared__ float xs[];                   // [B][d]
  const int k = blockIdx.y;                       // head index 0..D-1 (head k+1)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < B * d; i += 256) {
    const int b = i / d, c = i % d;
    xs[i] = mode == 0 ? bf16_to_f32(hb[(size_t)b * d + c]) : uf[((size_t)b * D + k) * d + c];
  }
  __syncthreads();
  const u16* Wk = W + (size_t)k * rows * d;
  const int r_lo = blockIdx.x * GEMV_ROWS_PER_WG;
  const int r_hi = min(rows, r_lo + GEMV_ROWS_PER_WG);
  for (int r0 = r_lo + wave * GEMV_RW; r0 < r_hi; r0 += 4 * GEMV_RW) {
    float acc[GEMV_RW][MAXB];
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i)
#pragma unroll
      for (int b = 0; b < MAXB; ++b) acc[i][b] = 0.f;
    for (int c = lane * 8; c < d; c += 512) {
      uint4 w[GEMV_RW];
#pragma unroll
      for (int i = 0; i < GEMV_RW; ++i) {
        const int r = min(r0 + i, r_hi - 1);
        w[i] = *reinterpret_cast<const uint4*>(Wk + (size_t)r * d + c);
      }
#pragma unroll
      for (int b = 0; b < MAXB; ++b) {
        if (b >= B) break;
        const float4 x0 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c);
        const float4 x1 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c + 4);
#pragma unroll
        for (int i = 0; i < GEMV_RW; ++i) {
          float a = acc[i][b];
          a += bf16lo(w[i].x) * x0.x + bf16hi(w[i].x) * x0.y;
          a += bf16lo(w[i].y) * x0.z + bf16hi(w[i].y) * x0.w;
          a += bf16lo(w[i].z) * x1.x + bf16hi(w[i].z) * x1.y;
          a += bf16lo(w[i].w) * x1.z + bf16hi(w[i].w) * x1.w;
          acc[i][b] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i) {
      const int r = r0 + i;
#pragma unroll
      for (int b = 0; b < MAXB; ++b) {
        if (b >= B) break;
        const float y = warp_sum(acc[i][b]);
        if (lane == 0 && r < r_hi) {
          const size_t o = ((size_t)b * D + k) * rows + r;
          out[o] = mode == 0 ? xs[(size_t)b * d + r] + silu_f(y) : y;
        }
      }
    }
  }
}

static hipError_t launch_gemv(const u16* hb, const float* uf, const u16* W, float* out, int B,
                              int D, int d, int rows, int mode, hipStream_t s) {
  dim3 grid((rows + GEMV_ROWS_PER_WG - 1) / GEMV_ROWS_PER_WG, D);
  const size_t lds = (size_t)B * d * sizeof(float);
  if (B == 1)
    hipLaunchKernelGGL((heads_gemv_kernel<1>), grid, dim3(256), lds, s, hb, uf, W, out, B, D, d, rows, mode);
  else if (B <= 4)
    hipLaunchKernelGGL((heads_gemv_kernel<4>), grid, dim3(256), lds, s, hb, uf, W, out, B, D, d, rows, mode);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_heads_w1(const u16* h, const u16* w1, float* u, int B, int D, int d,
                           hipStream_t s) {
  return launch_gemv(h, nullptr, w1, u, B, D, d, d, 0, s);
}

hipError_t launch_heads_w2(const float* u, const u16* w2, float* z, int B, int D, int d, int V,
                           hipStream_t s) {
  return launch_gemv(nullptr, u, w2, z, B, D, d, V, 1, s);
}

// ---------------------------------------------------------------------------
// Top-s of one row of V logits: larger value first, lower id first on ties.
// Each of the 256 threads keeps a sorted list of its best MAXS candidates
// (fixed-size insertion, stays in registers); then s rounds of a block-wide
// selection of the best list head.
// ---------------------------------------------------------------------------
template <int MAXS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ z, int V, int s_top,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ vals) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int swin;
  const int row = blockIdx.x;
  const float* zr = z + (size_t)row * V;
  float lv[MAXS];
  int li[MAXS];
#pragma unroll
  for (int j = 0; j < MAXS; ++j) {
    lv[j] = -INFINITY;
    li[j] = 0x7fffffff;
  }
  for (int i = threadIdx.x; i < V; i += 256) {
    float cv = zr[i];
    int ci = i;
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
      const bool better = cv > lv[j] || (cv == lv[j] && ci < li[j]);
      const float tv = better ? lv[j] : cv;
      const int ti = better ? li[j] : ci;
      lv[j] = better ? cv : lv[j];
      li[j] = better ? ci : li[j];
      cv = tv;
      ci = ti;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = 0; r < s_top; ++r) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      sv[wave] = bv;
      si[wave] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float wv = sv[0];
      int wi = si[0];
      for (int w = 1; w < 4; ++w)
        if (sv[w] > wv || (sv[w] == wv && si[w] < wi)) {
          wv = sv[w];
          wi = si[w];
        }
      ids[(size_t)row * s_top + r] = wi;
      vals[(size_t)row * s_top + r] = wv;
      swin = wi;
    }
    __syncthreads();
    if (li[0] == swin) {            // the owner pops its head
#pragma unroll
      for (int j = 0; j < MAXS - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[MAXS - 1] = -INFINITY;
      li[MAXS - 1] = 0x7fffffff;
    }
    __syncthreads();
  }
}

hipError_t launch_topk(const float* z, int rows, int V, int s_top, int32_t* ids, float* vals,
                       hipStream_t s) {
  if (s_top <= 16)
    hipLaunchKernelGGL((topk_kernel<16>), dim3(rows), dim3(256), 0, s, z, V, s_top, ids, vals);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// tok[b][v] = root[b] for v = 0, else top_ids[b][depth(v)-1][rank(v)].
__global__ void tree_fill_kernel(const int32_t* __restrict__ top_ids,
                                 const int32_t* __restrict__ root,
                                 const int32_t* __restrict__ depth_of,
                                 const int32_t* __restrict__ rank, int32_t* __restrict__ tok,
                                 int B, int T, int D, int s_top) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= B * T) return;
  const int b = e / T, v = e % T;
  const int dep = min(depth_of[e], D);
  const int rk = min(max(rank[e], 0), s_top - 1);
  tok[e] = (v == 0 || dep <= 0) ? root[b] : top_ids[((size_t)b * D + (dep - 1)) * s_top + rk];
}

hipError_t launch_tree_fill(const int32_t* top_ids, const int32_t* root, const int32_t* depth_of,
                            const int32_t* rank, int32_t* tok, int B, int T, int D, int s_top,
                            hipStream_t s) {
  hipLaunchKernelGGL(tree_fill_kernel, dim3((B * T + 255) / 256), dim3(256), 0, s, top_ids, root,
                     depth_of, rank, tok, B, T, D, s_top);
  return hipGetLastError();
}

}  // namespace mvk
