// Medusa heads: u_k = h + SiLU(W1_k h), z_k = W2_k u_k, then each head's
// top-s candidates fill the tree (node of depth k and rank i gets head k's
// i-th candidate; the root gets the root token).
//
// At batch size B the heads are matrix-vector products over bf16 weights
// that are read exactly once, so they are HBM-bound GEMVs: each wave owns
// whole weight rows, its 64 lanes read 16 contiguous bytes each (a 1 KiB
// coalesced piece of a row per instruction; eight pieces of each of two rows
// in flight), multiply by the fp32 input held in LDS and reduce across the
// wave.
#include "common.hpp"

namespace mvk {

constexpr int GEMV_RW = 2;            // rows per wave per iteration
constexpr int GEMV_ROWS_PER_WG = 64;  // 16 rows per wave
constexpr int GEMV_CH = 8;            // 1 KiB row pieces per lane in flight

// mode 0: y = W1 x -> u[b][k][j] = h[b][j] + SiLU(y) (x = h, bf16 input)
// mode 1: y = W2 x -> z[b][k][j] = y             (x = u[b][k], fp32 input)
template <int MAXB>
__global__ __launch_bounds__(256) void heads_gemv_kernel(const u16* __restrict__ hb,
                                                         const float* __restrict__ uf,
                                                         const u16* __restrict__ W,
                                                         float* __restrict__ out, int B, int D,
                                                         int d, int rows, int mode, int rpw) {
  extern __shared__ float xs[];                   // [B][d]
  const int k = blockIdx.y;                       // head index 0..D-1 (head k+1)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u16* Wk = W + (size_t)k * rows * d;
  const int r_lo = blockIdx.x * rpw;
  const int r_hi = min(rows, r_lo + rpw);
  // GEMV_CH 1 KiB pieces of each of the wave's GEMV_RW rows per block
  uint4 w[GEMV_CH][GEMV_RW];
  auto load = [&](int r0, int c0) {
#pragma unroll
    for (int j = 0; j < GEMV_CH; ++j) {
      const int c = min(c0 + j * 512 + lane * 8, d - 8);      // clamped: in bounds
#pragma unroll
      for (int i = 0; i < GEMV_RW; ++i) {
        const int r = min(r0 + i, r_hi - 1);
        w[j][i] = *reinterpret_cast<const uint4*>(Wk + (size_t)r * d + c);
      }
    }
  };
  // the wave's first block of weights is requested before the input rows
  // are staged, and every later block right after the previous one's math,
  // so that 2 * GEMV_CH loads per lane stay in flight across the reductions
  int r0 = r_lo + wave * GEMV_RW;
  if (r0 < r_hi) load(r0, 0);
  for (int i = threadIdx.x; i < B * d; i += 256) {
    const int b = i / d, c = i % d;
    xs[i] = mode == 0 ? bf16_to_f32(hb[(size_t)b * d + c]) : uf[((size_t)b * D + k) * d + c];
  }
  __syncthreads();
  for (; r0 < r_hi; r0 += 4 * GEMV_RW) {
    float acc[GEMV_RW][MAXB];
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i)
#pragma unroll
      for (int b = 0; b < MAXB; ++b) acc[i][b] = 0.f;
    for (int c0 = 0; c0 < d; c0 += 512 * GEMV_CH) {
#pragma unroll
      for (int j = 0; j < GEMV_CH; ++j) {
        const int c = c0 + j * 512 + lane * 8;
        if (c >= d) break;
#pragma unroll
        for (int b = 0; b < MAXB; ++b) {
          if (b >= B) break;
          const float4 x0 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c);
          const float4 x1 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c + 4);
#pragma unroll
          for (int i = 0; i < GEMV_RW; ++i) {
            float a = acc[i][b];
            a += bf16lo(w[j][i].x) * x0.x + bf16hi(w[j][i].x) * x0.y;
            a += bf16lo(w[j][i].y) * x0.z + bf16hi(w[j][i].y) * x0.w;
            a += bf16lo(w[j][i].z) * x1.x + bf16hi(w[j][i].z) * x1.y;
            a += bf16lo(w[j][i].w) * x1.z + bf16hi(w[j][i].w) * x1.w;
            acc[i][b] = a;
          }
        }
      }
      int nr = r0, nc = c0 + 512 * GEMV_CH;
      if (nc >= d) {
        nr = r0 + 4 * GEMV_RW;
        nc = 0;
      }
      if (nr < r_hi) load(nr, nc);
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

// rpw rows per workgroup (a multiple of 4 waves x GEMV_RW): fewer rows per
// workgroup when the matrix is short, so that the grid still covers the CUs.
static hipError_t launch_gemv(const u16* hb, const float* uf, const u16* W, float* out, int B,
                              int D, int d, int rows, int mode, hipStream_t s) {
  int rpw = GEMV_ROWS_PER_WG;
  while (rpw > 4 * GEMV_RW && (size_t)((rows + rpw - 1) / rpw) * D < 1024) rpw /= 2;
  dim3 grid((rows + rpw - 1) / rpw, D);
  // the fp32 input rows live in LDS: up to 4 x 8192 x 4 B = 128 KiB (gfx950
  // has 160 KiB per workgroup; above 64 KiB the launch must opt in)
  const size_t lds = (size_t)B * d * sizeof(float);
  if (lds > MV_HEADS_LDS_MAX) return hipErrorInvalidValue;
  if (lds > 65536) {
    const hipError_t e = B == 1
        ? hipFuncSetAttribute(reinterpret_cast<const void*>(&heads_gemv_kernel<1>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)MV_HEADS_LDS_MAX)
        : hipFuncSetAttribute(reinterpret_cast<const void*>(&heads_gemv_kernel<4>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)MV_HEADS_LDS_MAX);
    if (e != hipSuccess) return e;
  }
  if (B == 1)
    hipLaunchKernelGGL((heads_gemv_kernel<1>), grid, dim3(256), lds, s, hb, uf, W, out, B, D, d, rows, mode, rpw);
  else if (B <= 4)
    hipLaunchKernelGGL((heads_gemv_kernel<4>), grid, dim3(256), lds, s, hb, uf, W, out, B, D, d, rows, mode, rpw);
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
// Top-s of rows of V logits: larger value first, lower id first on ties.
// Stage 1: each wave takes 1024 consecutive logits (16 per lane, coalesced
// float4 loads) and selects its top s by s rounds of a wave-wide argmax over
// the lanes' best remaining values (shuffles only, no barriers); it writes
// s (value, id) candidates.  Stage 2: one wave per row selects the final s
// from the row's candidates the same way.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better_vi(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Best (value, id) of the wave in every lane: DPP lane moves inside each
// 16-lane row (quad swaps, half-row and row mirrors), then two cross-row
// shuffles.
template <int CTRL>
__device__ __forceinline__ void dpp_best(float& wv, int& wi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(wv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(wi, CTRL, 0xF, 0xF, false);
  if (better_vi(ov, oi, wv, wi)) {
    wv = ov;
    wi = oi;
  }
}
__device__ __forceinline__ void wave_best(float& wv, int& wi) {
  dpp_best<0xB1>(wv, wi);     // quad_perm [1,0,3,2]
  dpp_best<0x4E>(wv, wi);     // quad_perm [2,3,0,1]
  dpp_best<0x141>(wv, wi);    // row_half_mirror
  dpp_best<0x140>(wv, wi);    // row_mirror
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float ov = __shfl_xor(wv, o, 64);
    const int oi = __shfl_xor(wi, o, 64);
    if (better_vi(ov, oi, wv, wi)) {
      wv = ov;
      wi = oi;
    }
  }
}

// v/id: this lane's N (<= 32) candidates (id INT_MAX = empty).  Writes the
// wave's top s into outv/outi (lane r writes round r's winner).
template <int N>
__device__ __forceinline__ void wave_select(const float (&v)[N], const int (&id)[N], int s,
                                            float* outv, int* outi) {
  static_assert(N <= 32, "the taken mask holds 32 candidates");
  const int lane = threadIdx.x & 63;
  unsigned taken = 0;
  for (int r = 0; r < s; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff, bj = -1;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (!((taken >> j) & 1u) && better_vi(v[j], id[j], bv, bi)) {
        bv = v[j];
        bi = id[j];
        bj = j;
      }
    }
    float wv = bv;
    int wi = bi;
    wave_best(wv, wi);
    if (bj >= 0 && bi == wi) taken |= 1u << bj;     // ids are unique: one owner
    if (lane == r) {
      outv[0] = wv;
      outi[0] = wi;
    }
  }
}

__global__ __launch_bounds__(256) void topk_partial_kernel(const float* __restrict__ z, int V,
                                                           int s_top, float* __restrict__ cv,
                                                           int* __restrict__ ci) {
  const int row = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;                       // waves per row
  const int w = blockIdx.x * 4 + wave;
  const int base = w * 1024;
  const float* zr = z + (size_t)row * V;
  float v[16];
  int id[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = base + j * 256 + lane * 4;
    float4 x = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (i < V) x = *reinterpret_cast<const float4*>(zr + i);
    v[4 * j + 0] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) id[4 * j + e] = i + e < V ? i + e : 0x7fffffff;
  }
  float ov = 0.f;
  int oi = 0;
  wave_select(v, id, s_top, &ov, &oi);
  if (lane < s_top) {
    const size_t o = ((size_t)row * nw + w) * s_top + lane;
    cv[o] = ov;
    ci[o] = oi;
  }
}

// One wave per row: up to 1024 candidates (16 per lane).
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ cv,
                                                        const int* __restrict__ ci, int ncand,
                                                        int s_top, int32_t* __restrict__ ids,
                                                        float* __restrict__ vals) {
  const int row = blockIdx.x, lane = threadIdx.x;
  float v[16];
  int id[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int c = j * 64 + lane;
    v[j] = c < ncand ? cv[(size_t)row * ncand + c] : -INFINITY;
    id[j] = c < ncand ? ci[(size_t)row * ncand + c] : 0x7fffffff;
  }
  float ov = 0.f;
  int oi = 0;
  wave_select(v, id, s_top, &ov, &oi);
  if (lane < s_top) {
    ids[(size_t)row * s_top + lane] = oi;
    vals[(size_t)row * s_top + lane] = ov;
  }
}

int topk_waves(int V) { return ((V + 4095) / 4096) * 4; }

hipError_t launch_topk(const float* z, int rows, int V, int s_top, int32_t* ids, float* vals,
                       float* cand_v, int* cand_i, hipStream_t s) {
  if (s_top > 16 || s_top > 64) return hipErrorInvalidValue;
  const int nw = topk_waves(V);
  if (nw * s_top > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_partial_kernel, dim3(nw / 4, rows), dim3(256), 0, s, z, V, s_top, cand_v,
                     cand_i);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(rows), dim3(64), 0, s, cand_v, cand_i, nw * s_top,
                     s_top, ids, vals);
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
