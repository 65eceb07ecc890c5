// Medusa heads: u_k = h + SiLU(W1_k h), z_k = W2_k u_k, then each head's
// top-s candidates fill the tree (node of depth k and rank i gets head k's
// i-th candidate; the root gets the root token).
//
// At batch size B the heads are matrix-vector products over bf16 weights
// that are read exactly once, so they are HBM-bound GEMVs: each wave owns
// whole weight rows, its 64 lanes read 16 contiguous bytes each (a 1 KiB
// coalesced piece of a row per instruction, several rows and pieces in
// flight), multiply by the input and reduce across the wave.  At batch 1
// with d <= 4096 the input lives in registers (heads_gemv1_kernel); else it
// is staged once per workgroup in LDS as fp32 and each workgroup streams a
// long run of rows (heads_gemv_kernel).
#include "common.hpp"

namespace mvk {
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));   // a 16-byte register piece

constexpr int GEMV_RW = 2;            // rows per wave per iteration (batch-1 kernel)
constexpr int GEMV_ROWS_PER_WG = 64;  // 16 rows per wave
constexpr int GEMV_CH = 8;            // 1 KiB row pieces per lane in flight

// Batches (and batch 1 with d > 512 * GEMV_CH): the fp32 input rows [B][d]
// are staged once per workgroup in LDS, and the workgroup then streams a long
// run of rows of one head.  Eight waves; each takes GB_R rows at a time in
// blocks of GB_CH 1 KiB pieces of each, the next block's loads in flight
// during this block's math, so one LDS read of the input serves GB_R rows.
// The staging issues all its 16-byte loads before its first LDS store (a
// single memory round trip).  Measured at the 33B heads (B = 4, d = 6656,
// 2.06 GB): 1.55 ms with a per-element staging loop in 64-row workgroups,
// 0.45 ms with this layout and one block in flight, 0.42 ms with two.
constexpr int GB_WAVES = 8;
constexpr int GB_R = 4;
constexpr int GB_CH = 4;

// GB_CH pieces of GB_R rows from row r0, column c0 (rows clamped to r_last,
// columns to d - 8: always in bounds)
__device__ __forceinline__ void gb_load(u32x4v (&w)[GB_CH][GB_R], const u16* Wk, int r0, int c0,
                                        int r_last, int d, int lane) {
#pragma unroll
  for (int j = 0; j < GB_CH; ++j) {
    const int c = min(c0 + j * 512 + lane * 8, d - 8);
#pragma unroll
    for (int i = 0; i < GB_R; ++i) {
      const int r = min(r0 + i, r_last);
      w[j][i] = *reinterpret_cast<const u32x4v*>(Wk + (size_t)r * d + c);
    }
  }
}

// acc[i][b] += the block's pieces of row i against input row b
template <int MAXB>
__device__ __forceinline__ void gb_math(const u32x4v (&w)[GB_CH][GB_R], const float* xs, int d, int B,
                                        int c0, int lane, float (&acc)[GB_R][MAXB]) {
#pragma unroll
  for (int j = 0; j < GB_CH; ++j) {
    const int c = c0 + j * 512 + lane * 8;
    if (c >= d) break;
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b >= B) break;
      const float4 x0 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c);
      const float4 x1 = *reinterpret_cast<const float4*>(xs + (size_t)b * d + c + 4);
#pragma unroll
      for (int i = 0; i < GB_R; ++i) {
        float a = acc[i][b];
        a += bf16lo(w[j][i][0]) * x0.x + bf16hi(w[j][i][0]) * x0.y;
        a += bf16lo(w[j][i][1]) * x0.z + bf16hi(w[j][i][1]) * x0.w;
        a += bf16lo(w[j][i][2]) * x1.x + bf16hi(w[j][i][2]) * x1.y;
        a += bf16lo(w[j][i][3]) * x1.z + bf16hi(w[j][i][3]) * x1.w;
        acc[i][b] = a;
      }
    }
  }
}

// wave sums of the accumulators of rows r0 .. r0+GB_R-1; lane 0 stores the
// rows below r_end; the accumulators are cleared for the next row group
template <int MAXB>
__device__ __forceinline__ void gb_reduce(float (&acc)[GB_R][MAXB], const float* xs, float* out, int B,
                                          int D, int k, int d, int rows, int r0, int r_end, int mode,
                                          int lane) {
#pragma unroll
  for (int i = 0; i < GB_R; ++i) {
    const int r = r0 + i;
#pragma unroll
    for (int b = 0; b < MAXB; ++b) {
      if (b >= B) break;
      const float y = warp_sum(acc[i][b]);
      if (lane == 0 && r < r_end) {
        const size_t o = ((size_t)b * D + k) * rows + r;
        out[o] = mode == 0 ? xs[(size_t)b * d + r] + silu_f(y) : y;
      }
      acc[i][b] = 0.f;
    }
  }
}

// mode 0: y = W1 x -> u[b][k][j] = h[b][j] + SiLU(y) (x = h, bf16 input)
// mode 1: y = W2 x -> z[b][k][j] = y             (x = u[b][k], fp32 input)
template <int MAXB>
__global__ __launch_bounds__(GB_WAVES * 64) void heads_gemv_kernel(
    const u16* __restrict__ hb, const float* __restrict__ uf, const u16* __restrict__ W,
    float* __restrict__ out, int B, int D, int d, int rows, int mode, int rpw) {
  extern __shared__ float xs[];
  constexpr int NT = GB_WAVES * 64, RG = GB_WAVES * GB_R;
  const int k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u16* Wk = W + (size_t)k * rows * d;
  // the workgroup's rows r_lo .. r_hi-1 in groups of RG; wave w takes rows
  // w * GB_R .. +GB_R-1 of each group
  const int r_lo = blockIdx.x * rpw, r_hi = min(rows, r_lo + rpw);
  const int my_groups = r_hi > r_lo ? (r_hi - r_lo + RG - 1) / RG : 0;
  auto grp_row = [&](int g) { return r_lo + g * RG + wave * GB_R; };
  const int nch = (d + 512 * GB_CH - 1) / (512 * GB_CH);
  const int nblk = my_groups * nch;
  u32x4v wa[GB_CH][GB_R];
  u32x4v wb[GB_CH][GB_R];
  if (nblk > 0) gb_load(wa, Wk, grp_row(0), 0, rows - 1, d, lane);
  // ---- stage the input rows: d % 8 == 0, so a row is whole 16-byte pieces
  // (in rounds of SR pieces a thread, at most one round at 4 x 8192 fp32:
  // the loads of a round go out together; vector-typed registers and clamped
  // indexes keep the round in registers)
  constexpr int SR = 16;
  if (mode == 0) {
    const int n8 = B * d / 8;
    for (int base = 0; base < n8; base += SR * NT) {
      u32x4v t[SR];
#pragma unroll
      for (int it = 0; it < SR; ++it) {
        const int i = base + threadIdx.x + it * NT;
        t[it] = i < n8 ? reinterpret_cast<const u32x4v*>(hb)[i] : u32x4v{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int it = 0; it < SR; ++it) {
        const int i = base + threadIdx.x + it * NT;
        if (i < n8) {
          float4* dst = reinterpret_cast<float4*>(xs + 8 * i);
          dst[0] = float4{bf16lo(t[it][0]), bf16hi(t[it][0]), bf16lo(t[it][1]), bf16hi(t[it][1])};
          dst[1] = float4{bf16lo(t[it][2]), bf16hi(t[it][2]), bf16lo(t[it][3]), bf16hi(t[it][3])};
        }
      }
    }
  } else {
    const int q = d / 4, n4 = B * q;
    for (int base = 0; base < n4; base += SR * NT) {
      f32x4 t[SR];
#pragma unroll
      for (int it = 0; it < SR; ++it) {
        const int i = base + threadIdx.x + it * NT;
        const int ii = min(i, n4 - 1);
        const int b = ii / q, c4 = ii - b * q;
        t[it] = reinterpret_cast<const f32x4*>(uf + ((size_t)b * D + k) * d)[c4];
      }
#pragma unroll
      for (int it = 0; it < SR; ++it) {
        const int i = base + threadIdx.x + it * NT;
        if (i < n4) reinterpret_cast<f32x4*>(xs)[i] = t[it];
      }
    }
  }
  __syncthreads();
  float acc[GB_R][MAXB];
#pragma unroll
  for (int i = 0; i < GB_R; ++i)
#pragma unroll
    for (int b = 0; b < MAXB; ++b) acc[i][b] = 0.f;
  // blocks (row group, column chunk) in order, ping-ponging between two
  // register sets: the next block's loads go out before this block's math
  for (int bi = 0; bi < nblk; bi += 2) {
    {
      const int n1 = bi + 1;
      if (n1 < nblk) gb_load(wb, Wk, grp_row(n1 / nch), (n1 % nch) * 512 * GB_CH, rows - 1, d, lane);
      gb_math<MAXB>(wa, xs, d, B, (bi % nch) * 512 * GB_CH, lane, acc);
      if (bi % nch == nch - 1) gb_reduce<MAXB>(acc, xs, out, B, D, k, d, rows, grp_row(bi / nch), r_hi, mode, lane);
    }
    if (bi + 1 >= nblk) break;
    {
      const int n2 = bi + 2, b1 = bi + 1;
      if (n2 < nblk) gb_load(wa, Wk, grp_row(n2 / nch), (n2 % nch) * 512 * GB_CH, rows - 1, d, lane);
      gb_math<MAXB>(wb, xs, d, B, (b1 % nch) * 512 * GB_CH, lane, acc);
      if (b1 % nch == nch - 1) gb_reduce<MAXB>(acc, xs, out, B, D, k, d, rows, grp_row(b1 / nch), r_hi, mode, lane);
    }
  }
}

// Batch 1 with d <= 512 * GEMV_CH: the input row lives in registers (each
// lane holds the 8 values under each of its GEMV_CH weight pieces), so there
// is no LDS staging and no barrier before the first weight bytes are used;
// mode 0's residual input h[r] is requested with the weights of its rows.
__global__ __launch_bounds__(256) void heads_gemv1_kernel(const u16* __restrict__ hb,
                                                          const float* __restrict__ uf,
                                                          const u16* __restrict__ W,
                                                          float* __restrict__ out, int D, int d,
                                                          int rows, int mode, int rpw) {
  const int k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u16* Wk = W + (size_t)k * rows * d;
  const int r_lo = blockIdx.x * rpw;
  const int r_hi = min(rows, r_lo + rpw);
  uint4 w[GEMV_CH][GEMV_RW];
  float hres[GEMV_RW];
  auto load = [&](int r0) {
#pragma unroll
    for (int j = 0; j < GEMV_CH; ++j) {
      const int c = min(j * 512 + lane * 8, d - 8);            // clamped: in bounds
#pragma unroll
      for (int i = 0; i < GEMV_RW; ++i) {
        const int r = min(r0 + i, r_hi - 1);
        w[j][i] = *reinterpret_cast<const uint4*>(Wk + (size_t)r * d + c);
      }
    }
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i)
      hres[i] = mode == 0 ? bf16_to_f32(hb[min(r0 + i, r_hi - 1)]) : 0.f;
  };
  int r0 = r_lo + wave * GEMV_RW;
  if (r0 < r_hi) load(r0);
  float xv[GEMV_CH][8];
#pragma unroll
  for (int j = 0; j < GEMV_CH; ++j) {
    const int c = j * 512 + lane * 8;
    if (c < d && mode == 0) {
      const uint4 h8 = *reinterpret_cast<const uint4*>(hb + c);
      xv[j][0] = bf16lo(h8.x); xv[j][1] = bf16hi(h8.x); xv[j][2] = bf16lo(h8.y); xv[j][3] = bf16hi(h8.y);
      xv[j][4] = bf16lo(h8.z); xv[j][5] = bf16hi(h8.z); xv[j][6] = bf16lo(h8.w); xv[j][7] = bf16hi(h8.w);
    } else if (c < d) {
      const float4 a = *reinterpret_cast<const float4*>(uf + (size_t)k * d + c);
      const float4 b = *reinterpret_cast<const float4*>(uf + (size_t)k * d + c + 4);
      xv[j][0] = a.x; xv[j][1] = a.y; xv[j][2] = a.z; xv[j][3] = a.w;
      xv[j][4] = b.x; xv[j][5] = b.y; xv[j][6] = b.z; xv[j][7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[j][e] = 0.f;
    }
  }
  for (; r0 < r_hi; r0 += 4 * GEMV_RW) {
    float acc[GEMV_RW];
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < GEMV_CH; ++j) {
      if (j * 512 + lane * 8 >= d) break;
#pragma unroll
      for (int i = 0; i < GEMV_RW; ++i) {
        float a = acc[i];
        a += bf16lo(w[j][i].x) * xv[j][0] + bf16hi(w[j][i].x) * xv[j][1];
        a += bf16lo(w[j][i].y) * xv[j][2] + bf16hi(w[j][i].y) * xv[j][3];
        a += bf16lo(w[j][i].z) * xv[j][4] + bf16hi(w[j][i].z) * xv[j][5];
        a += bf16lo(w[j][i].w) * xv[j][6] + bf16hi(w[j][i].w) * xv[j][7];
        acc[i] = a;
      }
    }
    float hcur[GEMV_RW];
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i) hcur[i] = hres[i];
    if (r0 + 4 * GEMV_RW < r_hi) load(r0 + 4 * GEMV_RW);     // next rows before the reductions
#pragma unroll
    for (int i = 0; i < GEMV_RW; ++i) {
      const int r = r0 + i;
      const float y = warp_sum(acc[i]);
      if (lane == 0 && r < r_hi) out[(size_t)k * rows + r] = mode == 0 ? hcur[i] + silu_f(y) : y;
    }
  }
}

// The batch-1 kernel (input in registers) takes rpw rows per workgroup, a
// multiple of 4 waves x GEMV_RW, fewer when the matrix is short so that the
// grid still covers the CUs.  The staged kernel takes long row runs: about
// one workgroup per compute unit over all D heads (its LDS input allows no
// more), rpw a multiple of its 8 waves x GB_R.
static hipError_t launch_gemv(const u16* hb, const float* uf, const u16* W, float* out, int B,
                              int D, int d, int rows, int mode, hipStream_t s) {
  if (B == 1 && d <= 512 * GEMV_CH) {
    int rpw = GEMV_ROWS_PER_WG;
    while (rpw > 4 * GEMV_RW && (size_t)((rows + rpw - 1) / rpw) * D < 1024) rpw /= 2;
    dim3 grid((rows + rpw - 1) / rpw, D);
    hipLaunchKernelGGL(heads_gemv1_kernel, grid, dim3(256), 0, s, hb, uf, W, out, D, d, rows, mode, rpw);
    return hipGetLastError();
  }
  if (B < 1 || B > 4 || d % 8 || d > 8192) return hipErrorInvalidValue;
  constexpr int RG = GB_WAVES * GB_R;
  const long per_cu = ((long)rows * D + 255) / 256;
  const int rpw = (int)std::max<long>(RG, (per_cu + RG - 1) / RG * RG);
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
    hipLaunchKernelGGL((heads_gemv_kernel<1>), grid, dim3(GB_WAVES * 64), lds, s, hb, uf, W, out, B, D,
                       d, rows, mode, rpw);
  else
    hipLaunchKernelGGL((heads_gemv_kernel<4>), grid, dim3(GB_WAVES * 64), lds, s, hb, uf, W, out, B, D,
                       d, rows, mode, rpw);
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
// A (value, id) pair is ranked by one 64-bit key: an order-preserving map of
// the float (with -0 read as +0) in the high word and ~id in the low word, so
// that one unsigned comparison gives the order; NaNs get the key of an empty
// slot (-inf, id INT_MAX) and are never chosen over a number.
// Selection inside one wave: each lane sorts its (up to) 16 keys descending
// with a bitonic network and parks them in LDS; then s rounds each take the
// wave-wide maximum of the lanes' current heads (DPP inside 16-lane rows, row
// broadcasts across rows, lane 63 read into a scalar) and the winning lane
// moves to its next key.
// Stage 1: each wave takes 1024 consecutive logits (16 per lane, coalesced
// float4 loads) and writes its top s.  Stage 2: one wave per row selects the
// final s from the row's candidates the same way.
// ---------------------------------------------------------------------------
typedef unsigned long long u64;
constexpr u64 TOPK_EMPTY = ((u64)0x007fffffu << 32) | 0x80000000u;   // (-inf, INT_MAX)

__device__ __forceinline__ u64 topk_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                          // -0 ranks as +0
  const uint32_t o = (u >> 31) ? ~u : (u | 0x80000000u);
  return v != v ? TOPK_EMPTY : (((u64)o << 32) | (uint32_t)~id);
}
__device__ __forceinline__ float topk_value(u64 k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o >> 31) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int topk_id(u64 k) { return (int)~(uint32_t)k; }

template <int CTRL, bool BCAST>
__device__ __forceinline__ void key_max_step(uint32_t& hi, uint32_t& lo) {
  uint32_t ohi, olo;
  if constexpr (BCAST) {      // lanes without a source lane keep their own key
    ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
    olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  } else {
    ohi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xF, 0xF, false);
    olo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xF, 0xF, false);
  }
  if ((((u64)ohi << 32) | olo) > (((u64)hi << 32) | lo)) {
    hi = ohi;
    lo = olo;
  }
}
// The wave's largest key, in every lane.
__device__ __forceinline__ u64 wave_max_key(u64 k) {
  uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  key_max_step<0xB1, false>(hi, lo);     // quad_perm [1,0,3,2]
  key_max_step<0x4E, false>(hi, lo);     // quad_perm [2,3,0,1]
  key_max_step<0x141, false>(hi, lo);    // row_half_mirror
  key_max_step<0x140, false>(hi, lo);    // row_mirror: every lane holds its row's maximum
  key_max_step<0x142, true>(hi, lo);     // row_bcast:15: row r-1 folded into row r
  key_max_step<0x143, true>(hi, lo);     // row_bcast:31: rows 0-1 folded into rows 2-3
  return ((u64)__builtin_amdgcn_readlane(hi, 63) << 32) | (uint32_t)__builtin_amdgcn_readlane(lo, 63);
}

// key: this lane's N keys (TOPK_EMPTY = no candidate), already in descending
// order when SORTED; lst: the wave's LDS area [N][64].  Returns round r's
// winner in lane r (r < s <= 64).
template <int N, bool SORTED>
__device__ __forceinline__ u64 wave_top_keys(u64 (&key)[N], int s, u64 (*lst)[64]) {
  const int lane = threadIdx.x & 63;
  if constexpr (!SORTED) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)         // bitonic sort, descending
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const int l = i ^ j;
          if (l > i) {
            const bool desc = (i & k) == 0;
            const u64 x = key[i], y = key[l];
            const bool sw = desc ? x < y : x > y;
            key[i] = sw ? y : x;
            key[l] = sw ? x : y;
          }
        }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) lst[j][lane] = key[j];
  u64 head = key[0], nxt = key[1], mine = TOPK_EMPTY;
  int ptr = 1;                               // index of nxt
  for (int r = 0; r < s; ++r) {
    const u64 best = wave_max_key(head);
    if (head == best) {                      // keys are unique: one lane
      head = nxt;
      ++ptr;
      nxt = ptr < N ? lst[ptr][lane] : TOPK_EMPTY;
    }
    if (lane == r) mine = best;
  }
  return mine;
}

// Stage 1: wave w of a row takes logits [w * 64 * KPL, (w + 1) * 64 * KPL),
// KPL per lane in float4 pieces.
template <int KPL>
__global__ __launch_bounds__(256) void topk_partial_kernel(const float* __restrict__ z, int V,
                                                           int s_top, float* __restrict__ cv,
                                                           int* __restrict__ ci) {
  __shared__ u64 lst[4][KPL][64];
  const int row = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;                       // waves per row
  const int w = blockIdx.x * 4 + wave;
  const int base = w * 64 * KPL;
  const float* zr = z + (size_t)row * V;
  u64 key[KPL];
#pragma unroll
  for (int j = 0; j < KPL / 4; ++j) {
    const int i = base + j * 256 + lane * 4;
    float4 x = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (i + 3 < V) {
      x = *reinterpret_cast<const float4*>(zr + i);
    } else {
      if (i < V) x.x = zr[i];
      if (i + 1 < V) x.y = zr[i + 1];
      if (i + 2 < V) x.z = zr[i + 2];
    }
    const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) key[4 * j + e] = i + e < V ? topk_key(xv[e], i + e) : TOPK_EMPTY;
  }
  const u64 mine = wave_top_keys<KPL, false>(key, s_top, lst[wave]);
  if (lane < s_top) {
    const size_t o = ((size_t)row * nw + w) * s_top + lane;
    cv[o] = topk_value(mine);
    ci[o] = topk_id(mine);
  }
}

// Stage 2, one wave per row.  RUNS: lane L takes stage-1 wave L's s
// candidates, which are already in order (nw <= 64, s <= 16); otherwise the
// lanes take the ncand <= 1024 candidates 16 apiece and sort them.
template <bool RUNS>
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ cv,
                                                        const int* __restrict__ ci, int nw,
                                                        int s_top, int32_t* __restrict__ ids,
                                                        float* __restrict__ vals) {
  __shared__ u64 lst[16][64];
  const int row = blockIdx.x, lane = threadIdx.x;
  const int ncand = nw * s_top;
  u64 key[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int c = RUNS ? lane * s_top + j : j * 64 + lane;
    const bool ok = RUNS ? (lane < nw && j < s_top) : c < ncand;
    key[j] = ok ? topk_key(cv[(size_t)row * ncand + c], ci[(size_t)row * ncand + c]) : TOPK_EMPTY;
  }
  const u64 mine = wave_top_keys<16, RUNS>(key, s_top, lst);
  if (lane < s_top) {
    ids[(size_t)row * s_top + lane] = topk_id(mine);
    vals[(size_t)row * s_top + lane] = topk_value(mine);
  }
}

// logits per stage-1 lane: 8 up to a 32768-entry vocabulary, else 16
static int topk_kpl(int V) { return V <= 32768 ? 8 : 16; }
int topk_waves(int V) {
  const int span = 4 * 64 * topk_kpl(V);              // logits per workgroup
  return ((V + span - 1) / span) * 4;
}

hipError_t launch_topk(const float* z, int rows, int V, int s_top, int32_t* ids, float* vals,
                       float* cand_v, int* cand_i, hipStream_t s) {
  if (s_top < 1 || s_top > 16) return hipErrorInvalidValue;
  const int nw = topk_waves(V);
  if (nw * s_top > 1024) return hipErrorInvalidValue;
  if (topk_kpl(V) == 8)
    hipLaunchKernelGGL((topk_partial_kernel<8>), dim3(nw / 4, rows), dim3(256), 0, s, z, V, s_top,
                       cand_v, cand_i);
  else
    hipLaunchKernelGGL((topk_partial_kernel<16>), dim3(nw / 4, rows), dim3(256), 0, s, z, V, s_top,
                       cand_v, cand_i);
  if (nw <= 64)
    hipLaunchKernelGGL((topk_merge_kernel<true>), dim3(rows), dim3(64), 0, s, cand_v, cand_i, nw,
                       s_top, ids, vals);
  else
    hipLaunchKernelGGL((topk_merge_kernel<false>), dim3(rows), dim3(64), 0, s, cand_v, cand_i, nw,
                       s_top, ids, vals);
  return hipGetLastError();
}

// tok[b][v] = root[b] for v = 0, else top_ids[b][depth(v)-1][rank(v)].
// Calibration counts of the heads' ranks (Medusa paper digest, Method 4:
// accuracy of the i-th top prediction of head k alone): one thread per
// (position, head) adds 1 to counts[k][i] for every rank i whose candidate
// equals the label.  Integer atomics: the counts do not depend on order.
__global__ __launch_bounds__(256) void head_accuracy_kernel(const int32_t* __restrict__ top_ids,
                                                            const int32_t* __restrict__ labels,
                                                            int NK, int K, int s,
                                                            int32_t* __restrict__ counts) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= NK) return;
  const int k = t % K;
  const int lab = labels[t];
  for (int i = 0; i < s; ++i)
    if (top_ids[(size_t)t * s + i] == lab) atomicAdd(&counts[k * s + i], 1);
}

hipError_t launch_head_accuracy(const int32_t* top_ids, const int32_t* labels, int N, int K, int s,
                                int32_t* counts, hipStream_t st) {
  const int NK = N * K;
  if (NK > 0)
    hipLaunchKernelGGL(head_accuracy_kernel, dim3((NK + 255) / 256), dim3(256), 0, st, top_ids,
                       labels, NK, K, s, counts);
  return hipGetLastError();
}

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
