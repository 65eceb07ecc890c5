// Tree attention: every tree node (query) attends to the whole cached prefix
// (slots 0 .. n-1) and to the tree slots n + a of its own ancestors a (itself
// included), with position ids already applied to q and k by RoPE.
//
// Data: q bf16 [B][T][H][hd] (rows of the fused QKV output); K cache bf16
// [B][H][cap][hd]; V cache bf16 [B][H][cap/4][hd][4] (four consecutive slots
// interleaved per dim, so that the four keys a lane needs for one dim are one
// 8-byte load); ancestor bitmask uint64 [B][T][mask_words], bit a of node v's
// words set iff a is v or an ancestor of v.
//
// Decomposition: a workgroup owns one (key range, head, batch x 64-query
// group).  Key ranges split the prefix into `nsplit` tile-aligned pieces sized
// from the device-side n (so one launch shape serves every n up to the
// capacity); range `nsplit` is the tree itself.  The 4 waves each take 16
// queries and walk the range in 64-key tiles, sharing K/V tiles through the
// caches.  Per tile a wave issues all K and V loads at once, computes
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on rows, queries on columns:
// each lane then owns one query, so the softmax statistics and the rescaling
// of the output are lane-local up to a 4-lane reduction), updates an online
// softmax in the log2 domain, and accumulates O^T = V^T P^T with the
// probabilities reused straight from the S^T registers (the MFMA K index is
// permuted to match them).  Each range writes an unnormalised partial
// (o, m, l); attn_combine merges the ranges.
#include "common.hpp"

namespace mvk {

template <int HD>
__global__ __launch_bounds__(256) void tree_attention_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int32_t* __restrict__ n_prefix, const uint64_t* __restrict__ anc, int B, int T, int H,
    int cap, int mw, int nsplit, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int DB32 = (HD + 31) / 32;   // 32-dim blocks of the QK contraction
  constexpr int DB16 = HD / 16;          // 16-dim blocks of the output
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, qi = lane & 15;
  const int split = blockIdx.x, h = blockIdx.y;
  const int QG = (T + 63) / 64;
  const int b = blockIdx.z / QG, qg = blockIdx.z % QG;
  const int qidx = qg * 64 + wave * 16 + qi;         // this lane's query (tree node)
  const bool qvalid = qidx < T;
  const int qrow = qvalid ? qidx : T - 1;
  if (qg * 64 + wave * 16 >= T) return;              // whole wave idle (no barriers below)

  // n + T <= cap is the caller's contract; clamping keeps every load in bounds
  const int n = min(max(n_prefix[b], 0), cap - T);
  const int d = H * HD;
  int lo, hi;
  if (split < nsplit) {
    int per = (n + nsplit - 1) / nsplit;
    per = (per + 63) & ~63;
    lo = split * per;
    hi = min(n, lo + per);
  } else {
    lo = n;
    hi = n + T;
  }
  const size_t row = ((size_t)split * B * T + (size_t)b * T + qidx) * H + h;
  if (lo >= hi) {                    // empty range: marked by m = -inf alone
    if (qvalid && g == 0) {
      part_ml[row * 2 + 0] = -INFINITY;
      part_ml[row * 2 + 1] = 0.f;
    }
    return;
  }
  const size_t bh = (size_t)b * H + h;
  const u16* kbase = kc + bh * cap * HD;
  const u16* vbase = vc + bh * (size_t)(cap >> 2) * HD * 4;

  // Q^T fragments (B operand): lane owns query qi, dims 32*db + 8*g .. +8.
  bf16x8 qf[DB32];
#pragma unroll
  for (int db = 0; db < DB32; ++db) {
    const int dim = db * 32 + g * 8;
    qf[db] = dim < HD ? *reinterpret_cast<const bf16x8*>(q + ((size_t)(b * T + qrow) * d + h * HD + dim))
                      : bf16x8{};
  }
  uint64_t am[4] = {0, 0, 0, 0};
  if (split == nsplit) {
    for (int w = 0; w < mw && w < 4; ++w) am[w] = anc[((size_t)b * T + qrow) * mw + w];
  }

  const float scale = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(hd)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB16];
#pragma unroll
  for (int i = 0; i < DB16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s0 = lo & ~63; s0 < hi; s0 += 64) {
    // ---- all loads of the tile first: K (A operand of S^T) and V (A of O^T) ----
    bf16x8 kf[4][DB32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = s0 + kb * 16 + qi;
#pragma unroll
      for (int db = 0; db < DB32; ++db) {
        const int dim = db * 32 + g * 8;
        kf[kb][db] = dim < HD ? *reinterpret_cast<const bf16x8*>(kbase + (size_t)key * HD + dim)
                              : bf16x8{};
      }
    }
    // V^T operand, 32-key half kk: slot j<4 -> key kk*32 + 4g + j,
    // j>=4 -> kk*32 + 16 + 4g + j-4 (matches the S^T register layout)
    uint2 va[2][DB16], vb[2][DB16];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int sa = s0 + kk * 32 + g * 4, sb = sa + 16;
#pragma unroll
      for (int i = 0; i < DB16; ++i) {
        const int dim = i * 16 + qi;
        va[kk][i] = *reinterpret_cast<const uint2*>(vbase + (((size_t)(sa >> 2) * HD + dim) << 2));
        vb[kk][i] = *reinterpret_cast<const uint2*>(vbase + (((size_t)(sb >> 2) * HD + dim) << 2));
      }
    }
    // ---- S^T = K Q^T for 64 keys (4 blocks of 16) ----
    f32x4 st[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < DB32; ++db) st[kb] = mfma16x16x32(kf[kb][db], qf[db], st[kb]);
    }
    // ---- mask + online softmax (log2 domain); lane holds keys kb*16+4g+r ----
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = s0 + kb * 16 + g * 4 + r;
        bool ok = slot >= lo && slot < hi;
        if (split == nsplit && ok) {
          const int a = slot - n;
          ok = (am[a >> 6] >> (a & 63)) & 1ull;
        }
        const float sv = ok ? st[kb][r] * scale : -INFINITY;
        st[kb][r] = sv;
        tmax = fmaxf(tmax, sv);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (st[kb][r] == -INFINITY) ? 0.f : exp2f(st[kb][r] - m_new);
        st[kb][r] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DB16; ++i) o[i] *= alpha;

    // ---- O^T += V^T P^T over the two 32-key halves ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf[j] = (__bf16)st[2 * kk][j];
        pf[j + 4] = (__bf16)st[2 * kk + 1][j];
      }
      const int sa = s0 + kk * 32 + g * 4, sb = sa + 16;
      // values of slots outside the range are zeroed: never-written cache
      // memory could hold non-finite patterns and 0 * NaN would poison O
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int base = (e < 2 ? sa : sb) + (e & 1) * 2;
        keep[e] = ((base >= lo && base < hi) ? 0x0000ffffu : 0u) |
                  ((base + 1 >= lo && base + 1 < hi) ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int i = 0; i < DB16; ++i) {
        const uint4 w = {va[kk][i].x & keep[0], va[kk][i].y & keep[1], vb[kk][i].x & keep[2],
                         vb[kk][i].y & keep[3]};
        o[i] = mfma16x16x32(__builtin_bit_cast(bf16x8, w), pf, o[i]);
      }
    }
  }

  // ---- write the unnormalised partial of this range ----
  if (qvalid) {
    float* po = part_o + row * HD;
#pragma unroll
    for (int i = 0; i < DB16; ++i)
      *reinterpret_cast<float4*>(po + i * 16 + g * 4) = float4{o[i][0], o[i][1], o[i][2], o[i][3]};
    if (g == 0) {
      part_ml[row * 2 + 0] = m_run;
      part_ml[row * 2 + 1] = l_run;
    }
  }
}

// Merge the nsplit+1 range partials of one (row, head):
//   o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c.
// One wave per (row, head): lane c reads range c's (m, l) (nsplit + 1 <= 64),
// weights come from wave reductions, then each lane accumulates its dims of
// the non-empty ranges.  Output bf16, row-major [B*T][d] or fragment-packed
// [Mp][d] (the A operand of the O projection; pad rows written as zeros).
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           u16* __restrict__ out, int packed,
                                                           int BT, int H, int nsplit, int rows) {
  constexpr int PER = (HD + 63) / 64;            // dims per lane (hd 128 -> 2)
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= rows * H) return;
  const int m = wid / H, h = wid % H;
  const int d = H * HD;
  float val[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) val[j] = 0.f;
  if (m < BT) {
    const int ns = nsplit + 1;
    float ms = -INFINITY, ls = 0.f;
    if (lane < ns) {
      const size_t r = ((size_t)lane * BT + m) * H + h;
      ms = part_ml[r * 2];
      ls = part_ml[r * 2 + 1];
    }
    const float M = warp_max(ms);
    const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
    const float den = warp_sum(w * ls);
    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    for (int c = 0; c < ns; ++c) {
      const float wc = __shfl(w, c, 64);
      if (wc == 0.f) continue;
      const float* po = part_o + (((size_t)c * BT + m) * H + h) * HD;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = j * 64 + lane;
        if (i < HD) acc[j] += wc * po[i];
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) val[j] = acc[j] / den;
  } else if (!packed) {
    return;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * 64 + lane;
    if (i >= HD) continue;
    const int c = h * HD + i;
    const u16 ob = f32_to_bf16(val[j]);
    if (packed) out[packed_index(m, c, d)] = ob;
    else out[(size_t)m * d + c] = ob;
  }
}

hipError_t launch_attention(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                            const uint64_t* anc, int B, int T, int H, int hd, int cap, int mw,
                            int nsplit, float* part_o, float* part_ml, hipStream_t s) {
  const int QG = (T + 63) / 64;
  dim3 grid(nsplit + 1, H, B * QG);
  switch (hd) {
    case 16: hipLaunchKernelGGL((tree_attention_kernel<16>), grid, dim3(256), 0, s, q, kc, vc, n_prefix, anc, B, T, H, cap, mw, nsplit, part_o, part_ml); break;
    case 32: hipLaunchKernelGGL((tree_attention_kernel<32>), grid, dim3(256), 0, s, q, kc, vc, n_prefix, anc, B, T, H, cap, mw, nsplit, part_o, part_ml); break;
    case 64: hipLaunchKernelGGL((tree_attention_kernel<64>), grid, dim3(256), 0, s, q, kc, vc, n_prefix, anc, B, T, H, cap, mw, nsplit, part_o, part_ml); break;
    case 128: hipLaunchKernelGGL((tree_attention_kernel<128>), grid, dim3(256), 0, s, q, kc, vc, n_prefix, anc, B, T, H, cap, mw, nsplit, part_o, part_ml); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const float* part_o, const float* part_ml, u16* out, int packed,
                               int B, int T, int H, int hd, int nsplit, int Mp, hipStream_t s) {
  if (nsplit + 1 > 64) return hipErrorInvalidValue;
  const int rows = packed ? Mp : B * T;
  const int blocks = (rows * H + 3) / 4;
  switch (hd) {
    case 16: hipLaunchKernelGGL((attn_combine_kernel<16>), dim3(blocks), dim3(256), 0, s, part_o, part_ml, out, packed, B * T, H, nsplit, rows); break;
    case 32: hipLaunchKernelGGL((attn_combine_kernel<32>), dim3(blocks), dim3(256), 0, s, part_o, part_ml, out, packed, B * T, H, nsplit, rows); break;
    case 64: hipLaunchKernelGGL((attn_combine_kernel<64>), dim3(blocks), dim3(256), 0, s, part_o, part_ml, out, packed, B * T, H, nsplit, rows); break;
    case 128: hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(blocks), dim3(256), 0, s, part_o, part_ml, out, packed, B * T, H, nsplit, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mvk
