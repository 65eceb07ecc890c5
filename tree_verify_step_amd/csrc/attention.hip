// Tree attention: every tree node (query) attends to the whole cached prefix
// (slots 0 .. n-1) and to the tree slots n + a of its own ancestors a (itself
// included), with position ids already applied to q and k by RoPE.
//
// Data: q bf16 [B][T][H][hd] (rows of the fused QKV output); K and V caches
// in the layouts of kv_k_off / kv_v_off, per (sequence, head) block of
// cap * hd elements; ancestor bitmask uint64 [B][T][mask_words], bit a of
// node v's words set iff a is v or an ancestor of v.
//
// Key order inside a 32-key half kk of a tile: row R of S^T block 2*kk + e
// holds key 32*kk + 8*(R>>2) + 4*e + (R&3).  Lane group g then holds the
// probabilities of keys 32*kk + 8*g .. +7, in order, which is one 16-byte V
// load per dim, and the K operand rows of a block are 16 consecutive rows of
// the K layout: every K and V load instruction reads whole cache lines.
//
// Decomposition: a workgroup owns 16 queries of one (sequence, head); its NW
// waves split the key slots 0 .. n+T-1 (prefix, then tree) in 64-key tiles,
// tile t going to wave t mod NW, so every K/V byte is read once per query
// block and the tile count follows the device-side n (one launch shape
// serves every n up to the capacity).  Per tile a wave issues all K and V
// loads at once, computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on
// rows, queries on columns: each lane owns one query, so the softmax
// statistics and the rescaling of the output are lane-local up to a 4-lane
// reduction), masks (prefix: visible; tree: ancestor bit; past n+T: hidden),
// updates an online softmax in the log2 domain, and accumulates
// O^T = V^T P^T with the probabilities reused straight from the S^T registers
// (the MFMA K index is permuted to match them).  The waves' (m, l, o) are
// merged in LDS in wave order (deterministic) and the normalised output is
// written as bf16, row-major or fragment-packed (the O projection's operand).
#include "common.hpp"

namespace mvk {

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64) void tree_attention_kernel(
    const u16* __restrict__ q, const u16* __restrict__ kc, const u16* __restrict__ vc,
    const int32_t* __restrict__ n_prefix, const uint64_t* __restrict__ anc, int B, int T, int H,
    int cap, int mw, u16* __restrict__ out, int packed) {
  constexpr int DB32 = (HD + 31) / 32;   // 32-dim blocks of the QK contraction
  constexpr int DB16 = HD / 16;          // 16-dim blocks of the output
  constexpr int LDO = HD + 4;            // padded row of the LDS output slots
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ float s_o[NW][16 * LDO];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, qi = lane & 15;
  // XCD-aware placement: workgroups are dispatched round-robin over the 8
  // XCDs (separate L2s), so workgroup L runs on XCD L % 8.  All query blocks
  // of one (sequence, head) pair get ids congruent mod 8, so that pair's K/V
  // tiles are fetched into a single L2 and shared from there.  (Placement
  // only: any mapping computes the same result.)
  const int QB = (T + 15) >> 4;
  const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
  const int pair = xcd + 8 * (j / QB), qb = j % QB;
  if (pair >= B * H) return;
  const int b = pair / H, h = pair % H;
  const int qidx = qb * 16 + qi;                     // this lane's query (tree node)
  const int qrow = qidx < T ? qidx : T - 1;

  const int n_raw = n_prefix[b];    // issued first: loads complete in issue order
  const size_t bh = (size_t)b * H + h;
  const u16* kbase = kc + bh * cap * HD;
  const u16* vbase = vc + bh * cap * HD;

  // ---- K (A operand of S^T) and V (A operand of O^T) of one 64-key tile ----
  bf16x8 kf[4][DB32];
  // V^T operand of 32-key half kk: lane group g's keys 32*kk + 8g .. +7
  // (va: the first four, vb: the last four)
  uint2 va[2][DB16], vb[2][DB16];
  auto load_tile = [&](int s0) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // rows 16*(kb&1) .. +15 of the tile's 32-key group kb>>1
      const size_t grp = (size_t)(s0 >> 5) + (kb >> 1);
#pragma unroll
      for (int db = 0; db < DB32; ++db) {
        const int dim = db * 32 + g * 8;
        kf[kb][db] = dim < HD ? *reinterpret_cast<const bf16x8*>(
                                    kbase + ((grp * (HD / 8) + (dim >> 3)) * 32 + (kb & 1) * 16 + qi) * 8)
                              : bf16x8{};
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int sv = s0 + kk * 32 + g * 8;
#pragma unroll
      for (int i = 0; i < DB16; ++i) {
        const int dim = i * 16 + qi;
        const uint4 w = *reinterpret_cast<const uint4*>(vbase + ((size_t)(sv >> 3) * HD + dim) * 8);
        va[kk][i] = uint2{w.x, w.y};
        vb[kk][i] = uint2{w.z, w.w};
      }
    }
  };
  // this wave's first tile does not depend on n: its loads go out before n
  // is known (clamped into the cache; unused if the tile is past n + T)
  load_tile(min(wave, (cap >> 6) - 1) * 64);

  // n + T <= cap is the caller's contract; clamping keeps every load in bounds
  const int n = min(max(n_raw, 0), cap - T);
  const int d = H * HD;
  const int lo = 0, hi = n + T;
  const int ntiles = (hi + 63) >> 6;

  // Q^T fragments (B operand): lane owns query qi, dims 32*db + 8*g .. +8.
  bf16x8 qf[DB32];
#pragma unroll
  for (int db = 0; db < DB32; ++db) {
    const int dim = db * 32 + g * 8;
    qf[db] = dim < HD ? *reinterpret_cast<const bf16x8*>(q + ((size_t)(b * T + qrow) * d + h * HD + dim))
                      : bf16x8{};
  }
  uint64_t am[4];
#pragma unroll
  for (int w = 0; w < 4; ++w)                 // unrolled: no wait until the mask is used
    am[w] = w < mw ? anc[((size_t)b * T + qrow) * mw + w] : 0ull;

  const float scale = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(hd)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB16];
#pragma unroll
  for (int i = 0; i < DB16; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t = wave; t < ntiles; t += NW) {
    const int s0 = t * 64;
    if (t != wave) {           // later tiles: all K and V loads issued before the math
      load_tile(s0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- S^T = K Q^T for 64 keys (4 blocks of 16) ----
    f32x4 st[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < DB32; ++db) st[kb] = mfma16x16x32(kf[kb][db], qf[db], st[kb]);
    }
    // ---- mask + online softmax (log2 domain); lane holds keys
    // s0 + 32*(kb>>1) + 8g + 4*(kb&1) + r ----
    // prefix tiles (all keys below n) need no mask: a uniform fast path
    const bool full = s0 + 64 <= n;
    float tmax = -INFINITY;
    if (full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st[kb][r] *= scale;
          tmax = fmaxf(tmax, st[kb][r]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = s0 + (kb >> 1) * 32 + g * 8 + (kb & 1) * 4 + r;
          bool ok = slot < n;
          if (slot >= n && slot < hi) {
            const int a = slot - n;
            ok = (am[a >> 6] >> (a & 63)) & 1ull;
          }
          const float sv = ok ? st[kb][r] * scale : -INFINITY;
          st[kb][r] = sv;
          tmax = fmaxf(tmax, sv);
        }
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
      if (full) {
#pragma unroll
        for (int i = 0; i < DB16; ++i) {
          const uint4 w = {va[kk][i].x, va[kk][i].y, vb[kk][i].x, vb[kk][i].y};
          o[i] = mfma16x16x32(__builtin_bit_cast(bf16x8, w), pf, o[i]);
        }
      } else {
        const int sv = s0 + kk * 32 + g * 8;
        // values of slots outside the range are zeroed: never-written cache
        // memory could hold non-finite patterns and 0 * NaN would poison O
        uint32_t keep[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int base = sv + 2 * e;
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
  }


  // ---- merge the waves' partial softmax states (wave order) ----
  if (g == 0) {
    s_m[wave][qi] = m_run;
    s_l[wave][qi] = l_run;
  }
#pragma unroll
  for (int i = 0; i < DB16; ++i)
    *reinterpret_cast<float4*>(&s_o[wave][qi * LDO + i * 16 + g * 4]) =
        float4{o[i][0], o[i][1], o[i][2], o[i][3]};
  __syncthreads();
  // per query: wave w's weight 2^(m_w - M) / sum_w 2^(m_w - M) l_w; each
  // thread forms 8 consecutive output dims of one query (one 16-byte store)
  constexpr int PPQ = HD / 8;                   // output pieces per query
  for (int e = threadIdx.x; e < 16 * PPQ; e += NW * 64) {
    const int qq = e / PPQ, c8 = (e % PPQ) * 8;
    const int node = qb * 16 + qq;
    if (node >= T) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][qq]);
    float f[NW], den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = s_m[w][qq] == -INFINITY ? 0.f : exp2f(s_m[w][qq] - M);
      den += f[w] * s_l[w][qq];
    }
    const float inv = 1.f / den;
    float val[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) val[t] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = f[w] * inv;
      const float4 a = *reinterpret_cast<const float4*>(&s_o[w][qq * LDO + c8]);
      const float4 c = *reinterpret_cast<const float4*>(&s_o[w][qq * LDO + c8 + 4]);
      val[0] += wt * a.x; val[1] += wt * a.y; val[2] += wt * a.z; val[3] += wt * a.w;
      val[4] += wt * c.x; val[5] += wt * c.y; val[6] += wt * c.z; val[7] += wt * c.w;
    }
    uint32_t pk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      pk[t] = (uint32_t)f32_to_bf16(val[2 * t]) | ((uint32_t)f32_to_bf16(val[2 * t + 1]) << 16);
    const int m = b * T + node, c = h * HD + c8;
    u16* dst = packed ? out + packed_index(m, c, d) : out + (size_t)m * d + c;
    *reinterpret_cast<uint4*>(dst) = uint4{pk[0], pk[1], pk[2], pk[3]};
  }
}

// Launches with many (sequence, head, query block) triples use 4-wave
// workgroups: two of them fit a compute unit where one 8-wave workgroup does
// (212 registers a lane), so more K/V tiles are in flight per unit.
template <int HD>
static void launch_attention_hd(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                                const uint64_t* anc, int B, int T, int H, int cap, int mw,
                                u16* out, int packed, hipStream_t s) {
  const int QB = (T + 15) / 16, pairs = B * H;
  const dim3 grid(8 * ((pairs + 7) / 8) * QB);
  if ((size_t)pairs * QB > 512)
    hipLaunchKernelGGL((tree_attention_kernel<HD, 4>), grid, dim3(256), 0, s, q, kc, vc, n_prefix,
                       anc, B, T, H, cap, mw, out, packed);
  else
    hipLaunchKernelGGL((tree_attention_kernel<HD, 8>), grid, dim3(512), 0, s, q, kc, vc, n_prefix,
                       anc, B, T, H, cap, mw, out, packed);
}

hipError_t launch_attention(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                            const uint64_t* anc, int B, int T, int H, int hd, int cap, int mw,
                            u16* out, int packed, hipStream_t s) {
  switch (hd) {
    case 16: launch_attention_hd<16>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
    case 32: launch_attention_hd<32>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
    case 64: launch_attention_hd<64>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
    case 128: launch_attention_hd<128>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mvk
