// Tree attention: every tree node (query) attends to the whole cached prefix
// (slots 0 .. n-1) and to the tree slots n + a of its own ancestors a (itself
// included), with position ids already applied to q and k by RoPE.
//
// Data: q bf16 [B][T][H][hd] (rows of the fused QKV output); K and V caches
// in the layouts of kv_k_off / kv_v_off, per (sequence, head) block of
// cap * hd elements; ancestor bitmask uint64 [B][T][mask_words], bit a of
// node v's words set iff a is v or an ancestor of v.
//
// Two decompositions, chosen per launch shape on the host
// (attention_uses_splits): one workgroup per 16 queries for caches of up
// to 2048 slots or grids that fill the chip (tree_attention_qb_kernel,
// further below), and split key ranges for long caches under small grids:
//
// Split-KV: the key slots 0 .. n+T-1 of one (sequence, head) pair are cut
// into 64-key tiles, and the S workgroups of the pair take every S-th tile
// (split s: tiles s, s+S, ...).  A tile of K (16 KiB at hd = 128) and of V is
// one contiguous run of the cache in both layouts; the workgroup streams it
// into LDS once (two tiles' loads in flight ahead of the one in use) and all
// tree queries of the pair use it: wave w owns query blocks w*QPW ..
// w*QPW+QPW-1 (16 queries each).  So every K/V byte is read from memory once
// per layer, and the grid (pairs x S) fills the chip even at batch 1.  The
// tile count follows the device-side n: one launch shape serves every n up
// to the capacity, and at a given n the kernel uses the fewest splits that
// reach the shortest per-split tile count.
//
// Per tile and query block a wave computes S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (keys on rows, queries on columns: each lane owns
// one query, so the softmax statistics and the rescaling of the output are
// lane-local up to a 4-lane reduction), masks (prefix: visible; tree:
// ancestor bit; past n+T: hidden), updates an online softmax in the log2
// domain, and accumulates O^T = V^T P^T with the probabilities reused from
// the S^T registers.  Key order inside a 32-key half kk of a tile: row R of
// S^T block 2*kk + e holds key 32*kk + 8*(R>>2) + 4*e + (R&3), so lane group
// g holds the probabilities of keys 32*kk + 8*g .. +7 in order -- exactly the
// P^T operand -- and the K rows of block e are rows 16e .. 16e+15 of the K
// layout's 32-slot group, the V operand one 16-byte piece of the V layout.
//
// With S > 1 each split writes its unnormalised O, its running max m and
// sum l per query, and a second, small launch merges the S partial states in
// split order (deterministic) into the normalised output, bf16, row-major or
// fragment-packed (the O projection's operand).  (An exchange inside one
// launch -- write-through stores, an arrival counter and a wait -- measured
// about 10 us per layer of round trips on this part; the launch boundary
// makes the plain stores visible to every XCD for the price of a launch.)
// With S == 1 the single split writes the output itself.
#include "common.hpp"

namespace mvk {

// Visibility of the 64 key slots s0 .. s0+63 for one query: bit j is set iff
// slot s0 + j lies below hi = n + T and is either a prefix slot (below n) or
// the tree slot n + a of an ancestor a of the query (am: the query's
// ancestor words, bit a of word a / 64, zero past the tree).  The tree part
// is the 64-bit window of the ancestor mask that starts at index s0 - n: a
// funnel shift of two neighbouring words, indices below zero reading as
// zero.  s0, n and hi are the same for the whole wave, so the selects below
// are uniform; the per-key tests then become constant bit positions (the
// per-key form, with a branch and a dynamic word index per key, cost more
// than the tile's whole softmax).  The words come in by value: picked from
// an array by a computed index, they were placed in scratch memory.
__host__ __device__ __forceinline__ uint64_t slot_visibility(uint64_t a0, uint64_t a1, uint64_t a2,
                                                             uint64_t a3, int s0, int n, int hi) {
  auto low_bits = [](int c) { return c >= 64 ? ~0ull : c <= 0 ? 0ull : (1ull << c) - 1ull; };
  auto word = [&](int i) { return i == 0 ? a0 : i == 1 ? a1 : i == 2 ? a2 : i == 3 ? a3 : 0ull; };
  const int dl = s0 - n;                        // ancestor index of the tile's first slot
  uint64_t tree = 0ull;
  if (dl > -64 && dl < 0) {
    tree = a0 << (-dl);
  } else if (dl >= 0 && dl < 256) {
    const int wi = dl >> 6, sh = dl & 63;
    tree = sh == 0 ? word(wi) : (word(wi) >> sh) | (word(wi + 1) << (64 - sh));
  }
  return low_bits(n - s0) | (tree & low_bits(hi - s0));
}

struct AttnArgs {
  const u16* q;
  const u16* kc;
  const u16* vc;
  const int32_t* n_prefix;
  const uint64_t* anc;
  int B, T, H, cap, mw;
  u16* out;
  int packed;
  int S;               // key splits per (sequence, head)
  float* part_o;       // S > 1: [pairs][S][ceil(T/16)*16][hd] unnormalised outputs (fragment order)
  float2* part_ml;     //        [pairs][S][T] (running max, running sum)
};

// K and V tiles of 64 keys, their in-cache layouts kept (both are one
// contiguous run of 64 * HD bf16 per tensor).
template <int HD>
struct AttnTile {
  bf16x8 k[64 * HD / 8];
  bf16x8 v[64 * HD / 8];
};

// 16-byte pieces of one tile's K and V that one thread moves (a register
// stage of the global -> LDS pipeline)
template <int N>
struct TileRegs {
  bf16x8 k[N], v[N];
};

template <int HD, int QPW>
__global__ __launch_bounds__(256) void tree_attention_kernel(AttnArgs a) {
  constexpr int NW = 4;                      // waves
  constexpr int DB32 = (HD + 31) / 32;       // 32-dim blocks of the QK contraction
  constexpr int DB16 = HD / 16;              // 16-dim blocks of the output
  constexpr int PIECES = 64 * HD / 8;        // 16-byte pieces of one K (or V) tile
  constexpr int PPT = PIECES / (NW * 64);    // ... per thread (HD >= 32); HD = 16: 1/2
  constexpr int PPT_ = PPT > 0 ? PPT : 1;
  // tiles in flight ahead of the one being used: two while the registers
  // allow it (one query block per wave), else one
  constexpr int PF = QPW == 1 ? 2 : 1;
  __shared__ AttnTile<HD> tile[2];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, qi = lane & 15;
  // placement: workgroups are dispatched round-robin over the 8 XCDs, so
  // workgroup L runs on XCD L % 8; all splits of a pair get ids congruent
  // mod 8 (one L2 holds the pair's partial states)
  const int xcd = blockIdx.x & 7, j8 = blockIdx.x >> 3;
  const int pair = xcd + 8 * (j8 / a.S), split = j8 % a.S;
  if (pair >= a.B * a.H) return;
  const int b = pair / a.H, h = pair % a.H;
  const int T = a.T;
  const int n_raw = a.n_prefix[b];           // issued first
  const size_t bh = (size_t)b * a.H + h;
  const bf16x8* kbase = reinterpret_cast<const bf16x8*>(a.kc + bh * a.cap * HD);
  const bf16x8* vbase = reinterpret_cast<const bf16x8*>(a.vc + bh * a.cap * HD);

  // ---- the global -> register -> LDS tile pipeline.  Pieces are taken in
  // order, so each tensor's 64 * HD * 2 bytes are read as one coalesced run.
  auto load_tile = [&](TileRegs<PPT_>& r, int t) {
    const int t_c = min(t, (a.cap >> 6) - 1);          // clamped into the cache
#pragma unroll
    for (int i = 0; i < PPT_; ++i) {
      const int p = i * NW * 64 + threadIdx.x;
      if (PPT > 0 || p < PIECES) {
        r.k[i] = kbase[(size_t)t_c * PIECES + p];
        r.v[i] = vbase[(size_t)t_c * PIECES + p];
      }
    }
  };
  // values of slots at or past hi are zeroed: never-written cache memory
  // could hold non-finite patterns, and 0 * NaN would poison O
  auto store_tile = [&](const TileRegs<PPT_>& r, int buf, int t, int hi) {
#pragma unroll
    for (int i = 0; i < PPT_; ++i) {
      const int p = i * NW * 64 + threadIdx.x;
      if (PPT > 0 || p < PIECES) {
        tile[buf].k[p] = r.k[i];
        // V piece p holds slots 8 * (p / HD) .. +7 of dim p % HD
        const int s8 = t * 64 + 8 * (p / HD);
        bf16x8 v = r.v[i];
        if (s8 + 8 > hi) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (s8 + j >= hi) v[j] = (__bf16)0.f;
        }
        tile[buf].v[p] = v;
      }
    }
  };
  // this split's first tile does not depend on n: its loads go out now
  // (splits past the ones a short prefix uses waste them)
  TileRegs<PPT_> ra, rb;
  load_tile(ra, split);

  // Q^T fragments (B operand) of the wave's query blocks: lane owns query
  // 16 * qb + qi, dims 32 * db + 8 * g .. +8; and its ancestor words
  const int d = a.H * HD;
  bf16x8 qf[QPW][DB32];
  uint64_t am[QPW][4];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qidx = (wave * QPW + j) * 16 + qi;
    const int qrow = min(qidx, T - 1);
#pragma unroll
    for (int db = 0; db < DB32; ++db) {
      const int dim = db * 32 + g * 8;
      qf[j][db] = dim < HD ? *reinterpret_cast<const bf16x8*>(
                                 a.q + ((size_t)(b * T + qrow) * d + h * HD + dim))
                           : bf16x8{};
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) am[j][w] = w < a.mw ? a.anc[((size_t)b * T + qrow) * a.mw + w] : 0ull;
  }
  // query blocks of this wave that hold real queries
  const int qb_live = min(QPW, max(0, (T + 15) / 16 - wave * QPW));

  // n + T <= cap is the caller's contract; clamping keeps every load in bounds
  const int n = min(max(n_raw, 0), a.cap - T);
  const int hi = n + T;
  const int ntiles = (hi + 63) >> 6;
  // splits in use at this n: the fewest that reach the shortest per-split
  // tile count (so no split waits on one with an extra tile); the others exit
  const int per = (ntiles + a.S - 1) / a.S;
  const int S = (ntiles + per - 1) / per;
  if (split >= S) return;
  const int my_tiles = (ntiles - 1 - split) / S + 1;
  if (PF == 2 && my_tiles > 1) load_tile(rb, split + S);

  const float scale = 1.4426950408889634f / sqrtf((float)HD);   // log2(e) / sqrt(hd)
  float m_run[QPW], l_run[QPW];
  f32x4 o[QPW][DB16];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int i = 0; i < DB16; ++i) o[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // one tile of keys from LDS buffer buf for all the wave's query blocks
  auto use_tile = [&](int buf, int t) {
    const int s0 = t * 64;
    const bool full = s0 + 64 <= n;                      // all keys in the prefix
    const AttnTile<HD>& tl = tile[buf];
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      if (j >= qb_live) break;                            // wave-uniform
      // ---- S^T = K Q^T for 64 keys (blocks kb = 2 * kk + e) ----
      f32x4 st[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kk = kb >> 1, e = kb & 1;
#pragma unroll
        for (int db = 0; db < DB32; ++db) {
          const int piece = 4 * db + g;                   // 8-dim piece of the lane's k-chunk
          const bf16x8 kf = piece < HD / 8 ? tl.k[(kk * (HD / 8) + piece) * 32 + 16 * e + qi]
                                           : bf16x8{};
          st[kb] = mfma16x16x32(kf, qf[j][db], st[kb]);
        }
      }
      // ---- mask + online softmax (log2 domain); lane holds keys
      // s0 + 32 * kk + 8 * g + 4 * e + r ----
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
        // lane group g's keys: bits 8g .. 8g+7 (kk = 0) and 32+8g .. (kk = 1)
        const uint64_t vis = slot_visibility(am[j][0], am[j][1], am[j][2], am[j][3], s0, n, hi);
        const uint32_t vbits[2] = {(uint32_t)(vis >> (8 * g)) & 0xffu, (uint32_t)(vis >> (32 + 8 * g)) & 0xffu};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = (vbits[kb >> 1] >> ((kb & 1) * 4 + r)) & 1u;
            const float sv = ok ? st[kb][r] * scale : -INFINITY;
            st[kb][r] = sv;
            tmax = fmaxf(tmax, sv);
          }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[j], tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run[j] - m_new);
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
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
#pragma unroll
      for (int i = 0; i < DB16; ++i) o[j][i] *= alpha;
      // ---- O^T += V^T P^T over the two 32-key halves ----
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[r] = (__bf16)st[2 * kk][r];
          pf[r + 4] = (__bf16)st[2 * kk + 1][r];
        }
#pragma unroll
        for (int i = 0; i < DB16; ++i)
          o[j][i] = mfma16x16x32(tl.v[(4 * kk + g) * HD + 16 * i + qi], pf, o[j][i]);
      }
    }
  };

  // tile it sits in LDS buffer it & 1; with PF = 2 the registers hold the
  // loads of tiles it + 1 and it + 2, so each tile's loads stay in flight
  // for two tiles' work
  store_tile(ra, 0, split, hi);
  __syncthreads();
  if constexpr (PF == 2) {
    for (int it = 0; it < my_tiles; it += 2) {
      const int t = split + it * S;
      if (it + 2 < my_tiles) load_tile(ra, t + 2 * S);
      use_tile(0, t);
      if (it + 1 < my_tiles) store_tile(rb, 1, t + S, hi);
      __syncthreads();
      if (it + 1 >= my_tiles) break;
      if (it + 3 < my_tiles) load_tile(rb, t + 3 * S);
      use_tile(1, t + S);
      if (it + 2 < my_tiles) store_tile(ra, 0, t + 2 * S, hi);
      __syncthreads();
    }
  } else {
    for (int it = 0; it < my_tiles; ++it) {
      const int t = split + it * S;
      if (it + 1 < my_tiles) load_tile(ra, t + S);
      use_tile(it & 1, t);
      if (it + 1 < my_tiles) store_tile(ra, (it + 1) & 1, t + S, hi);
      __syncthreads();
    }
  }

  // ---- output: lane holds dims 16 * i + 4 * g .. +3 of query 16 * qb + qi
  auto out_ptr = [&](int node, int c) -> u16* {
    const int m = b * T + node, col = h * HD + c;
    return a.packed ? a.out + packed_index(m, col, d) : a.out + (size_t)m * d + col;
  };
  if (S == 1) {
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int node = (wave * QPW + j) * 16 + qi;
      if (j >= qb_live || node >= T) continue;
      const float inv = 1.f / l_run[j];
#pragma unroll
      for (int i = 0; i < DB16; ++i) {
        const uint32_t lo = (uint32_t)f32_to_bf16(o[j][i][0] * inv) |
                            ((uint32_t)f32_to_bf16(o[j][i][1] * inv) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16(o[j][i][2] * inv) |
                             ((uint32_t)f32_to_bf16(o[j][i][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out_ptr(node, 16 * i + 4 * g)) = uint2{lo, hi2};
      }
    }
    return;
  }

  // ---- S > 1: this split's partial state in fragment order: the 1 KiB of
  // (query block, 16-dim block) is the 64 lanes' 16-byte pieces in lane
  // order, so every store writes whole lines.  The merge launch that follows
  // reads them (the launch boundary makes them visible on every XCD).
  const int QB = (T + 15) >> 4;
  const size_t pslot = (size_t)pair * a.S + split;
  f32x4* po = reinterpret_cast<f32x4*>(a.part_o + pslot * QB * 16 * HD);
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qb = wave * QPW + j;
    const int node = qb * 16 + qi;
    if (j >= qb_live) continue;                   // wave-uniform
#pragma unroll
    for (int i = 0; i < DB16; ++i) po[(qb * DB16 + i) * 64 + lane] = o[j][i];
    if (g == 0 && node < T) a.part_ml[pslot * T + node] = make_float2(m_run[j], l_run[j]);
  }
}

// The S partial states of each (sequence, head) pair merged into the output:
// per query, split s weighs 2^(m_s - M) with M the largest m_s (splits in
// order, deterministic).  One thread per 16-byte piece of the fragment order
// (4 output dims of one query); every split's loads are issued before any
// is used.  The split count follows n exactly as the attention launch's.
template <int HD>
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnArgs a) {
  constexpr int DB16 = HD / 16;
  constexpr int SMAX = 16;
  const int QB = (a.T + 15) >> 4;
  const int FR = QB * DB16 * 64;               // pieces of one split's state
  const int per_pair = (FR + 255) >> 8;        // workgroups per pair
  const int pair = blockIdx.x / per_pair;
  const int e = (blockIdx.x % per_pair) * 256 + threadIdx.x;
  if (pair >= a.B * a.H || e >= FR) return;
  const int b = pair / a.H, h = pair % a.H;
  const int T = a.T;
  const int n_raw = a.n_prefix[b];
  const int ln = e & 63, fb = e >> 6;
  const int qq = (fb / DB16) * 16 + (ln & 15), c4 = (fb % DB16) * 16 + 4 * (ln >> 4);
  const f32x4* po = reinterpret_cast<const f32x4*>(a.part_o) + (size_t)pair * a.S * FR + e;
  const float2* pm = a.part_ml + (size_t)pair * a.S * T + min(qq, T - 1);
  // all splits' pieces requested before n is known (the unused ones are
  // never read for the result)
  f32x4 x[SMAX];
  float2 ml[SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    if (s < a.S) {
      x[s] = po[(size_t)s * FR];
      ml[s] = pm[(size_t)s * T];
    }
  }
  const int n = min(max(n_raw, 0), a.cap - T);
  const int ntiles = (n + T + 63) >> 6;
  const int per = (ntiles + a.S - 1) / a.S;
  const int S = (ntiles + per - 1) / per;
  if (S == 1 || qq >= T) return;               // one split wrote the output itself
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < SMAX; ++s)
    if (s < S) M = fmaxf(M, ml[s].x);
  float den = 0.f, val[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    if (s >= S || ml[s].x == -INFINITY) continue;   // no visible key in the split
    const float f = exp2f(ml[s].x - M);
    den += f * ml[s].y;
#pragma unroll
    for (int u = 0; u < 4; ++u) val[u] += f * x[s][u];
  }
  const float inv = 1.f / den;
  const uint32_t lo = (uint32_t)f32_to_bf16(val[0] * inv) | ((uint32_t)f32_to_bf16(val[1] * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(val[2] * inv) | ((uint32_t)f32_to_bf16(val[3] * inv) << 16);
  const int d = a.H * HD, m = b * T + qq, col = h * HD + c4;
  u16* dst = a.packed ? a.out + packed_index(m, col, d) : a.out + (size_t)m * d + col;
  *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
}

// ---------------------------------------------------------------------------
// Per-query-block variant, for short caches: a workgroup owns 16 queries of
// one (sequence, head); its NW waves split the key slots 0 .. n+T-1 in
// 64-key tiles (tile t to wave t mod NW), each wave holding its tile's K and
// V in registers, so every K/V byte is read once per query block (the
// pair's query blocks share one XCD, whose L2 serves the repeats) and no
// partial state leaves the workgroup: the waves' (m, l, o) are merged in
// LDS in wave order.  Up to a few thousand keys this beats splitting the key
// range, whose merge costs a launch.
// ---------------------------------------------------------------------------
template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 2) void tree_attention_qb_kernel(
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
      // lane group g's keys: bits 8g .. 8g+7 (kk = 0) and 32+8g .. (kk = 1)
      const uint64_t vis = slot_visibility(am[0], am[1], am[2], am[3], s0, n, hi);
      const uint32_t vbits[2] = {(uint32_t)(vis >> (8 * g)) & 0xffu, (uint32_t)(vis >> (32 + 8 * g)) & 0xffu};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (vbits[kb >> 1] >> ((kb & 1) * 4 + r)) & 1u;
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
      // every slot below hi holds written K/V (the prefix and this tree):
      // only a tile that runs past n + T has values to clip
      if (s0 + 64 <= hi) {
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
// (212 registers a lane; the kernel's launch bounds ask for two waves per
// SIMD, which keeps the 4-wave variant under 256), so more K/V tiles are in
// flight per unit.
template <int HD>
static void launch_attention_qb(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                                const uint64_t* anc, int B, int T, int H, int cap, int mw,
                                u16* out, int packed, hipStream_t s) {
  const int QB = (T + 15) / 16, pairs = B * H;
  const dim3 grid(8 * ((pairs + 7) / 8) * QB);
  if ((size_t)pairs * QB > 512)
    hipLaunchKernelGGL((tree_attention_qb_kernel<HD, 4>), grid, dim3(256), 0, s, q, kc, vc, n_prefix,
                       anc, B, T, H, cap, mw, out, packed);
  else
    hipLaunchKernelGGL((tree_attention_qb_kernel<HD, 8>), grid, dim3(512), 0, s, q, kc, vc, n_prefix,
                       anc, B, T, H, cap, mw, out, packed);
}

// Key splits per (sequence, head): about two workgroups per compute unit
// for trees of up to 64 nodes (one for the wider query blocks of larger
// trees), at most 16 (the partial states grow with S); the kernel uses fewer
// when the tiles at the current n do not need them.
int attention_splits(int B, int H, int T) {
  const int pairs = B * H;
  return std::max(1, std::min(16, (T <= 64 ? 512 : 256) / std::max(pairs, 1)));
}

template <int HD, int QPW>
static void launch_attention_q(const AttnArgs& a, hipStream_t s) {
  const int pairs8 = (a.B * a.H + 7) / 8 * 8;   // whole groups of 8 pairs (one per XCD)
  hipLaunchKernelGGL((tree_attention_kernel<HD, QPW>), dim3(pairs8 * a.S), dim3(256), 0, s, a);
  if (a.S > 1) {
    const int FR = (a.T + 15) / 16 * (HD / 16) * 64;
    hipLaunchKernelGGL((attention_merge_kernel<HD>), dim3(a.B * a.H * ((FR + 255) / 256)),
                       dim3(256), 0, s, a);
  }
}

template <int HD>
static void launch_attention_hd(const AttnArgs& a, hipStream_t s) {
  const int qb = (a.T + 15) / 16;              // 16-query blocks, four waves
  if (qb <= 4) launch_attention_q<HD, 1>(a, s);
  else if (qb <= 8) launch_attention_q<HD, 2>(a, s);
  else launch_attention_q<HD, 4>(a, s);
}

bool attention_uses_splits(int B, int H, int T, int cap) {
  // Per query block while the cache holds at most 2048 slots or that grid
  // already gives every compute unit a workgroup; split keys for long caches
  // under a small grid.  Measured per launch: 8.7 against 14 us at the 7B
  // shape with n = 512, 34 against 55 us for 256-node trees at the 13B shape
  // (640 workgroups), 57 against 86 us for the 33B batch of four (832); the
  // split kernel wins for 32 heads of a 64-node tree at n = 4096.
  return cap > 2048 && B * H * ((T + 15) / 16) < 256;
}

hipError_t launch_attention(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                            const uint64_t* anc, int B, int T, int H, int hd, int cap, int mw,
                            u16* out, int packed, float* part_o, float2* part_ml, hipStream_t s) {
  if (T < 1 || T > 256) return hipErrorInvalidValue;
  if (!attention_uses_splits(B, H, T, cap)) {
    switch (hd) {
      case 16: launch_attention_qb<16>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
      case 32: launch_attention_qb<32>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
      case 64: launch_attention_qb<64>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
      case 128: launch_attention_qb<128>(q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  AttnArgs a{q, kc, vc, n_prefix, anc, B, T, H, cap, mw, out, packed, attention_splits(B, H, T),
             part_o, part_ml};
  if (a.S > 1 && (!part_o || !part_ml)) return hipErrorInvalidValue;
  switch (hd) {
    case 16: launch_attention_hd<16>(a, s); break;
    case 32: launch_attention_hd<32>(a, s); break;
    case 64: launch_attention_hd<64>(a, s); break;
    case 128: launch_attention_hd<128>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mvk
