// Skinny bf16 GEMM for the tree-verify forward: Y[M][N] = A[M][K] * W[N][K]^T
// with M = batch x tree nodes (16..1024), N and K the model's widths.
//
// At M ~ 64 every weight byte is used 64 times, so the kernel is bound by
// streaming W from HBM once; the MFMA units (v_mfma_f32_16x16x32_bf16) only
// need to keep up.  Layout of the work (measured on MI355X):
//  * Weights are fragment-packed k-block-major ([K/32][N/16][64 lanes][8]):
//    the 1 KiB operand blocks of all columns of one 32-wide k-block are
//    adjacent, so the grid sweeps a dense window of memory.
//  * Each wave owns NBW 16-column blocks over the workgroup's k-range and
//    keeps a register ring of KC k-blocks of them in flight (consumed, then
//    refilled in place; scheduling barriers keep the refill after the MFMAs
//    that read the stage, so no register copies undo the prefetch).
//  * The activation operand is staged once per workgroup in LDS in chunks of
//    KCA k-blocks, double-buffered, and shared by the W waves; k-blocks past
//    the range are staged as zeros, so the main loop has no branches and the
//    compiler's wait counts stay partial.  The unsplit gate/up GEMM takes two
//    ring lengths per chunk (half the barriers), the split GEMMs, whose
//    k-ranges are short, one, and the 128- and 256-row tiles 32 KiB chunks
//    inside a ring length.  In 64-row tiles the next step's fragments are
//    read from LDS before the current step's MFMAs.
//  * 128- and 256-row tiles give each wave one column block (gate/up: gate
//    and up blocks in different waves; QKV: RoPE partners in neighbouring
//    waves, exchanged through LDS), which leaves registers for an 8-deep ring.
//    QKV tiles of up to 64 rows do the same with 4 waves (64 columns): their
//    count covers the chip without splitting K, so no partials are exchanged.
//  * K is split over `splits` workgroups when the column tiles alone cannot
//    fill the chip.  Each split writes its partial tile with write-through
//    (system-scope) stores, waits for them, and bumps the tile's arrival
//    counter; the last workgroup to arrive reads all partials with batched
//    cache-bypassing loads and sums them in split order (a deterministic
//    result, no separate reduce launch, no L2-wide invalidation).
// RMSNorm is folded in: the operand of a normalised GEMM is bf16(x * gain)
// and the per-row factor 1/sqrt(mean(x^2) + 1e-5) is applied to the
// accumulators, from row sums of squares that the producing GEMM wrote per
// column tile (requested with the first weight chunk, summed after the main
// loop).
// Epilogues:
//   STORE   out = y                          (LM head logits)
//   ADD     x += y (residual stream: O-proj, down); optionally the next
//           norm's operand bf16(x * gain) and the rows' sums of squares
//   SWIGLU  h = SiLU(g) * u -> bf16 (gate block j and up block j in one
//           wave, or in waves j and j + W/2)
//   QKV     RoPE on q, k at each row's position; q -> bf16 rows; k, v ->
//           KV cache slot n + node index
#include "common.hpp"

namespace mvk {

// Logical output feature of packed weight row p of the fused QKV matrix.
// q/k rows are permuted (when the head is wider than 16) so that each pair
// of 16-row blocks holds 16 first-half dims of one head and their RoPE
// partners (dim + hd/2), which then meet in the same lane of one wave; v rows
// are never permuted.
__host__ __device__ __forceinline__ int qkv_feature(int p, int d, int hd) {
  if (hd < 32 || p >= 2 * d) return p;
  const int h = p / hd, e = p % hd, j = e / 32, ee = e % 32;
  return h * hd + (ee < 16 ? j * 16 + ee : hd / 2 + j * 16 + (ee - 16));
}

// Split-K partial exchange between workgroups that may sit on different
// XCDs (separate L2s): 16-byte buffer stores and loads with the system-scope
// cache policy (sc0 sc1: stores written through to memory, loads bypassing
// the caches, so no L2-wide invalidation is needed).  They are ordinary
// compiler-tracked memory operations, so the loads of a batch are issued
// together and waited for once.  Raw buffer accesses are range-checked by
// the hardware: an offset past the resource's size reads zeros, which the
// batches use for splits that do not exist.
#define MV_CPOL_SYS 17              /* sc0 | sc1 */
#define MV_BUF_DWORD3 0x00020000    /* raw (untyped) buffer resource */
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define MV_BUF_NONE 0x7ffffff0      /* an offset past any partial buffer */

// A float moved between lanes of a 16-lane DPP row (VALU lane moves, no LDS
// round trips): quad_perm 0xB1 and 0x4E swap lanes xor 1 and xor 2,
// row_half_mirror (0x141) and row_mirror (0x140) reverse 8 and 16 lanes.
#define MV_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false))

// One step of a (value, column) maximum over a DPP row: larger value, then
// lower column.
template <int CTRL>
__device__ __forceinline__ void row16_best(float& bv, int& bi) {
  const float ov = MV_DPP(bv, CTRL);
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// KC: depth of the weight ring in k-blocks (per wave, KC * NBW KiB in
// flight).  KCA: k-blocks per activation chunk (KCA * MB KiB per LDS
// buffer, one barrier per chunk).  Up to 64 rows: an 8-deep ring, with two
// ring lengths per chunk for the unsplit gate/up GEMM and one otherwise.
// 128- and 256-row tiles with one column block per wave keep the 8-deep ring
// and stage 32 KiB chunks (a half or a quarter of a ring length); with two
// blocks per wave their accumulators leave registers for a 4- or 2-deep ring
// only, one ring length per chunk.
template <int MB, int NBW, int EPI>
struct GemmShape {
  static constexpr int KC = MB <= 4 || NBW == 1 ? 8 : 32 / MB;
  static constexpr int KCA = MB <= 4 ? (EPI == EPI_SWIGLU ? 2 * KC : KC) : 32 / MB;
};

int gemm_kc(int MB) { return MB <= 4 ? 8 : 32 / MB; }   // k-blocks per activation chunk

// Reads the cached prefix K and V of one layer (slots 0 .. n-1 of every
// (sequence, head) block: the first ceil(n/32) K groups and ceil(n/8) V runs,
// contiguous at the start of the block) and discards the values.  Workgroups
// appended to the QKV launch, on compute units its tiles leave idle, do this
// so that the attention launch that follows finds the prefix in the
// memory-side cache instead of waiting on HBM.  Each reads at most budget16
// 16-byte pieces, so that it ends well before the tiles do (long prefixes
// are then read in part).
__device__ __forceinline__ void prefetch_prefix_kv(const QkvArgs& q, int p, int P, int budget16) {
  uint32_t sink = 0;
  const int ranges = 2 * q.B * q.H;
  for (int r = p; r < ranges && budget16 > 0; r += P) {
    const int pair = r >> 1, b = pair / q.H;
    const int n = min(max(q.n_prefix[b], 0), q.cap - q.T);
    const int slots = (r & 1) ? ((n + 7) & ~7) : ((n + 31) & ~31);
    const uint4* src = reinterpret_cast<const uint4*>(((r & 1) ? q.vcache : q.kcache) +
                                                      (size_t)pair * q.cap * q.hd);
    const int n16 = min(slots * q.hd / 8, budget16);  // 16-byte pieces (within the budget)
    budget16 -= n16;
    int i = threadIdx.x;
    for (; i + 7 * (int)blockDim.x < n16; i += 8 * blockDim.x) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[i + u * blockDim.x];
#pragma unroll
      for (int u = 0; u < 8; ++u) sink ^= v[u].x ^ v[u].w;
    }
    for (; i < n16; i += blockDim.x) sink ^= src[i].x;
  }
  asm volatile("" ::"v"(sink));
}

template <int MB, int W, int NBW, int EPI>
__global__ __launch_bounds__(W * 64) void gemm_kernel(GemmArgs g) {
  constexpr int KC = GemmShape<MB, NBW, EPI>::KC;     // weight ring depth (k-blocks)
  constexpr int KCA = GemmShape<MB, NBW, EPI>::KCA;   // k-blocks per activation chunk
  // the main loop runs in segments of SG k-blocks; each stages SG k-blocks of
  // the next activation chunk (PARTS segments fill one chunk)
  constexpr int SG = KCA < KC ? KCA : KC;
  constexpr int UO = KCA < KC ? KC : KCA;      // k-blocks per outer iteration
  constexpr int NSEG = UO / SG;
  constexpr int PARTS = KCA / SG;
  constexpr int APS = SG * MB;                 // 1 KiB activation pieces per segment
  constexpr int APC = KCA * MB;                // ... per chunk
  constexpr int AI = (APS + W - 1) / W;        // pieces staged per thread per segment
  static_assert(PARTS <= 2 && (KCA < KC ? KC % KCA == 0 : KCA % KC == 0), "chunk and ring align");
  constexpr int TR = MB * 16;                  // rows of a tile
  __shared__ bf16x8 As[2][APC][64];            // [buf][kl * MB + rb][lane]
  __shared__ float rs_s[TR];
  __shared__ int s_last;
  __shared__ int s_slot0[MV_MAX_BATCH];        // QKV: cache slot of each sequence's node 0

  // SwiGLU with one block per wave: waves 0 .. FW-1 take gate blocks, waves
  // FW .. W-1 the up blocks of the same features (FW feature blocks a tile)
  constexpr bool SPLIT_GU = EPI == EPI_SWIGLU && NBW == 1;
  constexpr int FW = SPLIT_GU ? W / 2 : W;
  constexpr int PER_TILE = EPI == EPI_SWIGLU ? FW : W * NBW;  // 16-column blocks per tile
  const int NT = (g.N / 16 + PER_TILE - 1) / PER_TILE;          // column tiles
  if constexpr (EPI == EPI_QKV) {
    if ((int)blockIdx.x >= NT) {               // appended prefetch workgroups
      prefetch_prefix_kv(g.qkv, ((int)blockIdx.x - NT) * gridDim.y + blockIdx.y,
                         ((int)gridDim.x - NT) * gridDim.y, g.pf_budget16);
      return;
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
  const int KB = g.K >> 5;
  const int lo = (int)((long long)KB * split / g.splits);
  const int hi = (int)((long long)KB * (split + 1) / g.splits);
  const int nouter = (hi - lo + UO - 1) / UO;
  const int NBtot = g.N >> 4;                  // 16-column blocks of W (and of W2)
  const int MBtot = g.Mp >> 4;

  // this wave's column blocks (waves past the last block compute on a
  // clamped block and store nothing)
  const int wb = SPLIT_GU ? nt * FW + wave % FW : nt * W + wave;
  const int first_blk = EPI == EPI_SWIGLU ? wb : wb * NBW;
  const int blk_cnt = EPI == EPI_SWIGLU ? 1 : NBW;
  const bool active = first_blk + blk_cnt <= NBtot;
  const int cb = min(first_blk, NBtot - blk_cnt);
  const bf16x8* Bp[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (SPLIT_GU)
      Bp[nb] = reinterpret_cast<const bf16x8*>(wave < FW ? g.W : g.W2) + (size_t)cb * 64 + lane;
    else if (EPI == EPI_SWIGLU)
      Bp[nb] = reinterpret_cast<const bf16x8*>(nb == 0 ? g.W : g.W2) + (size_t)cb * 64 + lane;
    else
      Bp[nb] = reinterpret_cast<const bf16x8*>(g.W) + (size_t)(cb + nb) * 64 + lane;
  }
  const bf16x8* Ap = reinterpret_cast<const bf16x8*>(g.A) + lane;

  // per-row normalisation factors of this tile.  Row m's partial sums of
  // squares are contiguous.  Usually LPR adjacent lanes share a row: their
  // 16-byte loads go out right after the first weight chunk's, and the sums
  // are formed after the main loop (they only scale the accumulators), so no
  // wave waits on them before streaming.  Otherwise (few lanes per row, or
  // many tiles) one lane per row sums them here, before the main loop.
  constexpr int SS_Q = 4;                              // f32x4 per lane
  // lanes per row: a power of two up to one DPP row (16), as the reduction
  // below assumes; rows per pass = W * 64 / LPR >= TR
  constexpr int LPR_MAX = TR <= W * 64 ? (W * 64) / TR : 0;
  constexpr int LPR = LPR_MAX >= 16 ? 16 : LPR_MAX >= 8 ? 8 : LPR_MAX >= 4 ? 4 : LPR_MAX >= 2 ? 2 : LPR_MAX;
  const int ss_n4 = g.ss_tiles >> 2;
  const bool ss_late = g.ss != nullptr && LPR > 0 && ss_n4 <= LPR * SS_Q;
  if (g.ss && !ss_late) {
    for (int r = threadIdx.x; r < TR; r += W * 64) {
      const int m = mt * TR + r;
      float s = 0.f;
      if (m < g.M) {
        const float* row = g.ss + (size_t)m * g.ss_ld;
        const f32x4* p4 = reinterpret_cast<const f32x4*>(row);
        int t = 0;
        for (; t + 8 <= ss_n4; t += 8) {
          f32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = p4[t + u];
#pragma unroll
          for (int u = 0; u < 8; ++u) s = s + v[u][0] + v[u][1] + v[u][2] + v[u][3];
        }
        for (; t < ss_n4; ++t) {
          const f32x4 v = p4[t];
          s = s + v[0] + v[1] + v[2] + v[3];
        }
        for (int e = ss_n4 * 4; e < g.ss_tiles; ++e) s += row[e];
      }
      rs_s[r] = 1.0f / sqrtf(s / (float)g.K + 1e-5f);
    }
  }

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int rb = 0; rb < MB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // part h (SG k-blocks) of activation chunk c
  bf16x8 ar[AI];
  auto loadA = [&](bf16x8 (&dst)[AI], int c, int h) {
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      // waves past the segment's pieces (when W does not divide them) repeat the last
      const int piece = APS % W == 0 ? i * W + wave : min(i * W + wave, APS - 1);
      const int kl = h * SG + piece / MB, rb = piece % MB;
      const int k = min(lo + c * KCA + kl, hi - 1);
      const int rbg = min(mt * MB + rb, MBtot - 1);
      dst[i] = Ap[((size_t)rbg * KB + k) * 64];
    }
  };
  auto storeA = [&](const bf16x8 (&src)[AI], int buf, int c, int h) {   // past the range: zeros
#pragma unroll
    for (int i = 0; i < AI; ++i) {
      const int piece = i * W + wave;
      const int kl = h * SG + piece / MB;
      if (APS % W == 0 || piece < APS)
        As[buf][h * APS + piece][lane] = (lo + c * KCA + kl < hi) ? src[i] : bf16x8{};
    }
  };
  bf16x8 br[KC][NBW];
  auto loadB = [&](int s, int kb) {
    const int k = min(kb, hi - 1);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) br[s][nb] = Bp[nb][(size_t)k * NBtot * 64];
  };

  // QKV: prefix lengths (loaded first, stored to LDS once the operand loads
  // are out; n + T <= cap is the caller's contract, clamping keeps every
  // store in bounds)
  int nraw = 0;
  if (EPI == EPI_QKV && threadIdx.x < g.qkv.B) nraw = g.qkv.n_prefix[threadIdx.x];
  if constexpr (PARTS == 2) {
    bf16x8 a0[AI];
    loadA(a0, 0, 0);
#pragma unroll
    for (int s = 0; s < KC; ++s) loadB(s, lo + s);
    loadA(ar, 0, 1);
    storeA(a0, 0, 0, 0);
  } else {
    loadA(ar, 0, 0);
#pragma unroll
    for (int s = 0; s < KC; ++s) loadB(s, lo + s);
  }
  f32x4 ssv[SS_Q];
  float ss_rest = 0.f;
  if (ss_late) {
    // lanes past the tile's rows (when the lane count caps LPR) load nothing
    const int r = (int)threadIdx.x / max(LPR, 1), j = (int)threadIdx.x % max(LPR, 1);
    const float* row = g.ss + (size_t)min(mt * TR + min(r, TR - 1), g.M - 1) * g.ss_ld;
#pragma unroll
    for (int q = 0; q < SS_Q; ++q) {
      const int t = j + q * LPR;
      ssv[q] = (r < TR && t < ss_n4) ? reinterpret_cast<const f32x4*>(row)[t] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int e = ss_n4 * 4 + j; r < TR && e < g.ss_tiles; e += LPR) ss_rest += row[e];
  }
  storeA(ar, 0, 0, PARTS - 1);
  if (EPI == EPI_QKV && threadIdx.x < g.qkv.B)
    s_slot0[threadIdx.x] = min(max(nraw, 0), g.qkv.cap - g.qkv.T);
  __syncthreads();
  // the weight k-block consumed at (o, sg, kk) is lo + o*UO + sg*SG + kk; its
  // ring stage is refilled with the k-block KC further on
  for (int o = 0; o < nouter; ++o) {
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      const int c = PARTS == 1 ? o * NSEG + sg : o;        // chunk being read
      const int h = PARTS == 1 ? 0 : sg;                   // part staged for chunk c + 1
      const int buf = c & 1;
      loadA(ar, c + 1, h);
      // the next step's activation fragments are read from LDS before this
      // step's MFMAs, so their latency hides behind them (tiles up to 64
      // rows but gate/up, where it measured slower; the wider tiles have no
      // registers to spare)
      constexpr bool PIPE = MB <= 4 && EPI != EPI_SWIGLU;
      const int apos0 = PARTS == 1 ? 0 : sg * SG;
      bf16x8 a[MB];
      if constexpr (PIPE) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) a[rb] = As[buf][apos0 * MB + rb][lane];
      }
#pragma unroll
      for (int kk = 0; kk < SG; ++kk) {
        const int stage = PARTS == 1 ? sg * SG + kk : kk;
        const int apos = apos0 + kk;
        bf16x8 an[MB];
        if constexpr (PIPE) {
          if (kk + 1 < SG) {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) an[rb] = As[buf][(apos + 1) * MB + rb][lane];
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int rb = 0; rb < MB; ++rb) a[rb] = As[buf][apos * MB + rb][lane];
        }
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc[rb][nb] = mfma16x16x32(a[rb], br[stage][nb], acc[rb][nb]);
        __builtin_amdgcn_sched_barrier(0);
        loadB(stage, lo + o * UO + sg * SG + kk + KC);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PIPE) {
          if (kk + 1 < SG) {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb) a[rb] = an[rb];
          }
        }
      }
      storeA(ar, buf ^ 1, c + 1, h);
      if (PARTS == 1 || sg == NSEG - 1) __syncthreads();
    }
  }

  if (ss_late) {      // the row's sum: each lane's quads in order, then over its LPR lanes
    float sm = ss_rest;
#pragma unroll
    for (int q = 0; q < SS_Q; ++q) sm = sm + ssv[q][0] + ssv[q][1] + ssv[q][2] + ssv[q][3];
    if constexpr (LPR >= 2) sm += MV_DPP(sm, 0xB1);     // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) sm += MV_DPP(sm, 0x4E);     // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) sm += MV_DPP(sm, 0x141);    // row_half_mirror
    if constexpr (LPR >= 16) sm += MV_DPP(sm, 0x140);   // row_mirror
    static_assert(LPR <= 16, "a row's lanes lie inside one DPP row");
    const int r = (int)threadIdx.x / max(LPR, 1);
    if ((int)threadIdx.x % max(LPR, 1) == 0 && r < TR) rs_s[r] = 1.0f / sqrtf(sm / (float)g.K + 1e-5f);
    __syncthreads();
  }

  // ---- the epilogue's own memory operands, loaded before the split-K
  // exchange so that their latency overlaps it (rows past M and inactive
  // waves read clamped, valid addresses; the values are then unused)
  const int col = lane & 15;
  const int row0 = mt * TR + 4 * (lane >> 4);
  // ADD: the thread's 16-byte pieces of the tile (8 columns of one row):
  // residual x and the next norm's gains
  constexpr int ATC = W * NBW * 16;           // columns of an ADD tile
  constexpr int APR = ATC / 8;                // pieces per row (8 or 16)
  constexpr int ANP = (TR * APR + W * 64 - 1) / (W * 64);
  f32x4 xr[ANP][2];
  uint4 gr[ANP];
  float2 cs[MB][4];                           // QKV: RoPE (cos, sin) per row
  // QKV: the lane's two blocks are packed rows p0 (block 0) and p0 + 16
  // (block 1); with heads wider than 16 they hold dims i and i + hd/2 of one
  // head (RoPE partners, same (cos, sin)); with 16-wide heads each block is
  // one head and partners sit 8 lanes apart
  const int p0 = cb * 16 + col;
  const bool rot = EPI == EPI_QKV && p0 < 2 * g.qkv.d;
  const bool wide = g.qkv.hd >= 32;
  const int f0 = (rot && wide) ? qkv_feature(p0, g.qkv.d, g.qkv.hd) : p0;
  const int half = g.qkv.hd >> 1;
  if constexpr (EPI == EPI_ADD) {
#pragma unroll
    for (int i = 0; i < ANP; ++i) {
      const int p = i * W * 64 + threadIdx.x;
      const int m = min(mt * TR + p / APR, g.M - 1);
      const int c = min(nt * ATC + 8 * (p % APR), g.N - 8);
      const f32x4* xp = reinterpret_cast<const f32x4*>(g.out_f32 + (size_t)m * g.N + c);
      xr[i][0] = xp[0];
      xr[i][1] = xp[1];
      gr[i] = g.next_gain ? *reinterpret_cast<const uint4*>(g.next_gain + c) : uint4{0, 0, 0, 0};
    }
  }
  // RoPE (cos, sin) of the lane's rows; 256-row tiles with one block per
  // wave have no registers to hold them across the split-K exchange and load
  // them after it
  auto load_cs = [&]() {
    const int ci = (f0 % g.qkv.d) % g.qkv.hd % half;  // RoPE frequency index of both blocks
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = min(row0 + rb * 16 + r, g.M - 1);
        cs[rb][r] = rot ? g.qkv.rope[(size_t)m * half + ci] : make_float2(1.f, 0.f);
      }
  };
  constexpr bool CS_LATE = EPI == EPI_QKV && NBW == 1 && MB == 16;
  if constexpr (EPI == EPI_QKV && !CS_LATE) load_cs();

  // ---- split-K: the last workgroup of the tile sums the splits in order
  if (g.splits > 1) {
    constexpr int WQ = MB * NBW;               // f32x4 items per lane of one wave
    constexpr int SB = WQ >= 16 ? 1 : 16 / WQ; // splits loaded per batch
    const int tile = mt * NT + nt;
    const int per_split = W * WQ * 256 * 4;    // bytes of one split's tile
    const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
        g.partial + (size_t)tile * g.splits * (per_split / 4), (short)0, g.splits * per_split,
        MV_BUF_DWORD3);
    const int lane_off = (wave * WQ * 256 + lane * 4) * 4;
#pragma unroll
    for (int q = 0; q < WQ; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(acc[q / NBW][q % NBW], part,
                                             split * per_split + lane_off + q * 1024, 0, MV_CPOL_SYS);
    __builtin_amdgcn_s_waitcnt(0);           // this thread's write-through stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(g.counters + tile, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == g.splits - 1;
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < g.splits; s0 += SB) {
      f32x4 v[SB][WQ];
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int base = s0 + s < g.splits ? (s0 + s) * per_split + lane_off : MV_BUF_NONE;
#pragma unroll
        for (int q = 0; q < WQ; ++q)
          v[s][q] = __builtin_amdgcn_raw_buffer_load_b128(
              part, base == MV_BUF_NONE ? MV_BUF_NONE : base + q * 1024, 0, MV_CPOL_SYS);
      }
#pragma unroll
      for (int s = 0; s < SB; ++s)
#pragma unroll
        for (int q = 0; q < WQ; ++q) acc[q / NBW][q % NBW] += v[s][q];
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(g.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogues: lane holds rows rb*16 + 4*(lane/16) + r, column lane%16 of each block
  if (g.ss) {
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = rs_s[rb * 16 + 4 * (lane >> 4) + r];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[rb][nb][r] *= f;
      }
  }
  if (EPI == EPI_STORE) {
    if (g.status) {      // non-finite logits of real rows are flagged (one atomic a wave)
      bool bad = false;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            bad |= active && row0 + rb * 16 + r < g.M && !__builtin_isfinite(acc[rb][nb][r]);
      if (__ballot(bad) != 0ull && lane == 0) atomicOr(g.status, MV_STATUS_NONFINITE);
    }
    // each row's argmax over this tile's columns; ties go to the lower
    // column, NaNs never win.  Tiles staged in LDS: W adjacent lanes take one
    // row, lane w scanning wave w's 16 columns (four 16-byte reads), then a
    // 3-step shuffle over the W lanes.  Otherwise the lanes of a 16-lane row
    // group reduce their registers (DPP), then the waves (LDS).
    constexpr bool STAGED = NBW == 1 && W * TR * 16 * 4 <= (int)sizeof(As);
    auto publish = [&](int m, float bv, int bi) {
      // the max only grows: a key at or below the stored one cannot win, so
      // most tiles skip the atomic (all column tiles share each row's key)
      const unsigned long long key = argmax_key(bv, bi);
      if (key > __hip_atomic_load(g.amax_key + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_fetch_max(g.amax_key + m, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    if constexpr (STAGED) {
      // staged per wave in the operand LDS, then written as 16-byte pieces
      // (4 columns of one row)
      float* stg_all = reinterpret_cast<float*>(&As[0][0][0]);
      float* stg = stg_all + wave * TR * 16;
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[(rb * 16 + 4 * (lane >> 4) + r) * 16 + col] = acc[rb][0][r];
      __syncthreads();
      if (active) {
#pragma unroll
        for (int p = lane; p < TR * 4; p += 64) {
          const int rl = p >> 2, m = mt * TR + rl;
          if (m < g.M)
            *reinterpret_cast<f32x4*>(g.out_f32 + (size_t)m * g.N + first_blk * 16 + 4 * (p & 3)) =
                *reinterpret_cast<const f32x4*>(stg + rl * 16 + 4 * (p & 3));
        }
      }
      if (g.amax_key) {
        static_assert((TR * W) % 64 == 0 && 64 % W == 0, "whole waves of W-lane row groups");
        for (int e = threadIdx.x; e < TR * W; e += W * 64) {      // uniform trip count
          const int rl = e / W, w = e % W;
          const int blk = nt * W + w;                 // column block of wave w
          float bv = -INFINITY;
          int bi = 0x7fffffff;
          if (blk < NBtot) {
            const f32x4* src = reinterpret_cast<const f32x4*>(stg_all + (w * TR + rl) * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 v = src[q];
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int i = blk * 16 + 4 * q + c;
                if (v[c] > bv || (v[c] == bv && i < bi)) { bv = v[c]; bi = i; }
              }
            }
          }
#pragma unroll
          for (int o = 1; o < W; o <<= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
          }
          const int m = mt * TR + rl;
          if (w == 0 && m < g.M) publish(m, bv, bi);
        }
      }
    } else {
      __shared__ float s_av[W][TR];
      __shared__ int s_ai[W][TR];
      if (g.amax_key) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
              const float v = active ? acc[rb][nb][r] : -INFINITY;
              const int i = (first_blk + nb) * 16 + col;
              if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
            }
            row16_best<0xB1>(bv, bi);     // quad swaps, half-row and row mirrors
            row16_best<0x4E>(bv, bi);
            row16_best<0x141>(bv, bi);
            row16_best<0x140>(bv, bi);
            if (col == 0) {
              s_av[wave][rb * 16 + 4 * (lane >> 4) + r] = bv;
              s_ai[wave][rb * 16 + 4 * (lane >> 4) + r] = bi;
            }
          }
      }
      if (active) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int m = row0 + rb * 16 + r;
              if (m < g.M) g.out_f32[(size_t)m * g.N + (first_blk + nb) * 16 + col] = acc[rb][nb][r];
            }
      }
      if (g.amax_key) {
        __syncthreads();                  // uniform: the waves' row maxima are in LDS
        for (int r = threadIdx.x; r < TR; r += W * 64) {
          const int m = mt * TR + r;
          if (m >= g.M) continue;
          float bv = s_av[0][r];
          int bi = s_ai[0][r];
#pragma unroll
          for (int w = 1; w < W; ++w)
            if (s_av[w][r] > bv || (s_av[w][r] == bv && s_ai[w][r] < bi)) { bv = s_av[w][r]; bi = s_ai[w][r]; }
          publish(m, bv, bi);
        }
      }
    }
  } else if constexpr (EPI == EPI_ADD) {
    // x += y, staged through LDS as fp32 so that every thread then owns
    // whole 16-byte pieces (8 columns of one row): x and the next norm's
    // operand are written as 16-byte stores, and a row's sum of squares over
    // the tile is a reduction over the APR adjacent lanes holding its pieces
    constexpr int LDF = ATC + 4;                 // padded staging row (floats)
    float* stg;
    if constexpr (TR * LDF * 4 <= (int)sizeof(As)) {
      stg = reinterpret_cast<float*>(&As[0][0][0]);
    } else {                                     // 256-row tiles: a buffer of its own
      __shared__ float stg_add[TR * LDF];
      stg = stg_add;
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stg[(rb * 16 + 4 * (lane >> 4) + r) * LDF + (wave * NBW + nb) * 16 + col] = acc[rb][nb][r];
    __syncthreads();
    const bool nxt = g.next_gain != nullptr && g.xn_out != nullptr;
    const bool ssq = g.next_gain != nullptr && g.ss_out != nullptr;
#pragma unroll
    for (int i = 0; i < ANP; ++i) {
      const int p = i * W * 64 + threadIdx.x;
      const int rl = p / APR, m = mt * TR + rl;
      const int c = nt * ATC + 8 * (p % APR);
      const bool st = p < TR * APR && m < g.M && c < g.N;
      const f32x4* sp = reinterpret_cast<const f32x4*>(stg + (p < TR * APR ? rl : 0) * LDF + 8 * (p % APR));
      const f32x4 x0 = xr[i][0] + sp[0], x1 = xr[i][1] + sp[1];
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sq += x0[e] * x0[e] + x1[e] * x1[e];
      if (st) {
        f32x4* xp = reinterpret_cast<f32x4*>(g.out_f32 + (size_t)m * g.N + c);
        xp[0] = x0;
        xp[1] = x1;
        if (nxt) {
          const uint32_t gw[4] = {gr[i].x, gr[i].y, gr[i].z, gr[i].w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a = (e < 2 ? x0 : x1)[(2 * e) & 3], b = (e < 2 ? x0 : x1)[(2 * e + 1) & 3];
            o[e] = (uint32_t)f32_to_bf16(a * bf16_to_f32((u16)(gw[e] & 0xffff))) |
                   ((uint32_t)f32_to_bf16(b * bf16_to_f32((u16)(gw[e] >> 16))) << 16);
          }
          *reinterpret_cast<uint4*>(g.xn_out + packed_index(m, c, g.N)) = uint4{o[0], o[1], o[2], o[3]};
        }
      }
      if (ssq) {
        sq = st ? sq : 0.f;
        sq += MV_DPP(sq, 0xB1);      // quad_perm [1,0,3,2]
        sq += MV_DPP(sq, 0x4E);      // quad_perm [2,3,0,1]
        sq += MV_DPP(sq, 0x141);     // row_half_mirror: the 8 lanes of a row's pieces
        if constexpr (APR == 16) sq += MV_DPP(sq, 0x140);   // row_mirror
        if (p % APR == 0 && p < TR * APR && m < g.M) g.ss_out[(size_t)m * g.ss_ld + nt] = sq;
      }
    }
  } else if constexpr (SPLIT_GU) {
    // gate wave w and up wave w + FW hold the same rows and columns in the
    // same lanes: the up waves park their accumulators in the operand LDS,
    // the gate waves form h = SiLU(gate) * up and stage it as bf16, then
    // write whole 16-byte pieces (8 features of one row)
    static_assert(FW * TR * 16 * 2 <= (int)sizeof(As), "SwiGLU staging fits the operand LDS");
    float* upv;
    if constexpr (FW * MB * 4 * 64 * 4 <= (int)sizeof(As)) {
      upv = reinterpret_cast<float*>(&As[0][0][0]);
    } else {                                     // 10-wave 256-row tiles: a buffer of its own
      __shared__ float upv_own[FW * MB * 4 * 64];
      upv = upv_own;
    }
    if (wave >= FW) {
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) upv[(((wave - FW) * MB + rb) * 4 + r) * 64 + lane] = acc[rb][0][r];
    }
    __syncthreads();
    u16 hv[MB][4];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        hv[rb][r] = wave < FW ? f32_to_bf16(silu_f(acc[rb][0][r]) *
                                            upv[((wave * MB + rb) * 4 + r) * 64 + lane])
                              : (u16)0;
    __syncthreads();
    u16* stg = reinterpret_cast<u16*>(&As[0][0][0]) + (wave % FW) * TR * 16;
    if (wave < FW) {
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[(rb * 16 + 4 * (lane >> 4) + r) * 16 + col] = hv[rb][r];
    }
    __syncthreads();
    if (wave < FW && active) {
#pragma unroll
      for (int p = lane; p < TR * 2; p += 64) {
        const int rl = p >> 1, m = mt * TR + rl;
        if (m < g.M)
          *reinterpret_cast<uint4*>(g.out_bf16 + packed_index(m, wb * 16 + 8 * (p & 1), g.N)) =
              *reinterpret_cast<const uint4*>(stg + rl * 16 + 8 * (p & 1));
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // h = SiLU(gate) * up, staged per wave in the operand LDS as bf16 so that
    // each lane then writes whole 16-byte pieces (8 features of one row)
    static_assert(W * TR * 16 * 2 <= (int)sizeof(As), "SwiGLU staging fits the operand LDS");
    u16* stg = reinterpret_cast<u16*>(&As[0][0][0]) + wave * TR * 16;
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        stg[(rb * 16 + 4 * (lane >> 4) + r) * 16 + col] =
            f32_to_bf16(silu_f(acc[rb][0][r]) * acc[rb][1][r]);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int p = lane; p < TR * 2; p += 64) {
        const int rl = p >> 1, m = mt * TR + rl;
        if (m < g.M)
          *reinterpret_cast<uint4*>(g.out_bf16 + packed_index(m, wb * 16 + 8 * (p & 1), g.N)) =
              *reinterpret_cast<const uint4*>(stg + rl * 16 + 8 * (p & 1));
      }
    }
  } else if constexpr (EPI == EPI_QKV) {
    // RoPE in registers, then the tile (TR rows x W*32 packed features) is
    // staged as bf16 in the operand LDS and written out in 16-byte pieces:
    // q rows, K pieces of 8 dims of one slot, V runs of 8 slots of one dim
    // (single elements where a run is not whole in this tile)
    const QkvArgs& q = g.qkv;
    constexpr int TC = W * NBW * 16;             // packed features of the tile
    constexpr int LDT = TC + 8;                  // padded staging row (u16)
    u16* stg;
    if constexpr (NBW == 2 && TR * LDT * 2 <= (int)sizeof(As)) {
      stg = reinterpret_cast<u16*>(&As[0][0][0]);
    } else {        // 256-row tiles, or the RoPE partners parked in the operand LDS: a buffer of its own
      __shared__ u16 stg_own[TR * LDT];
      stg = stg_own;
    }
    const bool first = ((f0 % q.d) % q.hd) < half;    // block 0 holds the first half (narrow heads)
    if constexpr (CS_LATE) load_cs();
    if constexpr (NBW == 2) {
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float y0 = acc[rb][0][r], y1 = acc[rb][1][r];
          float s0 = 0.f, s1 = 0.f;
          if (!wide) {             // uniform: 16-wide heads only
            s0 = __shfl_xor(y0, 8, 64);
            s1 = __shfl_xor(y1, 8, 64);
          }
          const float c = cs[rb][r].x, sn = cs[rb][r].y;
          float o0 = y0, o1 = y1;
          if (rot) {
            if (wide) {            // (x_i, x_{i+hd/2}) -> (x_i c - x_{i+h} s, x_{i+h} c + x_i s)
              o0 = y0 * c - y1 * sn;
              o1 = y1 * c + y0 * sn;
            } else {               // partners 8 lanes apart inside each block
              o0 = first ? y0 * c - s0 * sn : y0 * c + s0 * sn;
              o1 = first ? y1 * c - s1 * sn : y1 * c + s1 * sn;
            }
          }
          const int rl = rb * 16 + 4 * (lane >> 4) + r;
          stg[rl * LDT + wave * 32 + col] = f32_to_bf16(o0);
          stg[rl * LDT + wave * 32 + 16 + col] = f32_to_bf16(o1);
        }
    } else {
      // one block per wave: with heads wider than 16 the RoPE partners of an
      // even wave's block are the next (odd) wave's, in the same lanes; the
      // odd waves park their accumulators in the operand LDS and the even
      // waves rotate both blocks
      static_assert(NBW == 2 || (W % 2 == 0 && (W / 2) * MB * 4 * 64 * 4 <= (int)sizeof(As)),
                    "RoPE pairing fits the operand LDS");
      float* pv = reinterpret_cast<float*>(&As[0][0][0]);
      if (wide) {                // uniform
        if (wave & 1) {
#pragma unroll
          for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[(((wave >> 1) * MB + rb) * 4 + r) * 64 + lane] = acc[rb][0][r];
        }
        __syncthreads();
        if (!(wave & 1)) {
#pragma unroll
          for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float y0 = acc[rb][0][r], y1 = pv[(((wave >> 1) * MB + rb) * 4 + r) * 64 + lane];
              const float c = cs[rb][r].x, sn = cs[rb][r].y;
              const float o0 = rot ? y0 * c - y1 * sn : y0, o1 = rot ? y1 * c + y0 * sn : y1;
              const int rl = rb * 16 + 4 * (lane >> 4) + r;
              stg[rl * LDT + wave * 16 + col] = f32_to_bf16(o0);
              stg[rl * LDT + wave * 16 + 16 + col] = f32_to_bf16(o1);
            }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float y0 = acc[rb][0][r];
            const float s0 = __shfl_xor(y0, 8, 64);
            const float c = cs[rb][r].x, sn = cs[rb][r].y;
            const float o0 = rot ? (first ? y0 * c - s0 * sn : y0 * c + s0 * sn) : y0;
            const int rl = rb * 16 + 4 * (lane >> 4) + r;
            stg[rl * LDT + wave * 16 + col] = f32_to_bf16(o0);
          }
      }
    }
    __syncthreads();
    const int tc0 = nt * TC, mr0 = mt * TR;
    const int p_end = min(tc0 + TC, g.N);
    const int hs = __ffs(q.hd) - 1;              // hd is a power of two
    // the sequences with rows in this tile (at most MV_MAX_BATCH): their
    // first tile row, row count and the cache slot of that row
    const int m_hi = min(mr0 + TR, g.M);
    const int b_lo = mr0 / q.T;
    int sr0[MV_MAX_BATCH], sn[MV_MAX_BATCH], ss0[MV_MAX_BATCH];
#pragma unroll
    for (int e = 0; e < MV_MAX_BATCH; ++e) {
      const int b = b_lo + e;
      const int lo_m = max(mr0, b * q.T), hi_m = min(m_hi, (b + 1) * q.T);
      sn[e] = b < q.B ? max(hi_m - lo_m, 0) : 0;
      sr0[e] = lo_m - mr0;
      ss0[e] = sn[e] ? s_slot0[min(b, MV_MAX_BATCH - 1)] + (lo_m - b * q.T) : 0;
    }
    // q and K: 16-byte pieces of 8 consecutive features (8 consecutive packed
    // rows of a 16-row block are 8 consecutive dims of one head)
    if (tc0 < 2 * q.d) {
      constexpr int CU = TC / 8;
      const bool q_tile = tc0 + TC <= q.d;
      for (int u = threadIdx.x; u < TR * CU; u += W * 64) {
        // q: neighbouring threads take neighbouring pieces of a row;
        // K: neighbouring threads take neighbouring rows (slots) of a piece
        const int rl = q_tile ? u / CU : u % TR, cu = q_tile ? u % CU : u / TR;
        const int p = tc0 + cu * 8, m = mr0 + rl;
        if (p >= 2 * q.d || p >= p_end || m >= g.M) continue;
        int f = p;                                // qkv_feature with shifts
        if (q.hd >= 32) {
          const int e = p & (q.hd - 1), jj = e >> 5, ee = e & 31;
          f = (p - e) + (ee < 16 ? jj * 16 + ee : (q.hd >> 1) + jj * 16 + (ee - 16));
        }
        const uint4 v = *reinterpret_cast<const uint4*>(stg + rl * LDT + cu * 8);
        if (f < q.d) {
          *reinterpret_cast<uint4*>(q.q + (size_t)m * q.d + f) = v;
        } else {
          const int c = f - q.d, h = c >> hs, i = c & (q.hd - 1);
          int b = b_lo, slot = 0;
#pragma unroll
          for (int e = 0; e < MV_MAX_BATCH; ++e)
            if (rl >= sr0[e] && rl < sr0[e] + sn[e]) { b = b_lo + e; slot = ss0[e] + rl - sr0[e]; }
          *reinterpret_cast<uint4*>(q.kcache + ((size_t)b * q.H + h) * q.cap * q.hd +
                                    kv_k_off(slot, i, q.hd)) = v;
        }
      }
    }
    if (p_end > 2 * q.d) {
      // V: 8-slot groups (8-aligned) of each sequence's slots in this tile; a
      // whole group is one 16-byte store per dim, a partial one (first or
      // last of a sequence) is written element by element
      int gf[MV_MAX_BATCH], gc[MV_MAX_BATCH], G = 0;
#pragma unroll
      for (int e = 0; e < MV_MAX_BATCH; ++e) {
        gf[e] = ss0[e] >> 3;
        gc[e] = sn[e] ? ((ss0[e] + sn[e] - 1) >> 3) - gf[e] + 1 : 0;
        G += gc[e];
      }
      for (int u = threadIdx.x; u < G * TC; u += W * 64) {
        const int j = u % TC, p = tc0 + j;
        if (p < 2 * q.d || p >= p_end) continue;
        int k = u / TC, b = b_lo, r0 = 0, s0 = 0, n = 0, gs = 0;
#pragma unroll
        for (int e = 0; e < MV_MAX_BATCH; ++e) {
          if (k >= 0 && k < gc[e]) { b = b_lo + e; r0 = sr0[e]; s0 = ss0[e]; n = sn[e]; gs = (gf[e] + k) * 8; }
          k -= gc[e];
        }
        const int c = p - 2 * q.d, h = c >> hs, i = c & (q.hd - 1);
        u16* vb = q.vcache + ((size_t)b * q.H + h) * q.cap * q.hd;
        const int lo_s = max(gs, s0), hi_s = min(gs + 8, s0 + n);
        const u16* src = stg + (r0 + lo_s - s0) * LDT + j;
        if (lo_s == gs && hi_s == gs + 8) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)src[2 * e * LDT] | ((uint32_t)src[(2 * e + 1) * LDT] << 16);
          *reinterpret_cast<uint4*>(vb + kv_v_off(gs, i, q.hd)) = uint4{w[0], w[1], w[2], w[3]};
        } else {
          for (int sl = lo_s; sl < hi_s; ++sl) vb[kv_v_off(sl, i, q.hd)] = src[(sl - lo_s) * LDT];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide tiles for launches of more than 128 rows (a 256-node tree, a batch of
// four 64-node trees, 256-row prefill chunks).  There each weight byte meets
// 256 rows, next to the MFMA ridge, and the 16-row-block tiles above -- whose
// waves each read the whole 256-row operand from LDS for one 16-column block
// -- are bound by LDS reads.  Here a workgroup of 8 waves owns 256 rows x
// 32*NBH columns: wave (wm, wn) computes rows 64*wm .. +63 against column
// blocks NBH*wn .. +NBH-1 of the tile (4 x NBH accumulators of 16 x 16), so
// every fragment read from LDS feeds NBH or 4 MFMAs.  Both operands go from
// memory straight into LDS (buffer loads that write LDS, one 1 KiB fragment
// piece per instruction), WIDE_KS k-blocks a stage, in three stage buffers
// with two stages in flight; one barrier a stage.  (Staged through registers
// instead, three stages deep, the kernel held 195-256 VGPRs and ran 2-8%
// slower at the 13B and 33B shapes.)  The epilogues work
// on the tile staged in LDS as fp32 (SwiGLU: the up accumulators parked
// there), so that every global store is a whole 16-byte piece.
// SwiGLU tiles take gate blocks NBH*nt .. +NBH-1 (waves wn = 0) and the same
// up blocks (wn = 1); the others take column blocks 2*NBH*nt .. +2*NBH-1.
// Measured (13B gate/up, 256 rows, 216 tiles): 93 us against 97 us for the
// 16-row-block tiles; the loop is bound by LDS traffic (88 KiB a k-block and
// compute unit): with the memory loads removed it still takes 75 us, 55 us
// without the LDS stores, against 34 us of MFMA work.  A third LDS buffer
// with fragments read a stage ahead, and 4-wave tiles taking the
// activations straight from L2 (registers exhausted, accumulators moved
// between register files in the loop) were slower.
// ---------------------------------------------------------------------------
constexpr int WIDE_KS = 2;       // k-blocks per stage
constexpr int WIDE_TR = 256;     // rows of a tile

template <int NBH, int EPI>
struct WideShape {
  static constexpr int NB = 2 * NBH;                  // 16-column blocks of a tile
  static constexpr int TC = 16 * NB;                  // columns of a tile
  static constexpr int AP = 16 * WIDE_KS;             // activation pieces (1 KiB) a stage
  static constexpr int WP = NB * WIDE_KS;             // weight pieces a stage
  static constexpr int AL = AP / 8;                   // ... loaded per thread
  static constexpr int WL = (WP + 7) / 8;
  static constexpr int WPS = WP;                      // weight slots
  static constexpr int OPB = (AP + WPS) * 64;         // bf16x8 of one stage buffer
  static constexpr int NBUF = 3;                      // stage buffers in LDS
  static constexpr int LDF = TC + 4;                  // fp32 staging row (floats)
  static constexpr int FT = 16 * NBH;                 // SwiGLU: features of a tile
  static constexpr int LDH = FT + 8;                  // SwiGLU: bf16 staging row (u16)
  static constexpr int STG_BYTES = EPI == EPI_SWIGLU ? WIDE_TR * FT * 4 + WIDE_TR * LDH * 2
                                                     : WIDE_TR * LDF * 4;
  static constexpr int SMEM16 = (NBUF * OPB * 16 > STG_BYTES ? NBUF * OPB * 16 : STG_BYTES) / 16;
};

template <int NBH, int EPI>
__global__ __launch_bounds__(512) void gemm_wide_kernel(GemmArgs g) {
  using S = WideShape<NBH, EPI>;
  constexpr int NB = S::NB, TC = S::TC, AP = S::AP, WP = S::WP, AL = S::AL, WL = S::WL;
  constexpr int OPB = S::OPB, LDF = S::LDF;
  static_assert(AP % 8 == 0, "activation pieces divide over the waves");
  __shared__ bf16x8 smem[S::SMEM16];
  __shared__ float rs_s[WIDE_TR];
  __shared__ int s_last;
  __shared__ int s_slot0[MV_MAX_BATCH];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 3, wn = wave >> 2;
  const int nt = blockIdx.x, split = blockIdx.y, mt = blockIdx.z;
  const int KB = g.K >> 5;
  const int lo = (int)((long long)KB * split / g.splits);
  const int hi = (int)((long long)KB * (split + 1) / g.splits);
  const int nst = (hi - lo + WIDE_KS - 1) / WIDE_KS;
  const int NBtot = g.N >> 4;                  // 16-column blocks of W (SwiGLU: of gate and of up)
  const int MBtot = g.Mp >> 4;
  const int NT = EPI == EPI_SWIGLU ? (NBtot + NBH - 1) / NBH : (NBtot + NB - 1) / NB;

  // Operand loads are range-checked buffer loads: k-blocks past the split's
  // range get an offset past the buffer and read zeros, so the LDS copies
  // need no selects or branches.
  constexpr uint32_t OOB = 0x80000000u;        // past every operand (each < 2 GiB)
  // the weight block of tile block j (clamped: blocks past the matrix load
  // valid memory and are never stored)
  auto wblk = [&](int j) {
    const int blk = EPI == EPI_SWIGLU ? nt * NBH + (j < NBH ? j : j - NBH) : nt * NB + j;
    return min(blk, NBtot - 1);
  };

  // Stage st's pieces go from memory straight into LDS buffer buf, one
  // 1 KiB piece per instruction (the operands are stored in fragment order,
  // so a piece is contiguous in both): activation piece p = 8i + wave is
  // (kl = p / 16, row block p % 16), weight piece p = 8i + wave is
  // (kl = p / NB, block p % NB); the waves past the last weight piece copy
  // that piece again (the same bytes to the same place).  The copies are
  // inline assembly, which the compiler's wait insertion does not see (it
  // cannot tell the stage buffers apart and would hold every fragment read
  // until all copies had landed); each step waits for its own stage by hand,
  // and the only loads the compiler tracks (the norm factors) are used after
  // the loop.  The LDS address goes in as an m0 operand, so the compiler
  // itself sets m0 and knows its value is consumed there.
  constexpr int DPW = AL + WL;                 // copies per wave and stage
  auto piece_a = [&](int st, int i, uint32_t& off) {
    const int pc = i * 8 + wave;
    const int k = lo + st * WIDE_KS + pc / 16;
    const int rbg = min(mt * 16 + pc % 16, MBtot - 1);
    off = k < hi ? (uint32_t)((rbg * KB + k) * 64 + lane) * 16u : OOB;
    return pc;
  };
  auto piece_w = [&](int st, int i, uint32_t& off, bool& second) {
    const int pc = min(i * 8 + wave, WP - 1);
    const int k = lo + st * WIDE_KS + pc / NB, j = pc % NB;
    off = k < hi ? (uint32_t)((k * NBtot + wblk(j)) * 64 + lane) * 16u : OOB;
    second = EPI == EPI_SWIGLU && j >= NBH;
    return AP + pc;
  };
  const uint64_t ba = (uint64_t)g.A, bw = (uint64_t)g.W,
                 bw2 = (uint64_t)(EPI == EPI_SWIGLU ? g.W2 : g.W);
  const i32x4 qA = {(int)(uint32_t)ba, (int)(uint32_t)(ba >> 32), MBtot * KB * 1024, MV_BUF_DWORD3};
  const i32x4 qW = {(int)(uint32_t)bw, (int)(uint32_t)(bw >> 32), KB * NBtot * 1024, MV_BUF_DWORD3};
  const i32x4 qW2 = {(int)(uint32_t)bw2, (int)(uint32_t)(bw2 >> 32), KB * NBtot * 1024,
                     MV_BUF_DWORD3};
  auto lds_addr = [](const bf16x8* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) bf16x8*)p;
  };
  auto copy_asm = [&](int st, int buf) {
    bf16x8* sb = smem + buf * OPB;
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      uint32_t off;
      const int pc = piece_a(st, i, off);
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(sb + pc * 64));
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :: "v"(off), "s"(qA), "{m0}"(la) : "memory");
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      uint32_t off;
      bool second;
      const int pc = piece_w(st, i, off, second);
      const uint32_t la = __builtin_amdgcn_readfirstlane(lds_addr(sb + pc * 64));
      if (second)
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :: "v"(off), "s"(qW2), "{m0}"(la) : "memory");
      else
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :: "v"(off), "s"(qW), "{m0}"(la) : "memory");
    }
  };

  f32x4 acc[4][NBH];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NBH; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one k-block's fragments of this wave from stage buffer buf, and its MFMAs
  auto read_frags = [&](int buf, int kl, bf16x8 (&af)[4], bf16x8 (&wf)[NBH]) {
    const bf16x8* sb = smem + buf * OPB;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = sb[(kl * 16 + 4 * wm + i) * 64 + lane];
#pragma unroll
    for (int j = 0; j < NBH; ++j) wf[j] = sb[(AP + kl * NB + NBH * wn + j) * 64 + lane];
  };
  auto mfma_kb = [&](const bf16x8 (&af)[4], const bf16x8 (&wf)[NBH]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBH; ++j) acc[i][j] = mfma16x16x32(af[i], wf[j], acc[i][j]);
  };

  // norm factors: two threads a row, up to WIDE_SSQ f32x4 of partial sums
  // each, requested before the first copies and summed after the loop
  // (longer rows of partials: summed serially there)
  constexpr int WIDE_SSQ = 8;
  const bool ss_fast = g.ss != nullptr && g.ss_tiles <= 2 * 4 * WIDE_SSQ;
  f32x4 ssv[WIDE_SSQ];
  {
    const int r = threadIdx.x >> 1, hf = threadIdx.x & 1;
    const int m = min(mt * WIDE_TR + r, g.M - 1);
    const f32x4* p4 = reinterpret_cast<const f32x4*>(g.ss + (size_t)m * g.ss_ld);
#pragma unroll
    for (int u = 0; u < WIDE_SSQ; ++u) {
      const int t = 2 * u + hf;
      ssv[u] = ss_fast && 4 * t < g.ss_tiles ? p4[t] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  int nraw = 0;
  if (EPI == EPI_QKV && threadIdx.x < g.qkv.B) nraw = g.qkv.n_prefix[threadIdx.x];
  // three LDS stage buffers, two stages copied ahead
  copy_asm(0, 0);
  copy_asm(1, 1);
  // Step s: wait for this wave's copies of stage s (those of stage s + 1 may
  // still fly) and for its LDS reads, barrier (stage s is readable and the
  // buffer of stage s - 1 free), copy stage s + 2 into that buffer, then
  // multiply stage s.  Copies past the range read zeros; the loop drains
  // them before the epilogues reuse the LDS.
  constexpr int GATE = (DPW & 15) | (7 << 4) | ((DPW >> 4) << 14);   // vmcnt(DPW) lgkmcnt(0)
  for (int st = 0; st < nst; ++st) {
    asm volatile("s_waitcnt %0\n\ts_barrier" :: "i"(GATE) : "memory");
    copy_asm(st + 2, (st + 2) % 3);
    const int buf = st % 3;
    bf16x8 fa[4], fw[NBH];
#pragma unroll
    for (int kl = 0; kl < WIDE_KS; ++kl) {
      read_frags(buf, kl, fa, fw);
      mfma_kb(fa, fw);
    }
  }
  // the norm factors (their loads went out before the copies and are long
  // done), then the copies past the range drained and rs_s made visible
  if (ss_fast) {
    const int r = threadIdx.x >> 1, hf = threadIdx.x & 1;
    float sm = 0.f;
#pragma unroll
    for (int u = 0; u < WIDE_SSQ; ++u) {
      const int t = 2 * u + hf;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm += 4 * t + e < g.ss_tiles ? ssv[u][e] : 0.f;
    }
    sm += __shfl_xor(sm, 1, 64);
    if (hf == 0) rs_s[r] = mt * WIDE_TR + r < g.M ? 1.0f / sqrtf(sm / (float)g.K + 1e-5f) : 1.f;
  } else if (g.ss) {
    for (int r = threadIdx.x; r < WIDE_TR; r += 512) {
      const int m = mt * WIDE_TR + r;
      float sm = 0.f;
      if (m < g.M) {
        const float* row = g.ss + (size_t)m * g.ss_ld;
        for (int e = 0; e < g.ss_tiles; ++e) sm += row[e];
      }
      rs_s[r] = m < g.M ? 1.0f / sqrtf(sm / (float)g.K + 1e-5f) : 1.f;
    }
  }
  if (EPI == EPI_QKV && threadIdx.x < g.qkv.B)
    s_slot0[threadIdx.x] = min(max(nraw, 0), g.qkv.cap - g.qkv.T);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---- split-K: the last workgroup of the tile sums the splits in order
  if (g.splits > 1) {
    constexpr int WQ = 4 * NBH;                // f32x4 items per lane of one wave
    const int tile = mt * NT + nt;
    const int per_split = 8 * WQ * 256 * 4;    // bytes of one split's tile
    const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
        g.partial + (size_t)tile * g.splits * (per_split / 4), (short)0, g.splits * per_split,
        MV_BUF_DWORD3);
    const int lane_off = (wave * WQ * 256 + lane * 4) * 4;
#pragma unroll
    for (int q = 0; q < WQ; ++q)
      __builtin_amdgcn_raw_buffer_store_b128(acc[q / NBH][q % NBH], part,
                                             split * per_split + lane_off + q * 1024, 0, MV_CPOL_SYS);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(g.counters + tile, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == g.splits - 1;
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBH; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < g.splits; ++sp) {
      f32x4 v[WQ];
#pragma unroll
      for (int q = 0; q < WQ; ++q)
        v[q] = __builtin_amdgcn_raw_buffer_load_b128(part, sp * per_split + lane_off + q * 1024, 0,
                                                     MV_CPOL_SYS);
#pragma unroll
      for (int q = 0; q < WQ; ++q) acc[q / NBH][q % NBH] += v[q];
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(g.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogues: lane holds tile rows 64*wm + 16*i + 4*(lane/16) + r,
  // tile column 16*(NBH*wn + j) + lane%16
  if (g.ss) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = rs_s[64 * wm + 16 * i + 4 * (lane >> 4) + r];
#pragma unroll
        for (int j = 0; j < NBH; ++j) acc[i][j][r] *= f;
      }
  }
  const int col = lane & 15;
  const int mr0 = mt * WIDE_TR;
  if constexpr (EPI == EPI_SWIGLU) {
    // up waves park their accumulators; gate waves form h = SiLU(gate) * up
    // as bf16 [row][feature]; then 16-byte pieces (8 features of one row)
    constexpr int FT = S::FT, LDH = S::LDH;
    float* park = reinterpret_cast<float*>(smem);                       // [wm][i][j][r][lane]
    u16* hs = reinterpret_cast<u16*>(park + WIDE_TR * FT);              // [row][LDH]
    if (wn == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) park[(((wm * 4 + i) * NBH + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NBH; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float u = park[(((wm * 4 + i) * NBH + j) * 4 + r) * 64 + lane];
            hs[(64 * wm + 16 * i + 4 * (lane >> 4) + r) * LDH + 16 * j + col] =
                f32_to_bf16(silu_f(acc[i][j][r]) * u);
          }
    }
    __syncthreads();
    constexpr int PPR = FT / 8;                // pieces per row
    for (int p = threadIdx.x; p < WIDE_TR * PPR; p += 512) {
      const int rl = p / PPR, f = nt * FT + 8 * (p % PPR), m = mr0 + rl;
      if (m < g.M && f < g.N)
        *reinterpret_cast<uint4*>(g.out_bf16 + packed_index(m, f, g.N)) =
            *reinterpret_cast<const uint4*>(hs + rl * LDH + 8 * (p % PPR));
    }
    return;
  } else {
    float* stg = reinterpret_cast<float*>(smem);   // [row][LDF] fp32 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NBH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stg[(64 * wm + 16 * i + 4 * (lane >> 4) + r) * LDF + 16 * (NBH * wn + j) + col] = acc[i][j][r];
    __syncthreads();
    const int tc0 = nt * TC;
    if constexpr (EPI == EPI_STORE) {
      constexpr int PPR = TC / 4;              // float4 pieces per row
      bool bad = false;
      for (int p = threadIdx.x; p < WIDE_TR * PPR; p += 512) {
        const int rl = p / PPR, c = tc0 + 4 * (p % PPR), m = mr0 + rl;
        if (m < g.M && c < g.N) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + rl * LDF + 4 * (p % PPR));
          *reinterpret_cast<f32x4*>(g.out_f32 + (size_t)m * g.N + c) = v;
          bad |= !(__builtin_isfinite(v[0]) && __builtin_isfinite(v[1]) && __builtin_isfinite(v[2]) &&
                   __builtin_isfinite(v[3]));
        }
      }
      if (g.status && __ballot(bad) != 0ull && lane == 0) atomicOr(g.status, MV_STATUS_NONFINITE);
      if (g.amax_key) {
        // two threads a row, each over half the tile's columns; ties go to
        // the lower column, NaNs never win
        const int rl = threadIdx.x >> 1, hf = threadIdx.x & 1, m = mr0 + rl;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int c = hf * (TC / 2); c < (hf + 1) * (TC / 2); ++c) {
          if (tc0 + c >= g.N) break;
          const float v = stg[rl * LDF + c];
          if (v > bv) { bv = v; bi = tc0 + c; }
        }
        const float ov = __shfl_xor(bv, 1, 64);
        const int oi = __shfl_xor(bi, 1, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        if (hf == 0 && m < g.M) {
          const unsigned long long key = argmax_key(bv, bi);
          if (key > __hip_atomic_load(g.amax_key + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            __hip_atomic_fetch_max(g.amax_key + m, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else if constexpr (EPI == EPI_ADD) {
      // 16 adjacent lanes own the 16 pieces of 8 columns of one row: x += y,
      // the next norm's operand, and the row's sum of squares over the tile
      static_assert(TC == 128, "a row's pieces fill one DPP row");
      const bool nxt = g.next_gain != nullptr && g.xn_out != nullptr;
      const bool ssq = g.next_gain != nullptr && g.ss_out != nullptr;
      for (int p = threadIdx.x; p < WIDE_TR * 16; p += 512) {
        const int rl = p >> 4, c = tc0 + 8 * (p & 15), m = mr0 + rl;
        const bool st = m < g.M && c < g.N;
        const f32x4* sp = reinterpret_cast<const f32x4*>(stg + rl * LDF + 8 * (p & 15));
        f32x4 x0 = sp[0], x1 = sp[1];
        float sq = 0.f;
        if (st) {
          f32x4* xp = reinterpret_cast<f32x4*>(g.out_f32 + (size_t)m * g.N + c);
          x0 += xp[0];
          x1 += xp[1];
          xp[0] = x0;
          xp[1] = x1;
#pragma unroll
          for (int e = 0; e < 4; ++e) sq += x0[e] * x0[e] + x1[e] * x1[e];
          if (nxt) {
            const uint4 gr = *reinterpret_cast<const uint4*>(g.next_gain + c);
            const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a = (e < 2 ? x0 : x1)[(2 * e) & 3], b = (e < 2 ? x0 : x1)[(2 * e + 1) & 3];
              o[e] = (uint32_t)f32_to_bf16(a * bf16_to_f32((u16)(gw[e] & 0xffff))) |
                     ((uint32_t)f32_to_bf16(b * bf16_to_f32((u16)(gw[e] >> 16))) << 16);
            }
            *reinterpret_cast<uint4*>(g.xn_out + packed_index(m, c, g.N)) = uint4{o[0], o[1], o[2], o[3]};
          }
        }
        if (ssq) {
          sq += MV_DPP(sq, 0xB1);
          sq += MV_DPP(sq, 0x4E);
          sq += MV_DPP(sq, 0x141);
          sq += MV_DPP(sq, 0x140);
          if ((p & 15) == 0 && m < g.M) g.ss_out[(size_t)m * g.ss_ld + nt] = sq;
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      const QkvArgs& q = g.qkv;
      const int half = q.hd >> 1;
      const bool wide = q.hd >= 32;
      // RoPE in place on the q and k columns: packed column pairs (c, c + 16)
      // of each 32-group (heads of 32+ dims: dims i and i + hd/2 of one head)
      // or (c, c + 8) of each 16-block (16-dim heads)
      const int pw = wide ? 16 : 8;
      for (int it = threadIdx.x; it < WIDE_TR * (TC / 2); it += 512) {
        const int rl = it / (TC / 2), pr = it % (TC / 2);
        const int c = (pr / pw) * 2 * pw + pr % pw;   // first column of the pair
        const int pcol = tc0 + c, m = mr0 + rl;
        if (pcol >= 2 * q.d || m >= g.M) continue;
        const int f = wide ? qkv_feature(pcol, q.d, q.hd) : pcol;
        const int ci = (f % q.d) % q.hd % half;
        const float2 cs = q.rope[(size_t)m * half + ci];
        float* a = stg + rl * LDF + c;
        const float y0 = a[0], y1 = a[pw];
        a[0] = y0 * cs.x - y1 * cs.y;
        a[pw] = y1 * cs.x + y0 * cs.y;
      }
      __syncthreads();
      const int hs_ = __ffs(q.hd) - 1;           // hd is a power of two
      // q and K: 16-byte pieces of 8 consecutive features (8 consecutive
      // packed columns of a 16-block are 8 consecutive dims of one head)
      if (tc0 < 2 * q.d) {
        for (int u = threadIdx.x; u < WIDE_TR * (TC / 8); u += 512) {
          const int rl = u / (TC / 8), cu = u % (TC / 8);
          const int pcol = tc0 + cu * 8, m = mr0 + rl;
          if (pcol >= 2 * q.d || pcol >= g.N || m >= g.M) continue;
          const int f = wide ? qkv_feature(pcol, q.d, q.hd) : pcol;
          const f32x4* sp = reinterpret_cast<const f32x4*>(stg + rl * LDF + cu * 8);
          const f32x4 v0 = sp[0], v1 = sp[1];
          uint4 o;
          o.x = (uint32_t)f32_to_bf16(v0[0]) | ((uint32_t)f32_to_bf16(v0[1]) << 16);
          o.y = (uint32_t)f32_to_bf16(v0[2]) | ((uint32_t)f32_to_bf16(v0[3]) << 16);
          o.z = (uint32_t)f32_to_bf16(v1[0]) | ((uint32_t)f32_to_bf16(v1[1]) << 16);
          o.w = (uint32_t)f32_to_bf16(v1[2]) | ((uint32_t)f32_to_bf16(v1[3]) << 16);
          if (f < q.d) {
            *reinterpret_cast<uint4*>(q.q + (size_t)m * q.d + f) = o;
          } else {
            const int b = min(m / q.T, MV_MAX_BATCH - 1), node = m - b * q.T;
            const int cc = f - q.d, h = cc >> hs_, i = cc & (q.hd - 1);
            *reinterpret_cast<uint4*>(q.kcache + ((size_t)b * q.H + h) * q.cap * q.hd +
                                      kv_k_off(s_slot0[b] + node, i, q.hd)) = o;
          }
        }
      }
      // V: each thread one (8-slot group, dim) of a sequence's slots in this
      // tile: a whole group is one 16-byte store, a partial one (first or
      // last of a sequence) element by element
      if (tc0 + TC > 2 * q.d) {
        const int m_hi = min(mr0 + WIDE_TR, g.M);
        const int b_lo = mr0 / q.T;
        for (int e = 0; e < MV_MAX_BATCH; ++e) {
          const int b = b_lo + e;
          if (b >= q.B) break;
          const int lo_m = max(mr0, b * q.T), hi_m = min(m_hi, (b + 1) * q.T);
          if (lo_m >= hi_m) continue;
          const int s0 = s_slot0[b] + (lo_m - b * q.T), ns = hi_m - lo_m;
          const int gf = s0 >> 3, gc = ((s0 + ns - 1) >> 3) - gf + 1;
          for (int u = threadIdx.x; u < gc * TC; u += 512) {
            const int j = u % TC, pcol = tc0 + j;
            if (pcol < 2 * q.d || pcol >= g.N) continue;
            const int gs = (gf + u / TC) * 8;
            const int cc = pcol - 2 * q.d, h = cc >> hs_, i = cc & (q.hd - 1);
            u16* vb = q.vcache + ((size_t)b * q.H + h) * q.cap * q.hd;
            const int lo_s = max(gs, s0), hi_s = min(gs + 8, s0 + ns);
            const float* src = stg + (lo_m - mr0 + lo_s - s0) * LDF + j;
            if (lo_s == gs && hi_s == gs + 8) {
              uint32_t w4[4];
#pragma unroll
              for (int t = 0; t < 4; ++t)
                w4[t] = (uint32_t)f32_to_bf16(src[2 * t * LDF]) |
                        ((uint32_t)f32_to_bf16(src[(2 * t + 1) * LDF]) << 16);
              *reinterpret_cast<uint4*>(vb + kv_v_off(gs, i, q.hd)) = uint4{w4[0], w4[1], w4[2], w4[3]};
            } else {
              for (int sl = lo_s; sl < hi_s; ++sl)
                vb[kv_v_off(sl, i, q.hd)] = f32_to_bf16(src[(sl - lo_s) * LDF]);
            }
          }
        }
      }
    }
  }
}

template <int NBH>
static hipError_t launch_wide_nbh(const GemmArgs& g, dim3 grid, hipStream_t s) {
  if constexpr (NBH == 3) {       // narrow tiles: QKV and gate/up only
    if (g.epi == EPI_QKV) hipLaunchKernelGGL((gemm_wide_kernel<3, EPI_QKV>), grid, dim3(512), 0, s, g);
    else if (g.epi == EPI_SWIGLU)
      hipLaunchKernelGGL((gemm_wide_kernel<3, EPI_SWIGLU>), grid, dim3(512), 0, s, g);
    else return hipErrorInvalidValue;
  } else {
    switch (g.epi) {
      case EPI_SWIGLU:
        hipLaunchKernelGGL((gemm_wide_kernel<NBH, EPI_SWIGLU>), grid, dim3(512), 0, s, g);
        break;
      case EPI_STORE:
        if (NBH != 4) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_wide_kernel<4, EPI_STORE>), grid, dim3(512), 0, s, g);
        break;
      case EPI_ADD:
        if (NBH != 4) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_wide_kernel<4, EPI_ADD>), grid, dim3(512), 0, s, g);
        break;
      case EPI_QKV:
        if (NBH != 4) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_wide_kernel<4, EPI_QKV>), grid, dim3(512), 0, s, g);
        break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

int gemm_wide_ntiles(int epi, int N, int nbh) {
  const int blocks = N / 16;
  const int per_tile = epi == EPI_SWIGLU ? nbh : 2 * nbh;
  return (blocks + per_tile - 1) / per_tile;
}

int gemm_ntiles(int epi, int N, int w, int nbw) {
  const int blocks = N / 16;
  const int per_tile = epi == EPI_SWIGLU ? (nbw == 2 ? w : w / 2) : w * nbw;
  return (blocks + per_tile - 1) / per_tile;
}

int gemm_mb(int Mp) {
  const int rb = Mp / 16;
  return rb <= 1 ? 1 : rb <= 2 ? 2 : rb <= 4 ? 4 : rb <= 8 ? 8 : 16;
}

template <int MB, int W, int NBW>
static hipError_t launch_mb(const GemmArgs& g, dim3 grid, hipStream_t s) {
  const dim3 blk(W * 64);
  if constexpr (NBW == 1 && W == 8) {            // 8-wave tiles: LM head; gate/up of wide tiles
    if (g.epi == EPI_STORE) hipLaunchKernelGGL((gemm_kernel<MB, 8, 1, EPI_STORE>), grid, blk, 0, s, g);
    else if (MB >= 8 && g.epi == EPI_SWIGLU)
      hipLaunchKernelGGL((gemm_kernel<(MB >= 8 ? MB : 8), 8, 1, EPI_SWIGLU>), grid, blk, 0, s, g);
    else if (MB >= 8 && g.epi == EPI_QKV)
      hipLaunchKernelGGL((gemm_kernel<(MB >= 8 ? MB : 8), 8, 1, EPI_QKV>), grid, blk, 0, s, g);
    else return hipErrorInvalidValue;
  } else if constexpr (NBW == 1 && W == 10) {    // gate/up of wide tiles, 5 features blocks a tile
    if (MB >= 8 && g.epi == EPI_SWIGLU)
      hipLaunchKernelGGL((gemm_kernel<(MB >= 8 ? MB : 8), 10, 1, EPI_SWIGLU>), grid, blk, 0, s, g);
    else return hipErrorInvalidValue;
  } else if constexpr (NBW == 1) {
    if (g.epi == EPI_STORE) hipLaunchKernelGGL((gemm_kernel<MB, W, 1, EPI_STORE>), grid, blk, 0, s, g);
    else if (g.epi == EPI_ADD) hipLaunchKernelGGL((gemm_kernel<MB, W, 1, EPI_ADD>), grid, blk, 0, s, g);
    else if (MB <= 4 && g.epi == EPI_QKV)        // 64-column QKV tiles, RoPE partners in wave pairs
      hipLaunchKernelGGL((gemm_kernel<(MB <= 4 ? MB : 4), W, 1, EPI_QKV>), grid, blk, 0, s, g);
    else return hipErrorInvalidValue;
  } else {
    if (g.epi == EPI_SWIGLU) hipLaunchKernelGGL((gemm_kernel<MB, W, 2, EPI_SWIGLU>), grid, blk, 0, s, g);
    else if (g.epi == EPI_QKV) hipLaunchKernelGGL((gemm_kernel<MB, W, 2, EPI_QKV>), grid, blk, 0, s, g);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int W, int NBW>
static hipError_t launch_w(const GemmArgs& g, int MB, dim3 grid, hipStream_t s) {
  switch (MB) {
    case 1: return launch_mb<1, W, NBW>(g, grid, s);
    case 2: return launch_mb<2, W, NBW>(g, grid, s);
    case 4: return launch_mb<4, W, NBW>(g, grid, s);
    case 8: return launch_mb<8, W, NBW>(g, grid, s);
    case 16: return launch_mb<16, W, NBW>(g, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.wide) {
    const dim3 grid(gemm_wide_ntiles(g.epi, g.N, g.wide), g.splits, (g.Mp + WIDE_TR - 1) / WIDE_TR);
    if (g.wide == 4) return launch_wide_nbh<4>(g, grid, s);
    if (g.wide == 5 && g.epi == EPI_SWIGLU) return launch_wide_nbh<5>(g, grid, s);
    if (g.wide == 3) return launch_wide_nbh<3>(g, grid, s);
    return hipErrorInvalidValue;
  }
  const int MB = gemm_mb(g.Mp);
  const int mtiles = (g.Mp / 16 + MB - 1) / MB;
  const int ntiles = gemm_ntiles(g.epi, g.N, g.w, g.nbw);
  const dim3 grid(ntiles + (g.epi == EPI_QKV ? g.prefetch : 0), g.splits, mtiles);
  if (g.w == 4 && g.nbw == 1) return launch_w<4, 1>(g, MB, grid, s);
  if (g.w == 8 && g.nbw == 1) return launch_w<8, 1>(g, MB, grid, s);
  if (g.w == 10 && g.nbw == 1) return launch_w<10, 1>(g, MB, grid, s);
  if (g.w == 4 && g.nbw == 2) return launch_w<4, 2>(g, MB, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace mvk
