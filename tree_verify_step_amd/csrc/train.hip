// Medusa-1 head training step on a frozen backbone (Medusa paper digest,
// Method 6, eq. 1; lecture note 二.1): for heads k = 1..K over N positions,
//   a = H W1_k^T,  s = SiLU(a) + H,  z = s W2_k^T,
//   loss = sum_t -lambda_k log softmax(z_t)[y_t],
// and the gradients through the same steps:
//   g = lambda_k (softmax(z) - onehot(y))        (bf16, the GEMM operand)
//   dW2_k = g^T s,  ds = g W2_k,  da = ds * SiLU'(a),  dW1_k = da^T H.
// These are dense contractions (2 N V d flops each for z, dW2 and ds), so
// they run on one MFMA GEMM, C = A B^T with both operands row-major and
// K-contiguous; the other orientations go through a transpose kernel first
// (memory-bound, a small share of the time).  Element-wise steps and the
// row-wise cross-entropy are kernels of their own.
#include "common.hpp"

#include <algorithm>

namespace mvk {

// ---------------------------------------------------------------------------
// C[M][N] (fp32, ldc) = A[M][K] (bf16, lda) * B[N][K]^T (bf16, ldb), batched
// over blockIdx.y with element strides sa, sb, sc.  K % 64 == 0; lda, ldb %
// 8 == 0.  128 x 128 tiles, 64-deep K chunks staged in LDS (double-buffered,
// the next chunk's global loads in flight while the current one is used);
// four waves, each a 64 x 64 quarter: 4 x 4 v_mfma_f32_16x16x32_bf16 blocks.
// Tiles are ordered in groups of 8 row tiles (each group walks all column
// tiles), and each XCD takes a contiguous run of tiles, so the operands'
// tiles are reused from L2.
// ---------------------------------------------------------------------------
constexpr int TG_BM = 128, TG_BN = 128, TG_BK = 64, TG_LD = TG_BK + 8;   // LDS row: 144 bytes

__global__ __launch_bounds__(256) void gemm_nt_kernel(const u16* __restrict__ A, int lda, size_t sa,
                                                      const u16* __restrict__ B, int ldb, size_t sb,
                                                      float* __restrict__ C, int ldc, size_t sc,
                                                      int M, int N, int K) {
  __shared__ __align__(16) u16 As[2][TG_BM * TG_LD];
  __shared__ __align__(16) u16 Bs[2][TG_BN * TG_LD];
  const int tiles_m = (M + TG_BM - 1) / TG_BM, tiles_n = (N + TG_BN - 1) / TG_BN;
  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) / 8;
  const int t = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (t >= tiles) return;
  constexpr int GM = 8;                                   // row tiles per group
  const int in_group = GM * tiles_n;
  const int first_m = (t / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int mt = first_m + (t % in_group) % gsize, nt = (t % in_group) / gsize;
  A += sa * blockIdx.y;
  B += sb * blockIdx.y;
  C += sc * blockIdx.y;
  const int m0 = mt * TG_BM, n0 = nt * TG_BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, c = lane >> 4;

  // staging: 1024 16-byte pieces of each operand chunk, four per thread
  // (thread tid takes rows tid/8 + 32 i, 8 columns at (tid % 8) * 8)
  const int srow = tid >> 3, skc = (tid & 7) * 8;
  const u16* ap[4];
  const u16* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ap[i] = A + (size_t)min(m0 + srow + 32 * i, M - 1) * lda + skc;
    bp[i] = B + (size_t)min(n0 + srow + 32 * i, N - 1) * ldb + skc;
  }
  bf16x8 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define MV_TG_LOAD(k0)                                              \
  do {                                                              \
    ra0 = *reinterpret_cast<const bf16x8*>(ap[0] + (k0));           \
    ra1 = *reinterpret_cast<const bf16x8*>(ap[1] + (k0));           \
    ra2 = *reinterpret_cast<const bf16x8*>(ap[2] + (k0));           \
    ra3 = *reinterpret_cast<const bf16x8*>(ap[3] + (k0));           \
    rb0 = *reinterpret_cast<const bf16x8*>(bp[0] + (k0));           \
    rb1 = *reinterpret_cast<const bf16x8*>(bp[1] + (k0));           \
    rb2 = *reinterpret_cast<const bf16x8*>(bp[2] + (k0));           \
    rb3 = *reinterpret_cast<const bf16x8*>(bp[3] + (k0));           \
  } while (0)
#define MV_TG_STORE(buf)                                                            \
  do {                                                                              \
    *reinterpret_cast<bf16x8*>(&As[buf][(srow + 0) * TG_LD + skc]) = ra0;           \
    *reinterpret_cast<bf16x8*>(&As[buf][(srow + 32) * TG_LD + skc]) = ra1;          \
    *reinterpret_cast<bf16x8*>(&As[buf][(srow + 64) * TG_LD + skc]) = ra2;          \
    *reinterpret_cast<bf16x8*>(&As[buf][(srow + 96) * TG_LD + skc]) = ra3;          \
    *reinterpret_cast<bf16x8*>(&Bs[buf][(srow + 0) * TG_LD + skc]) = rb0;           \
    *reinterpret_cast<bf16x8*>(&Bs[buf][(srow + 32) * TG_LD + skc]) = rb1;          \
    *reinterpret_cast<bf16x8*>(&Bs[buf][(srow + 64) * TG_LD + skc]) = rb2;          \
    *reinterpret_cast<bf16x8*>(&Bs[buf][(srow + 96) * TG_LD + skc]) = rb3;          \
  } while (0)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = K / TG_BK;
  MV_TG_LOAD(0);
  MV_TG_STORE(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) MV_TG_LOAD((kt + 1) * TG_BK);
#pragma unroll
    for (int ks = 0; ks < TG_BK / 32; ++ks) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 64 + i * 16 + r) * TG_LD + ks * 32 + 8 * c]);
        b[i] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * 64 + i * 16 + r) * TG_LD + ks * 32 + 8 * c]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < KT) MV_TG_STORE(buf ^ 1);
    __syncthreads();
  }
#undef MV_TG_LOAD
#undef MV_TG_STORE
  // lane holds rows 4c .. 4c+3 of each 16 x 16 block, column r
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + r;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 64 + i * 16 + 4 * c + e;
        if (row < M) C[(size_t)row * ldc + col] = acc[i][j][e];
      }
    }
}

// The same product in 256 x 256 tiles, for launches with enough of them to
// fill the chip.  Eight waves, two a SIMD, each a 128 x 64 part (8 x 4
// blocks, 128 accumulators): a fragment read from LDS feeds 4 or 8 MFMAs,
// against 4 in the 128 x 128 tiles above, whose LDS reads bound them.  Per
// 64-deep chunk a workgroup copies 64 KiB into LDS and its waves read
// 192 KiB, against 8.4 MFLOP of matrix work.
//  - The chunks go global -> LDS directly (no registers), one 1 KiB run of
//    LDS per instruction: 8 rows of 64 bf16, whose eight 16-byte pieces sit
//    at position (piece ^ row) & 7, so that the eight rows a fragment read
//    touches in one pass fall in distinct banks.  Raw buffer loads: rows
//    past the matrix are past the buffer and read zeros (never stored).
//  - Two named buffers per operand, so that the compiler sees that reads of
//    one need not wait for the copies into the other; the chunk loop takes
//    two chunks a turn, copying chunk k + 1 while chunk k is multiplied, with
//    one barrier a chunk.
// Measured at the 7B head shapes: about 495 us for a 2048 x 32000 x 4096
// product (44% of the bf16 peak), against 700 us in 128 x 128 tiles.
constexpr int TB_BM = 256, TB_BK = 64;
constexpr int MV_BUF_RAW = 0x00020000;   // buffer resource word 3: raw (untyped) access

__global__ __launch_bounds__(512) void gemm_nt_big_kernel(const u16* __restrict__ A, int lda,
                                                          size_t sa, const u16* __restrict__ B,
                                                          int ldb, size_t sb, float* __restrict__ C,
                                                          int ldc, size_t sc, int M, int N, int K) {
  __shared__ __align__(16) u16 As0[TB_BM * TB_BK];
  __shared__ __align__(16) u16 As1[TB_BM * TB_BK];
  __shared__ __align__(16) u16 Bs0[TB_BM * TB_BK];
  __shared__ __align__(16) u16 Bs1[TB_BM * TB_BK];
  const int tiles_m = (M + TB_BM - 1) / TB_BM, tiles_n = (N + TB_BM - 1) / TB_BM;
  const int tiles = tiles_m * tiles_n;
  const int per = (tiles + 7) / 8;
  const int t = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (t >= tiles) return;
  constexpr int GM = 8;                                   // row tiles per group
  const int in_group = GM * tiles_n;
  const int first_m = (t / in_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int mt = first_m + (t % in_group) % gsize, nt = (t % in_group) / gsize;
  A += sa * blockIdx.y;
  B += sb * blockIdx.y;
  C += sc * blockIdx.y;
  const int m0 = mt * TB_BM, n0 = nt * TB_BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 15, c = lane >> 4;

  // copies: wave w's instruction i fills LDS rows 8 (4w + i) .. +7 of an
  // operand chunk; lane L takes row + L/8 and the piece stored at position
  // L % 8
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(A), (short)0, (int)((size_t)M * lda * 2), MV_BUF_RAW);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(B), (short)0, (int)((size_t)N * ldb * 2), MV_BUF_RAW);
  const int lrow = lane >> 3, lpiece = ((lane & 7) ^ lrow) * 8;
  uint32_t va[4], vb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (wave * 4 + i) * 8 + lrow;
    va[i] = ((uint32_t)(m0 + row) * (uint32_t)lda + lpiece) * 2u;
    vb[i] = ((uint32_t)(n0 + row) * (uint32_t)ldb + lpiece) * 2u;
  }
  auto copy = [&](u16* as, u16* bs, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, as + (wave * 4 + i) * 512, 16, va[i], k0 * 2, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, bs + (wave * 4 + i) * 512, 16, vb[i], k0 * 2, 0, 0);
    }
  };
  // fragment i of half ks: rows 16 i + r of the wave's part, 8 k at piece
  // q = 4 ks + c, stored at position (q ^ row) & 7 = (q ^ r) & 7
  int fo_a[2], fo_b[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    fo_a[ks] = (wm * 128 + r) * TB_BK + (((ks * 4 + c) ^ r) & 7) * 8;
    fo_b[ks] = (wn * 64 + r) * TB_BK + (((ks * 4 + c) ^ r) & 7) * 8;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Fragment reads run ahead of the MFMAs that use them, in a pinned order
  // (left to itself the scheduler waits for each read just before its row):
  // a chunk starts with the first half's four B fragments and first two A
  // fragments; each row of 4 MFMAs is followed by the read of the A fragment
  // two rows ahead; the last two rows of the first half are followed by the
  // second half's B fragments (a second set) and first A fragments.
  auto chunk = [&](const u16* as, const u16* bs) {
    bf16x8 a[8], b0[4], b1[4];
    auto ra = [&](int ks, int i) {
      a[i] = *reinterpret_cast<const bf16x8*>(as + fo_a[ks] + i * 16 * TB_BK);
    };
    auto rb = [&](int ks, bf16x8 (&b)[4], int j) {
      b[j] = *reinterpret_cast<const bf16x8*>(bs + fo_b[ks] + j * 16 * TB_BK);
    };
    auto row = [&](const bf16x8 (&b)[4], int i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) rb(0, b0, j);
    ra(0, 0);
    ra(0, 1);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      row(b0, i);
      ra(0, i + 2);
    }
    row(b0, 6);
    rb(1, b1, 0);
    rb(1, b1, 1);
    ra(1, 0);
    row(b0, 7);
    rb(1, b1, 2);
    rb(1, b1, 3);
    ra(1, 1);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      row(b1, i);
      ra(1, i + 2);
    }
    row(b1, 6);
    row(b1, 7);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // chunk kt lives in buffers kt & 1 (the launcher asks for an even count)
  const int KT = K / TB_BK;
  copy(As0, Bs0, 0);
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < KT; kt += 2) {
    copy(As1, Bs1, (kt + 1) * TB_BK);
    chunk(As0, Bs0);
    __syncthreads();
    if (kt + 2 < KT) copy(As0, Bs0, (kt + 2) * TB_BK);
    chunk(As1, Bs1);
    __syncthreads();
  }
  // lane holds rows 4c .. 4c+3 of each 16 x 16 block, column r
  float* cw = C + (size_t)(m0 + wm * 128 + 4 * c) * ldc + n0 + wn * 64 + r;
  if (m0 + TB_BM <= M && n0 + TB_BM <= N) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) cw[(size_t)(i * 16 + e) * ldc + j * 16] = acc[i][j][e];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * 128 + i * 16 + 4 * c + e;
          const int col = n0 + wn * 64 + j * 16 + r;
          if (row < M && col < N) cw[(size_t)(i * 16 + e) * ldc + j * 16] = acc[i][j][e];
        }
  }
}

hipError_t launch_gemm_nt(const u16* A, int lda, size_t sa, const u16* B, int ldb, size_t sb,
                          float* C, int ldc, size_t sc, int M, int N, int K, int batch,
                          hipStream_t s) {
  if (M < 1 || N < 1 || K < TG_BK || K % TG_BK || lda % 8 || ldb % 8 || batch < 1)
    return hipErrorInvalidValue;
  // 256 x 256 tiles when there are about enough of them for one round over
  // the compute units, else 128 x 128
  const int big = ((M + TB_BM - 1) / TB_BM) * ((N + TB_BM - 1) / TB_BM);
  // the copies' byte offsets (rows up to a tile past the matrix) fit 31 bits
  const bool off31 = (uint64_t)(M + TB_BM) * lda * 2 < (1ull << 31) &&
                     (uint64_t)(N + TB_BM) * ldb * 2 < (1ull << 31);
  if (big * batch >= 240 && off31 && K % (2 * TB_BK) == 0) {
    hipLaunchKernelGGL(gemm_nt_big_kernel, dim3(8 * ((big + 7) / 8), batch), dim3(512), 0, s, A,
                       lda, sa, B, ldb, sb, C, ldc, sc, M, N, K);
    return hipGetLastError();
  }
  const int tiles = ((M + TG_BM - 1) / TG_BM) * ((N + TG_BN - 1) / TG_BN);
  hipLaunchKernelGGL(gemm_nt_kernel, dim3(8 * ((tiles + 7) / 8), batch), dim3(256), 0, s, A, lda,
                     sa, B, ldb, sb, C, ldc, sc, M, N, K);
  return hipGetLastError();
}

// C = sum over s of P[s] (fp32 [S][n], n % 4 == 0), in split order.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ P, int S,
                                                         size_t n, float* __restrict__ C) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 v = *reinterpret_cast<const float4*>(P + i);
  for (int sp = 1; sp < S; ++sp) {
    const float4 w = *reinterpret_cast<const float4*>(P + sp * n + i);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  *reinterpret_cast<float4*>(C + i) = v;
}

// C[M][N] (ldc = N) = A B^T for products with few 256 x 256 tiles and a long
// K: the K range is split S ways (S tiles-rounds of the chip at most one,
// each split a multiple of 128 deep), the splits' products go to `part`
// (S M N floats available) and a second launch sums them in split order.
// Falls back to the single launch when no split applies.
hipError_t launch_gemm_nt_splitk(const u16* A, int lda, const u16* B, int ldb, float* C, int M,
                                 int N, int K, float* part, size_t part_elems, hipStream_t s) {
  const int big = ((M + TB_BM - 1) / TB_BM) * ((N + TB_BM - 1) / TB_BM);
  const size_t mn = (size_t)M * N;
  int S = std::max(1, std::min(8, 256 / std::max(big, 1)));
  while (S > 1 && (K % (S * 2 * TB_BK) != 0 || (size_t)S * mn > part_elems || big * S < 240)) --S;
  const bool off31 = (uint64_t)(M + TB_BM) * lda * 2 < (1ull << 31) &&
                     (uint64_t)(N + TB_BM) * ldb * 2 < (1ull << 31);
  if (S <= 1 || N % 4 || !off31) return launch_gemm_nt(A, lda, 0, B, ldb, 0, C, N, 0, M, N, K, 1, s);
  const int Ks = K / S;
  hipLaunchKernelGGL(gemm_nt_big_kernel, dim3(8 * ((big + 7) / 8), S), dim3(512), 0, s, A, lda,
                     (size_t)Ks, B, ldb, (size_t)Ks, part, N, mn, M, N, Ks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, s, part,
                     S, mn, C);
  return hipGetLastError();
}

// out[c][r] = in[r][c] for a bf16 [R][C] matrix (R, C % 64 == 0), batched
// over blockIdx.z; 64 x 64 tiles through LDS, 16-byte loads and stores.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const u16* __restrict__ in, size_t s_in,
                                                             u16* __restrict__ out, size_t s_out,
                                                             int R, int Cc) {
  __shared__ u16 tl[64][64 + 2];
  in += s_in * blockIdx.z;
  out += s_out * blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i, rr = q >> 3, cc = (q & 7) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(in + (size_t)(r0 + rr) * Cc + c0 + cc);
    const u16* e = reinterpret_cast<const u16*>(&v);
#pragma unroll
    for (int j = 0; j < 8; ++j) tl[rr][cc + j] = e[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i, cc = q >> 3, rr = (q & 7) * 8;
    u16 e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = tl[rr + j][cc];
    *reinterpret_cast<uint4*>(out + (size_t)(c0 + cc) * R + r0 + rr) = *reinterpret_cast<const uint4*>(e);
  }
}

hipError_t launch_transpose_bf16(const u16* in, size_t s_in, u16* out, size_t s_out, int R, int C,
                                 int batch, hipStream_t s) {
  if (R % 64 || C % 64 || R < 64 || C < 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(C / 64, R / 64, batch), dim3(256), 0, s, in, s_in,
                     out, s_out, R, C);
  return hipGetLastError();
}

// s = bf16(SiLU(a) + h) over n elements (a fp32, h bf16), 8 per thread.
__global__ void medusa1_act_kernel(const float* __restrict__ a, const u16* __restrict__ h,
                                   u16* __restrict__ s, size_t n8) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 a0 = reinterpret_cast<const float4*>(a)[2 * i];
    const float4 a1 = reinterpret_cast<const float4*>(a)[2 * i + 1];
    const uint4 hv = reinterpret_cast<const uint4*>(h)[i];
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = silu_f(av[2 * j]) + bf16lo(hw[j]);
      const float hi = silu_f(av[2 * j + 1]) + bf16hi(hw[j]);
      o[j] = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
    }
    reinterpret_cast<uint4*>(s)[i] = uint4{o[0], o[1], o[2], o[3]};
  }
}

// da = bf16(ds * SiLU'(a)), SiLU'(a) = sigma(a) (1 + a (1 - sigma(a))).
__global__ void medusa1_dact_kernel(const float* __restrict__ ds, const float* __restrict__ a,
                                    u16* __restrict__ da, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x) {
    const float4 g = reinterpret_cast<const float4*>(ds)[i];
    const float4 x = reinterpret_cast<const float4*>(a)[i];
    const float gv[4] = {g.x, g.y, g.z, g.w}, xv[4] = {x.x, x.y, x.z, x.w};
    float o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sg = 1.0f / (1.0f + __expf(-xv[j]));
      o[j] = gv[j] * sg * (1.0f + xv[j] * (1.0f - sg));
    }
    reinterpret_cast<uint2*>(da)[i] =
        uint2{(uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16),
              (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16)};
  }
}

// One workgroup per position t of head k: the row's log-sum-exp (fp64
// sums), loss_tk[t][k] = lambda (lse - z[y]) and the logits' gradient row
// g = bf16(lambda (exp(z - lse) - [v == y])); rows without a label (y < 0
// or y >= V) give 0.
__global__ __launch_bounds__(256) void medusa1_ce_kernel(const float* __restrict__ z,
                                                         const int32_t* __restrict__ labels,
                                                         int ldl, int k, float lambda, int V,
                                                         float* __restrict__ loss_tk,
                                                         u16* __restrict__ g) {
  __shared__ double red[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* zr = z + (size_t)t * V;
  u16* gr = g + (size_t)t * V;
  const int y = labels[(size_t)t * ldl + k];
  const bool lab = y >= 0 && y < V;
  float mx = -INFINITY;
  for (int i = tid * 4; i < V; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(zr + i);
    mx = fmaxf(mx, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  mx = warp_max(mx);
  __shared__ float rmax[4];
  if (lane == 0) rmax[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(rmax[0], rmax[1]), fmaxf(rmax[2], rmax[3]));
  double sum = 0.0;
  for (int i = tid * 4; i < V; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(zr + i);
    sum += (double)__expf(v.x - mx) + (double)__expf(v.y - mx) + (double)__expf(v.z - mx) +
           (double)__expf(v.w - mx);
  }
  sum = warp_sum_d(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  const double S = (red[0] + red[1]) + (red[2] + red[3]);
  const float lse = mx + (float)log(S);
  if (tid == 0) loss_tk[(size_t)t * ldl + k] = lab ? lambda * (lse - zr[y]) : 0.f;
  for (int i = tid * 4; i < V; i += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(zr + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
    u16 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __expf(vv[j] - lse);
      o[j] = lab ? f32_to_bf16(lambda * (p - (i + j == y ? 1.f : 0.f))) : (u16)0;
    }
    *reinterpret_cast<uint2*>(gr + i) = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                              (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
  }
}

// The same for rows of at most NT * J * 4 logits, each read once: thread
// tid holds float4 pieces tid + j NT (j < J) in registers through the max,
// the sum and the gradient passes (the looping form reads the row three
// times).
template <int NT, int J>
__global__ __launch_bounds__(NT) void medusa1_ce_regs_kernel(const float* __restrict__ z,
                                                             const int32_t* __restrict__ labels,
                                                             int ldl, int k, float lambda, int V,
                                                             float* __restrict__ loss_tk,
                                                             u16* __restrict__ g) {
  constexpr int NW = NT / 64;
  __shared__ float rmax[NW];
  __shared__ double red[NW];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* zr = z + (size_t)t * V;
  u16* gr = g + (size_t)t * V;
  const int y = labels[(size_t)t * ldl + k];
  const bool lab = y >= 0 && y < V;
  const int V4 = V >> 2;
  float4 v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = tid + j * NT;
    v[j] = i < V4 ? reinterpret_cast<const float4*>(zr)[i]
                  : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < J; ++j) mx = fmaxf(mx, fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w)));
  mx = warp_max(mx);
  if (lane == 0) rmax[wave] = mx;
  __syncthreads();
  mx = rmax[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, rmax[w]);
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j)
    sum += (double)__expf(v[j].x - mx) + (double)__expf(v[j].y - mx) +
           (double)__expf(v[j].z - mx) + (double)__expf(v[j].w - mx);
  sum = warp_sum_d(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  double S = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) S += red[w];
  const float lse = mx + (float)log(S);
  if (tid == 0) loss_tk[(size_t)t * ldl + k] = lab ? lambda * (lse - zr[y]) : 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i4 = tid + j * NT;
    if (i4 >= V4) continue;
    const float vv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
    u16 o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = __expf(vv[e] - lse);
      o[e] = lab ? f32_to_bf16(lambda * (p - (i4 * 4 + e == y ? 1.f : 0.f))) : (u16)0;
    }
    *reinterpret_cast<uint2*>(gr + i4 * 4) = uint2{(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                   (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
  }
}

// loss = sum of loss_tk [n] in a fixed order (one workgroup, fp64).
__global__ __launch_bounds__(256) void medusa1_sum_kernel(const float* __restrict__ v, int n,
                                                          double* __restrict__ out) {
  __shared__ double red[4];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += (double)v[i];
  s = warp_sum_d(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) *out = (red[0] + red[1]) + (red[2] + red[3]);
}

static int ew_blocks(size_t n) {
  return (int)std::min<size_t>((n + 255) / 256, 8192);
}

hipError_t launch_medusa1_act(const float* a, const u16* h, u16* s, size_t n, hipStream_t st) {
  hipLaunchKernelGGL(medusa1_act_kernel, dim3(ew_blocks(n / 8)), dim3(256), 0, st, a, h, s, n / 8);
  return hipGetLastError();
}
hipError_t launch_medusa1_dact(const float* ds, const float* a, u16* da, size_t n, hipStream_t st) {
  hipLaunchKernelGGL(medusa1_dact_kernel, dim3(ew_blocks(n / 4)), dim3(256), 0, st, ds, a, da, n / 4);
  return hipGetLastError();
}
hipError_t launch_medusa1_ce(const float* z, const int32_t* labels, int ldl, int k, float lambda,
                             int N, int V, float* loss_tk, u16* g, hipStream_t st) {
  if (V / 4 <= 1024 * 8)
    hipLaunchKernelGGL((medusa1_ce_regs_kernel<1024, 8>), dim3(N), dim3(1024), 0, st, z, labels, ldl,
                       k, lambda, V, loss_tk, g);
  else
    hipLaunchKernelGGL(medusa1_ce_kernel, dim3(N), dim3(256), 0, st, z, labels, ldl, k, lambda, V,
                       loss_tk, g);
  return hipGetLastError();
}
hipError_t launch_medusa1_sum(const float* v, int n, double* out, hipStream_t st) {
  hipLaunchKernelGGL(medusa1_sum_kernel, dim3(1), dim3(256), 0, st, v, n, out);
  return hipGetLastError();
}

}  // namespace mvk
