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

hipError_t launch_gemm_nt(const u16* A, int lda, size_t sa, const u16* B, int ldb, size_t sb,
                          float* C, int ldc, size_t sc, int M, int N, int K, int batch,
                          hipStream_t s) {
  if (M < 1 || N < 1 || K < TG_BK || K % TG_BK || lda % 8 || ldb % 8 || batch < 1)
    return hipErrorInvalidValue;
  const int tiles = ((M + TG_BM - 1) / TG_BM) * ((N + TG_BN - 1) / TG_BN);
  hipLaunchKernelGGL(gemm_nt_kernel, dim3(8 * ((tiles + 7) / 8), batch), dim3(256), 0, s, A, lda,
                     sa, B, ldb, sb, C, ldc, sc, M, N, K);
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
  hipLaunchKernelGGL(medusa1_ce_kernel, dim3(N), dim3(256), 0, st, z, labels, ldl, k, lambda, V,
                     loss_tk, g);
  return hipGetLastError();
}
hipError_t launch_medusa1_sum(const float* v, int n, double* out, hipStream_t st) {
  hipLaunchKernelGGL(medusa1_sum_kernel, dim3(1), dim3(256), 0, st, v, n, out);
  return hipGetLastError();
}

}  // namespace mvk
