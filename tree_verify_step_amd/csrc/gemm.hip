// Skinny bf16 GEMM for the tree-verify forward: Y[M][N] = X[M][K] * W[N][K]^T
// with M = batch x tree nodes (16..256), N and K the model's widths.
//
// At M ~ 64 every weight byte is used 64 times, so the kernel is bound by
// streaming W from HBM once; the MFMA units (v_mfma_f32_16x16x32_bf16) only
// need to keep up.  Both operands are stored fragment-packed (see
// common.hpp), so every load is a coalesced 1 KiB block per wave.
//
// Work decomposition: a workgroup (4 waves) owns an N tile of NBW x 16
// columns, an M tile of MB x 16 rows and a contiguous range of the K blocks
// (K split over `splits` workgroups).  Its 4 waves split that K range four
// ways and stream their share with a two-stage register pipeline; the four
// partial tiles are summed through LDS and an epilogue is applied:
//   STORE   out = y                         (LM head logits)
//   ADD     out += y                        (residual stream, O-proj / down)
//   SWIGLU  h = SiLU(gate) * up -> bf16 packed activations of the down proj
//   QKV     RoPE(q), RoPE(k) at each row's position; q -> bf16 rows;
//           k, v -> the KV cache at slot n + node index
//   PARTIAL fp32 partial tile per K split (reduced by gemm_reduce_kernel,
//           which then applies STORE / ADD / SWIGLU / QKV).
#include "common.hpp"

namespace mvk {

// Logical output feature of packed weight row p of the fused QKV matrix.
// When a tile (16*NBW columns) is narrower than a head, q/k rows are
// permuted so that each tile holds P = 8*NBW first-half dims of one head and
// their RoPE partners (dim + hd/2); v rows are never permuted.
__host__ __device__ __forceinline__ int qkv_feature(int p, int d, int hd, int P, bool perm) {
  if (!perm || p >= 2 * d) return p;
  const int h = p / hd, e = p % hd, j = e / (2 * P), ee = e % (2 * P);
  return h * hd + (ee < P ? j * P + ee : hd / 2 + j * P + (ee - P));
}

struct EpiCtx {
  const GemmArgs* g;
};

// Column permutation flag of the QKV tile for a given NBW.
__host__ __device__ __forceinline__ bool qkv_perm(int NBW, int hd) { return 16 * NBW < hd; }

// Apply the QKV epilogue to one output element (row m, packed column p) whose
// value is y and whose RoPE partner value (packed column pp) is yp.
__device__ __forceinline__ void qkv_store(const QkvArgs& a, int m, int f, float y, float yp) {
  const int d = a.d, hd = a.hd;
  const int sec = f / d, c = f % d, h = c / hd, i = c % hd;
  const int b = m / a.T, v = m % a.T;
  float out = y;
  if (sec < 2) {
    const int half = hd >> 1;
    const float2 cs = a.rope[(size_t)m * half + (i % half)];
    out = (i < half) ? (y * cs.x - yp * cs.y) : (y * cs.x + yp * cs.y);
  }
  const u16 ob = f32_to_bf16(out);
  if (sec == 0) {
    a.q[(size_t)m * d + c] = ob;
  } else {
    // n + T <= cap is the caller's contract; clamping keeps every store in bounds
    const int n = min(max(a.n_prefix[b], 0), a.cap - a.T);
    const int slot = n + v;
    const size_t bh = (size_t)b * a.H + h;
    if (sec == 1) {
      a.kcache[(bh * a.cap + slot) * hd + i] = ob;
    } else {
      a.vcache[((bh * (a.cap >> 2) + (slot >> 2)) * hd + i) * 4 + (slot & 3)] = ob;
    }
  }
}

// Partner packed column of packed column p (global index) for RoPE.
__device__ __forceinline__ int qkv_partner(int p, int f, int d, int hd, int P, bool perm) {
  if (f >= 2 * d) return p;
  if (perm) {
    const int ee = (p % hd) % (2 * P);
    return ee < P ? p + P : p - P;
  }
  const int i = (f % d) % hd;
  return i < hd / 2 ? p + hd / 2 : p - hd / 2;
}

template <int MB, int NBW, int U, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int TM = MB * 16, TN = NBW * 16, LDT = TN + 1;
  __shared__ float red[4][TM * LDT];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mt = blockIdx.x, nt = blockIdx.y, split = blockIdx.z;
  const int KB = g.K >> 5;
  const int kb_lo = (int)((long long)KB * split / g.splits);
  const int kb_hi = (int)((long long)KB * (split + 1) / g.splits);
  const int len = kb_hi - kb_lo;
  const int w_lo = kb_lo + len * wave / 4, w_hi = kb_lo + len * (wave + 1) / 4;
  const int MBtot = g.Mp >> 4;

  const bf16x8* A = reinterpret_cast<const bf16x8*>(g.A);
  const bf16x8* Arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int rb = mt * MB + mb;
    rb = rb < MBtot ? rb : MBtot - 1;          // rows beyond M are ignored below
    Arow[mb] = A + (size_t)rb * KB * 64 + lane;
  }
  const bf16x8* Brow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const u16* base = g.W;
    int rb = nt * NBW + nb;
    if (EPI == EPI_SWIGLU) {
      // first half of the tile: gate rows, second half: the same up rows
      base = nb < NBW / 2 ? g.W : g.W2;
      rb = nt * (NBW / 2) + (nb % (NBW / 2));
    }
    Brow[nb] = reinterpret_cast<const bf16x8*>(base) + (size_t)rb * KB * 64 + lane;
  }

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 a0[U][MB], b0[U][NBW], a1[U][MB], b1[U][NBW];
  auto load = [&](bf16x8 (&a)[U][MB], bf16x8 (&b)[U][NBW], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + u < w_hi ? kb + u : w_hi - 1;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) b[u][nb] = Brow[nb][(size_t)k * 64];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) a[u][mb] = Arow[mb][(size_t)k * 64];
    }
  };
  auto mma = [&](bf16x8 (&a)[U][MB], bf16x8 (&b)[U][NBW], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb + u < w_hi) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = mfma16x16x32(a[u][mb], b[u][nb], acc[mb][nb]);
      }
    }
  };

  int kb = w_lo;
  if (kb < w_hi) load(a0, b0, kb);
  for (; kb + U < w_hi; kb += 2 * U) {
    load(a1, b1, kb + U);
    mma(a0, b0, kb);
    if (kb + 2 * U < w_hi) load(a0, b0, kb + 2 * U);
    mma(a1, b1, kb + U);
  }
  if (kb < w_hi) mma(a0, b0, kb);

  // Partial tiles of the 4 waves -> LDS (row-major, padded).
  float* my = red[wave];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        my[(mb * 16 + (lane >> 4) * 4 + r) * LDT + nb * 16 + (lane & 15)] = acc[mb][nb][r];
  __syncthreads();

  const int m0 = mt * TM;
  if (EPI == EPI_SWIGLU) {
    constexpr int P = TN / 2;
    for (int e = threadIdx.x; e < TM * P; e += 256) {
      const int r = e / P, c = e % P, m = m0 + r;
      if (m >= g.Mp) continue;
      float gv = 0.f, uv = 0.f;
      if (m < g.M) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gv += red[w][r * LDT + c];
          uv += red[w][r * LDT + c + P];
        }
      }
      const float h = m < g.M ? silu_f(gv) * uv : 0.f;
      g.out_bf16[packed_index(m, nt * P + c, g.N)] = f32_to_bf16(h);
    }
    return;
  }
  for (int e = threadIdx.x; e < TM * TN; e += 256) {
    const int r = e / TN, c = e % TN, m = m0 + r;
    if (m >= g.M) continue;
    const int n = nt * TN + c;
    float y = red[0][r * LDT + c] + red[1][r * LDT + c] + red[2][r * LDT + c] + red[3][r * LDT + c];
    if (EPI == EPI_STORE) {
      g.out_f32[(size_t)m * g.N + n] = y;
    } else if (EPI == EPI_ADD) {
      g.out_f32[(size_t)m * g.N + n] += y;
    } else if (EPI == EPI_PARTIAL) {
      g.partial[((size_t)split * g.M + m) * g.N + n] = y;
    } else if (EPI == EPI_QKV) {
      const QkvArgs& q = g.qkv;
      const bool perm = qkv_perm(NBW, q.hd);
      const int f = qkv_feature(n, q.d, q.hd, TN / 2, perm);
      const int pn = qkv_partner(n, f, q.d, q.hd, TN / 2, perm);
      const int pc = pn - nt * TN;
      const float yp = red[0][r * LDT + pc] + red[1][r * LDT + pc] + red[2][r * LDT + pc] +
                       red[3][r * LDT + pc];
      qkv_store(q, m, f, y, yp);
    }
  }
}

// Sums the K-split partials of a PARTIAL gemm and applies the final
// epilogue (g.epi).  One thread per output element (pairs for SWIGLU).
template <int NBW>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs g) {
  const int epi = g.epi;
  const size_t MN = (size_t)g.M * g.N;
  if (epi == EPI_SWIGLU) {
    // partial columns: tile t holds [gate P | up P], P = 8*NBW, for h cols t*P..
    constexpr int P = NBW * 8;
    const int F = g.N;                  // output columns
    const size_t total = (size_t)g.Mp * F;
    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
      const int m = (int)(e / F), j = (int)(e % F);
      float h = 0.f;
      if (m < g.M) {
        const int t = j / P, c = j % P;
        const size_t col_g = (size_t)t * 2 * P + c, col_u = col_g + P;
        float gv = 0.f, uv = 0.f;
        for (int s = 0; s < g.splits; ++s) {
          const float* ps = g.partial + (size_t)s * g.M * (2 * F) + (size_t)m * (2 * F);
          gv += ps[col_g];
          uv += ps[col_u];
        }
        h = silu_f(gv) * uv;
      }
      g.out_bf16[packed_index(m, j, F)] = f32_to_bf16(h);
    }
    return;
  }
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < MN; e += (size_t)gridDim.x * 256) {
    const int m = (int)(e / g.N), n = (int)(e % g.N);
    float y = 0.f;
    for (int s = 0; s < g.splits; ++s) y += g.partial[(size_t)s * MN + e];
    if (epi == EPI_STORE) {
      g.out_f32[e] = y;
    } else if (epi == EPI_ADD) {
      g.out_f32[e] += y;
    } else if (epi == EPI_QKV) {
      const QkvArgs& q = g.qkv;
      const bool perm = qkv_perm(NBW, q.hd);
      const int f = qkv_feature(n, q.d, q.hd, NBW * 8, perm);
      const int pn = qkv_partner(n, f, q.d, q.hd, NBW * 8, perm);
      float yp = 0.f;
      for (int s = 0; s < g.splits; ++s) yp += g.partial[(size_t)s * MN + (size_t)m * g.N + pn];
      qkv_store(q, m, f, y, yp);
    }
  }
}

template <int MB, int NBW, int U>
static hipError_t launch_mb(const GemmArgs& g, dim3 grid, hipStream_t s) {
  const int epi = g.splits > 1 ? EPI_PARTIAL : g.epi;
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<MB, NBW, U, EPI_STORE>), grid, dim3(256), 0, s, g); break;
    case EPI_ADD: hipLaunchKernelGGL((gemm_kernel<MB, NBW, U, EPI_ADD>), grid, dim3(256), 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<MB, NBW, U, EPI_SWIGLU>), grid, dim3(256), 0, s, g); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<MB, NBW, U, EPI_QKV>), grid, dim3(256), 0, s, g); break;
    default: hipLaunchKernelGGL((gemm_kernel<MB, NBW, U, EPI_PARTIAL>), grid, dim3(256), 0, s, g); break;
  }
  return hipGetLastError();
}

// Number of 16-row blocks per M tile.
static int gemm_mb(int Mp) { return Mp <= 16 ? 1 : (Mp <= 32 ? 2 : 4); }

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  constexpr int NBW = 4;
  const int MB = gemm_mb(g.Mp);
  const int mtiles = (g.Mp / 16 + MB - 1) / MB;
  // SWIGLU: N is the output width F; each tile produces 8*NBW columns
  // from gate and up rows.  PARTIAL for SWIGLU writes 2F interleaved columns.
  const int ncols = g.epi == EPI_SWIGLU ? g.N / (NBW * 8) : g.N / (NBW * 16);
  dim3 grid(mtiles, ncols, g.splits);
  GemmArgs a = g;
  if (g.epi == EPI_SWIGLU && g.splits > 1) a.N = 2 * g.N;   // partial row width
  if (MB == 1) return launch_mb<1, NBW, 2>(a, grid, s);
  if (MB == 2) return launch_mb<2, NBW, 2>(a, grid, s);
  return launch_mb<4, NBW, 1>(a, grid, s);
}

hipError_t launch_gemm_reduce(const GemmArgs& g, hipStream_t s) {
  const size_t total = g.epi == EPI_SWIGLU ? (size_t)g.Mp * g.N : (size_t)g.M * g.N;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL((gemm_reduce_kernel<4>), dim3(blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace mvk
