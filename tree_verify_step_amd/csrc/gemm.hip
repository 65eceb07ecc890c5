// Skinny bf16 GEMM for the tree-verify forward: Y[M][N] = A[M][K] * W[N][K]^T
// with M = batch x tree nodes (16..256), N and K the model's widths.
//
// At M ~ 64 every weight byte is used 64 times, so the kernel is bound by
// streaming W from HBM once; the MFMA units (v_mfma_f32_16x16x32_bf16) only
// need to keep up.  Three measured choices shape it:
//  * Weights are fragment-packed k-block-major ([K/32][N/16][64 lanes][8]):
//    the 1 KiB operand blocks of all columns for one 32-wide k-block are
//    adjacent, and the 4 waves of a workgroup take interleaved k-blocks, so
//    the whole grid sweeps a dense window of memory (as a plain streaming
//    copy does) instead of thousands of streams at power-of-two strides that
//    alias onto few HBM channels.
//  * The main loop is a branch-free register pipeline (A and B fragments of
//    D k-blocks in flight); out-of-range stages are zeroed by selects, so the
//    compiler's wait counts stay partial.
//  * K is split over `splits` workgroups when the N tiles alone cannot fill
//    the chip.  Each split writes its partial tile with write-through
//    (system-scope) stores, waits for them, and bumps the tile's arrival
//    counter; the last workgroup to arrive reads the partials with
//    cache-bypassing loads, sums them in split order and applies the
//    epilogue: one kernel, a deterministic result, and no L2-wide
//    invalidation (which would evict the other workgroups' operands).
// Epilogues:
//   STORE   out = y                          (LM head logits)
//   ADD     out += y                         (residual stream: O-proj, down)
//   SWIGLU  tile = [gate cols | up cols]; h = SiLU(g) * u -> bf16 packed
//   QKV     RoPE on q, k at each row's position; q -> bf16 rows; k, v ->
//           KV cache slot n + node index
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

__device__ __forceinline__ int qkv_partner(int p, int f, int d, int hd, int P, bool perm) {
  if (f >= 2 * d) return p;
  if (perm) {
    const int ee = (p % hd) % (2 * P);
    return ee < P ? p + P : p - P;
  }
  const int i = (f % d) % hd;
  return i < hd / 2 ? p + hd / 2 : p - hd / 2;
}

// QKV epilogue of one element (row m, logical feature f) with RoPE partner yp.
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

// Split-K partial exchange between workgroups that may sit on different
// XCDs (separate L2s): system-scope stores (written through to memory) and
// 16-byte vector loads that bypass the caches (system-coherent sc0 sc1).
// The compiler waits for every system-scope atomic load on its own, which
// serialises them; these loads are issued as a batch and waited for once
// (the compiler does not track inline-asm loads, hence the explicit vmcnt
// wait).  Stores stay compiler-generated so that its hazard checks (store
// data registers rewritten right after issue) still apply.
__device__ __forceinline__ void store_sys(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ f32x4 load_nc16(const float* p) {
  f32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off sc0 sc1" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Orders a register's later uses after the preceding wait_vmem().
__device__ __forceinline__ void after_wait(f32x4& v) { asm volatile("" : "+v"(v)); }

template <int MB, int NBW, int D, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int TM = MB * 16, TN = NBW * 16, LDT = TN + 1;
  __shared__ float red[TM * LDT];
  __shared__ int s_last;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mt = blockIdx.x, nt = blockIdx.y, split = blockIdx.z;
  const int KB = g.K >> 5;
  const int kb_lo = (int)((long long)KB * split / g.splits);
  const int kb_hi = (int)((long long)KB * (split + 1) / g.splits);
  const int first = kb_lo + wave;
  const int count = first < kb_hi ? (kb_hi - first + 3) / 4 : 0;
  const int rounds = (count + D - 1) / D;

  // B block (kb, nb) at (kb * NBtot + nb) * 64 + lane
  const int NBtot = g.N >> 4;
  const bf16x8* Wg = reinterpret_cast<const bf16x8*>(g.W) + lane;
  const bf16x8* Wu = reinterpret_cast<const bf16x8*>(g.W2) + lane;
  const int nb0 = EPI == EPI_SWIGLU ? nt * (NBW / 2) : nt * NBW;   // gate/up share row blocks
  // A block (rb, kb) at (rb * KB + kb) * 64 + lane (rows beyond M are zeros)
  const bf16x8* Ap = reinterpret_cast<const bf16x8*>(g.A) + lane;
  const int MBtot = g.Mp >> 4;

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 ab[D][MB], bb[D][NBW];
  auto load = [&](int d, int j) {      // this wave's j-th k-block into stage d
    const int k = min(first + 4 * j, kb_hi - 1);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      if (EPI == EPI_SWIGLU) {
        const bf16x8* base = nb < NBW / 2 ? Wg : Wu;
        bb[d][nb] = base[((size_t)k * NBtot + nb0 + (nb % (NBW / 2))) * 64];
      } else {
        bb[d][nb] = Wg[((size_t)k * NBtot + nb0 + nb) * 64];
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int rb = min(mt * MB + mb, MBtot - 1);
      ab[d][mb] = Ap[((size_t)rb * KB + k) * 64];
    }
  };

  if (count > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) load(d, d);
  }
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const bool valid = r * D + d < count;
      bf16x8 av[MB], bv[NBW];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[mb] = valid ? ab[d][mb] : bf16x8{};
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) bv[nb] = bb[d][nb];
      load(d, r * D + d + D);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = mfma16x16x32(av[mb], bv[nb], acc[mb][nb]);
    }
  }

  // ---- sum the 4 waves' partial tiles in LDS (wave order: deterministic)
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* p = &red[(mb * 16 + (lane >> 4) * 4 + r) * LDT + nb * 16 + (lane & 15)];
            *p = (w == 0 ? 0.f : *p) + acc[mb][nb][r];
          }
    }
    __syncthreads();
  }

  // ---- split-K: the last workgroup of the tile sums the splits in order
  if (g.splits > 1) {
    constexpr int NQ = TM * TN / 4;            // float4 pieces per tile
    constexpr int Q = (NQ + 255) / 256;        // pieces per thread
    const int tile = mt * gridDim.y + nt;
    float* part = g.partial + (size_t)tile * g.splits * (TM * TN);
#pragma unroll
    for (int i = 0; i < Q; ++i) {
      const int e = (i * 256 + threadIdx.x) * 4, r = e / TN, c = e % TN;
      if (e < TM * TN) {
        const float* src = &red[r * LDT + c];
        float* dst = part + (size_t)split * (TM * TN) + e;
#pragma unroll
        for (int j = 0; j < 4; ++j) store_sys(dst + j, src[j]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);       // this thread's write-through stores are done
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(g.counters + tile, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == g.splits - 1;
    }
    __syncthreads();
    if (!s_last) return;
    for (int s0 = 0; s0 < g.splits; s0 += 4) {
      f32x4 v[4][Q];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < Q; ++i)
          if (s0 + s < g.splits && (i * 256 + threadIdx.x) < NQ)
            v[s][i] = load_nc16(part + (size_t)(s0 + s) * (TM * TN) + (i * 256 + threadIdx.x) * 4);
      wait_vmem();
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < Q; ++i)
          if (s0 + s < g.splits && (i * 256 + threadIdx.x) < NQ) after_wait(v[s][i]);
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const int e = (i * 256 + threadIdx.x) * 4, r = e / TN, c = e % TN;
        if (e >= TM * TN) continue;
        float* dst = &red[r * LDT + c];
        f32x4 y = s0 == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : f32x4{dst[0], dst[1], dst[2], dst[3]};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s0 + s < g.splits) {
            y += v[s][i];
          }
        dst[0] = y[0];
        dst[1] = y[1];
        dst[2] = y[2];
        dst[3] = y[3];
      }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(g.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }

  // ---- epilogues on the complete tile
  const int m0 = mt * TM;
  if (EPI == EPI_SWIGLU) {
    constexpr int P = TN / 2;
    for (int e = threadIdx.x; e < TM * P; e += 256) {
      const int r = e / P, c = e % P, m = m0 + r;
      if (m >= g.Mp) continue;
      const float gv = red[r * LDT + c], uv = red[r * LDT + c + P];
      const float h = m < g.M ? silu_f(gv) * uv : 0.f;
      g.out_bf16[packed_index(m, nt * P + c, g.N)] = f32_to_bf16(h);
    }
  } else if (EPI == EPI_STORE || EPI == EPI_ADD) {
    for (int e = threadIdx.x; e < TM * TN; e += 256) {
      const int r = e / TN, c = e % TN, m = m0 + r;
      if (m >= g.M) continue;
      float* o = g.out_f32 + (size_t)m * g.N + nt * TN + c;
      if (EPI == EPI_ADD) *o += red[r * LDT + c];
      else *o = red[r * LDT + c];
    }
  } else if (EPI == EPI_QKV) {
    const QkvArgs& q = g.qkv;
    const bool perm = 16 * NBW < q.hd;
    for (int e = threadIdx.x; e < TM * TN; e += 256) {
      const int r = e / TN, c = e % TN, m = m0 + r;
      if (m >= g.M) continue;
      const int n = nt * TN + c;
      const int f = qkv_feature(n, q.d, q.hd, TN / 2, perm);
      const int pc = qkv_partner(n, f, q.d, q.hd, TN / 2, perm) - nt * TN;
      qkv_store(q, m, f, red[r * LDT + c], red[r * LDT + pc]);
    }
  }
}

template <int MB, int NBW, int D>
static hipError_t launch_cfg(const GemmArgs& g, dim3 grid, hipStream_t s) {
  const dim3 blk(256);
  switch (g.epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<MB, NBW, D, EPI_STORE>), grid, blk, 0, s, g); break;
    case EPI_ADD: hipLaunchKernelGGL((gemm_kernel<MB, NBW, D, EPI_ADD>), grid, blk, 0, s, g); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<MB, NBW, D, EPI_SWIGLU>), grid, blk, 0, s, g); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<MB, NBW, D, EPI_QKV>), grid, blk, 0, s, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 16-row blocks per workgroup tile.
static int gemm_mb(int Mp) { return Mp <= 16 ? 1 : (Mp <= 32 ? 2 : 4); }

int gemm_tiles(const GemmArgs& g, int* mtiles, int* ntiles) {
  const int MB = gemm_mb(g.Mp);
  *mtiles = (g.Mp / 16 + MB - 1) / MB;
  *ntiles = g.epi == EPI_SWIGLU ? g.N / (g.nbw * 8) : g.N / (g.nbw * 16);
  return MB * 16 * g.nbw * 16;          // elements of one tile
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  int mtiles, ntiles;
  gemm_tiles(g, &mtiles, &ntiles);
  const int MB = gemm_mb(g.Mp);
  dim3 grid(mtiles, ntiles, g.splits);
  if (g.nbw == 4) {
    if (MB == 1) return launch_cfg<1, 4, 1>(g, grid, s);
    if (MB == 2) return launch_cfg<2, 4, 1>(g, grid, s);
    return launch_cfg<4, 4, 1>(g, grid, s);
  }
  if (g.nbw == 2) {
    if (MB == 1) return launch_cfg<1, 2, 4>(g, grid, s);
    if (MB == 2) return launch_cfg<2, 2, 4>(g, grid, s);
    return launch_cfg<4, 2, 4>(g, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mvk
