// Row-wise kernels of the tree-verify forward: weight packing, embedding
// gather, RMSNorm into the packed GEMM operand, RoPE tables, KV compaction
// and small state updates.
#include "common.hpp"

namespace mvk {

__host__ __device__ __forceinline__ int qkv_feature_h(int p, int d, int hd, int P, bool perm) {
  if (!perm || p >= 2 * d) return p;
  const int h = p / hd, e = p % hd, j = e / (2 * P), ee = e % (2 * P);
  return h * hd + (ee < P ? j * P + ee : hd / 2 + j * P + (ee - P));
}

// dst (fragment-packed [R][C]) <- src (row-major [R][C]); when rope_hd > 0 the
// first rope_rows rows (q and k of a fused QKV matrix) are reordered so that
// each 64-row tile holds 32 first-half dims of a head and their RoPE partners
// (the order the QKV GEMM's epilogue expects when a tile is narrower than a
// head).  One thread per 16-byte piece.
__global__ void pack_kernel(const u16* __restrict__ src, u16* __restrict__ dst, int R, int C,
                            int rope_hd, int rope_rows) {
  const size_t pieces = (size_t)R * (C / 8);
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < pieces;
       e += (size_t)gridDim.x * blockDim.x) {
    const int p = (int)(e / (C / 8));            // packed row
    const int c = (int)(e % (C / 8)) * 8;
    int r = p;
    if (rope_hd > 0 && p < rope_rows) {
      const bool perm = 64 < rope_hd;             // tile width 64 narrower than a head
      r = qkv_feature_h(p, rope_rows / 2, rope_hd, 32, perm);
    }
    const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * C + c);
    *reinterpret_cast<uint4*>(dst + packed_index(p, c, C)) = v;
  }
}

hipError_t launch_pack(const u16* src, u16* dst, int R, int C, int rope_hd, int rope_rows,
                       hipStream_t s) {
  const size_t pieces = (size_t)R * (C / 8);
  int blocks = (int)((pieces + 255) / 256);
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, src, dst, R, C, rope_hd,
                     rope_rows);
  return hipGetLastError();
}

// x[m][:] = E[tok[m]][:] widened to fp32.  Token ids outside [0, V) are
// clamped (validated on the host for host-provided ids).
__global__ void embed_kernel(const int32_t* __restrict__ tok, const u16* __restrict__ E,
                             float* __restrict__ x, int M, int d, int V) {
  const int m = blockIdx.x;
  int t = tok[m];
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const u16* e = E + (size_t)t * d;
  float* xr = x + (size_t)m * d;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(e + c);
    float4 a = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
    float4 b = {bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
    *reinterpret_cast<float4*>(xr + c) = a;
    *reinterpret_cast<float4*>(xr + c + 4) = b;
  }
}

hipError_t launch_embed(const int32_t* tok, const u16* E, float* x, int M, int d, int V,
                        hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(256), 0, s, tok, E, x, M, d, V);
  return hipGetLastError();
}

// out = g * x / sqrt(mean(x^2) + 1e-5), as bf16, into the fragment-packed
// operand [Mp][d] (rows >= M written as zeros) and optionally row-major.
__global__ __launch_bounds__(256) void rmsnorm_pack_kernel(const float* __restrict__ x,
                                                           const u16* __restrict__ gain,
                                                           u16* __restrict__ outp,
                                                           u16* __restrict__ outr, int M,
                                                           int d) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float rs = 0.f;
  if (m < M) {
    const float* xr = x + (size_t)m * d;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
      const float4 v = *reinterpret_cast<const float4*>(xr + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = warp_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    rs = 1.0f / sqrtf(ss / (float)d + 1e-5f);
  }
  for (int c = threadIdx.x * 8; c < d; c += 2048) {
    uint4 o = {0, 0, 0, 0};
    if (m < M) {
      const float* xr = x + (size_t)m * d + c;
      const uint4 gw = *reinterpret_cast<const uint4*>(gain + c);
      const float gv[8] = {bf16lo(gw.x), bf16hi(gw.x), bf16lo(gw.y), bf16hi(gw.y),
                           bf16lo(gw.z), bf16hi(gw.z), bf16lo(gw.w), bf16hi(gw.w)};
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u16 lo = f32_to_bf16(xr[2 * j] * rs * gv[2 * j]);
        const u16 hi = f32_to_bf16(xr[2 * j + 1] * rs * gv[2 * j + 1]);
        pk[j] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      o = {pk[0], pk[1], pk[2], pk[3]};
      if (outr) *reinterpret_cast<uint4*>(outr + (size_t)m * d + c) = o;
    }
    *reinterpret_cast<uint4*>(outp + packed_index(m, c, d)) = o;
  }
}

hipError_t launch_rmsnorm_pack(const float* x, const u16* g, u16* out_packed, u16* out_rows,
                               int M, int Mp, int d, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_pack_kernel, dim3(Mp), dim3(256), 0, s, x, g, out_packed, out_rows,
                     M, d);
  return hipGetLastError();
}

// (cos, sin) of position * 10000^(-2i/hd) for each tree row, position =
// n[b] + depth[b][v]; angles in double precision.
__global__ void rope_table_kernel(const int32_t* __restrict__ n_prefix,
                                  const int32_t* __restrict__ depth_of, float2* __restrict__ rope,
                                  int B, int T, int hd) {
  const int half = hd >> 1;
  const int total = B * T * half;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
    const int m = e / half, i = e % half;
    const int b = m / T;
    const double pos = (double)(n_prefix[b] + depth_of[m]);
    const double inv = pow(10000.0, -2.0 * (double)i / (double)hd);
    double sv, cv;
    sincos(pos * inv, &sv, &cv);
    rope[e] = make_float2((float)cv, (float)sv);
  }
}

hipError_t launch_rope_table(const int32_t* n_prefix, const int32_t* depth_of, float2* rope,
                             int B, int T, int hd, hipStream_t s) {
  const int total = B * T * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, s, n_prefix,
                     depth_of, rope, B, T, hd);
  return hipGetLastError();
}

// KV compaction: for each (layer, sequence, head) and m = 0..accept_len,
// slot n + m <- slot n + path[m], for K and V.  Each thread owns a set of
// dims of one (layer, b, head) and reads every source row before writing any
// row, so overlapping sources and destinations are safe.
#define MV_MAX_PATH 17
__global__ void compact_kernel(u16* __restrict__ kc, u16* __restrict__ vc, int L, int B, int H,
                               int hd, int cap, const int32_t* __restrict__ path, int path_stride,
                               const int32_t* __restrict__ accept_len,
                               const int32_t* __restrict__ n_prefix) {
  // thread -> (layer, b, h, dim)
  const size_t total = (size_t)L * B * H * hd;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int dim = (int)(e % hd);
    const size_t lbh = e / hd;                    // (l*B + b)*H + h
    const int b = (int)((lbh / H) % B);
    const int n = max(n_prefix[b], 0);
    int cnt = accept_len[b] + 1;
    cnt = cnt > path_stride ? path_stride : (cnt < 1 ? 1 : cnt);
    const int32_t* pb = path + (size_t)b * path_stride;
    u16 kv[MV_MAX_PATH], vv[MV_MAX_PATH];
    u16* kp = kc + lbh * (size_t)cap * hd;
    u16* vp = vc + lbh * (size_t)(cap >> 2) * hd * 4;
    if (n + cnt > cap) continue;                  // out of contract: leave the cache alone
    for (int m = 0; m < cnt; ++m) {
      const int s = min(n + max(pb[m], 0), cap - 1);
      kv[m] = kp[(size_t)s * hd + dim];
      vv[m] = vp[((size_t)(s >> 2) * hd + dim) * 4 + (s & 3)];
    }
    for (int m = 0; m < cnt; ++m) {
      const int s = n + m;
      kp[(size_t)s * hd + dim] = kv[m];
      vp[((size_t)(s >> 2) * hd + dim) * 4 + (s & 3)] = vv[m];
    }
  }
}

hipError_t launch_compact(u16* kc, u16* vc, int L, int B, int H, int hd, int cap,
                          const int32_t* path, int path_stride, const int32_t* accept_len,
                          const int32_t* n_prefix, hipStream_t s) {
  const size_t total = (size_t)L * B * H * hd;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(compact_kernel, dim3(blocks), dim3(256), 0, s, kc, vc, L, B, H, hd, cap,
                     path, path_stride, accept_len, n_prefix);
  return hipGetLastError();
}

// n[b] += 1 + accept_len[b]; optionally bump a step counter.
__global__ void advance_kernel(int32_t* n_prefix, const int32_t* accept_len, int B,
                               int32_t* counter) {
  const int b = threadIdx.x;
  if (b < B) n_prefix[b] += 1 + accept_len[b];
  if (b == 0 && counter) counter[0] += 1;
}

hipError_t launch_advance(int32_t* n_prefix, const int32_t* accept_len, int B, int32_t* counter,
                          hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, s, n_prefix, accept_len, B, counter);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s) {
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace mvk
