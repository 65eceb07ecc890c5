// Row-wise kernels of the tree-verify forward: weight packing, embedding
// gather (with the rows' sums of squares and RoPE tables), KV compaction and
// small state updates.
#include "common.hpp"

namespace mvk {

// Logical q/k feature stored at packed row p (see the QKV GEMM epilogue):
// with heads wider than 16, each group of 32 rows holds 16 first-half dims of
// a head followed by their RoPE partners (dim + hd/2).
__host__ __device__ __forceinline__ int qkv_feature_h(int p, int d, int hd) {
  if (hd < 32 || p >= 2 * d) return p;
  const int h = p / hd, e = p % hd, j = e / 32, ee = e % 32;
  return h * hd + (ee < 16 ? j * 16 + ee : hd / 2 + j * 16 + (ee - 16));
}

// dst (fragment-packed, k-block-major [R][C]) <- src (row-major [R][C]);
// when rope_hd > 0 the first rope_rows rows (q and k of a fused QKV matrix)
// are reordered as qkv_feature_h says.  One thread per 16-byte piece.
__global__ void pack_kernel(const u16* __restrict__ src, u16* __restrict__ dst, int R, int C,
                            int rope_hd, int rope_rows) {
  const size_t pieces = (size_t)R * (C / 8);
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < pieces;
       e += (size_t)gridDim.x * blockDim.x) {
    const int p = (int)(e / (C / 8));            // packed row
    const int c = (int)(e % (C / 8)) * 8;
    int r = p;
    if (rope_hd > 0 && p < rope_rows) r = qkv_feature_h(p, rope_rows / 2, rope_hd);
    const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * C + c);
    *reinterpret_cast<uint4*>(dst + packed_index_kmajor(p, c, R)) = v;
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

__device__ __forceinline__ float block_sum256(float v) {
  __shared__ float red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  v = warp_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return v;
}

// One workgroup per row m: x[m][:] = E[tok[m]][:] widened to fp32, ss[m] =
// sum of squares of the row; optionally the row's RoPE table: (cos, sin) of
// position * 10000^(-2i/hd), position = n[b] + depth[m], angles in double.
// Token ids outside [0, V) are clamped.
// With et.top_ids the token is the tree's own (root for node 0, else the
// node's rank in its depth's head top-s list) and is written to et.tok_out;
// with en.gain the row also leaves the first norm's GEMM operand: packed
// bf16(x * gain) and its sum of squares at en.ss[m * en.ss_ld].
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok,
                                                    const u16* __restrict__ E,
                                                    float* __restrict__ x, float* __restrict__ ss,
                                                    int d, int V,
                                                    const int32_t* __restrict__ n_prefix,
                                                    const int32_t* __restrict__ depth_of,
                                                    float2* __restrict__ rope, int T, int hd,
                                                    EmbedTree et, EmbedNorm en) {
  const int m = blockIdx.x;
  // requests that depend on nothing go out first: the node's depth and rank,
  // the root, the prefix length, the norm's gains
  constexpr int EC = 4;                         // 8-column chunks per thread (d <= 8192)
  const bool regs = d <= EC * 2048;
  uint4 gw[EC];
#pragma unroll
  for (int j = 0; j < EC; ++j) {
    const int c = threadIdx.x * 8 + j * 2048;
    gw[j] = (en.gain && regs && c < d) ? *reinterpret_cast<const uint4*>(en.gain + c)
                                        : uint4{0u, 0u, 0u, 0u};
  }
  const int T_ = T > 0 ? T : 1;
  const int b = m / T_, v = m - b * T_;
  const int dep_m = depth_of ? depth_of[m] : 0;
  const int npre = rope ? n_prefix[b] : 0;
  int t;
  if (et.top_ids) {
    const int dep = min(dep_m, et.D);
    const int rk = min(max(et.rank[m], 0), et.s_top - 1);
    const int rt = et.root[b];
    t = (v == 0 || dep <= 0) ? rt : et.top_ids[((size_t)b * et.D + (dep - 1)) * et.s_top + rk];
  } else {
    t = tok[m];
  }
  // the RoPE table row needs only the position: computed while the token's
  // id is in flight
  if (rope) {
    const int half = hd >> 1;
    const double pos = (double)(npre + dep_m);
    for (int i = threadIdx.x; i < half; i += 256) {
      const double inv = pow(10000.0, -2.0 * (double)i / (double)hd);
      double sv, cv;
      sincos(pos * inv, &sv, &cv);
      rope[(size_t)m * half + i] = make_float2((float)cv, (float)sv);
    }
  }
  if (et.top_ids && threadIdx.x == 0) et.tok_out[m] = t;
  t = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const u16* e = E + (size_t)t * d;
  float* xr = x + (size_t)m * d;
  float sq = 0.f;
  auto one_chunk = [&](int c, const uint4& gwc) {
    const uint4 w = *reinterpret_cast<const uint4*>(e + c);
    float4 a = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
    float4 bb = {bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
    *reinterpret_cast<float4*>(xr + c) = a;
    *reinterpret_cast<float4*>(xr + c + 4) = bb;
    sq += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + bb.x * bb.x + bb.y * bb.y + bb.z * bb.z +
          bb.w * bb.w;
    if (en.gain) {
      uint4 o;
      o.x = f32_to_bf16(a.x * bf16lo(gwc.x)) | ((uint32_t)f32_to_bf16(a.y * bf16hi(gwc.x)) << 16);
      o.y = f32_to_bf16(a.z * bf16lo(gwc.y)) | ((uint32_t)f32_to_bf16(a.w * bf16hi(gwc.y)) << 16);
      o.z = f32_to_bf16(bb.x * bf16lo(gwc.z)) | ((uint32_t)f32_to_bf16(bb.y * bf16hi(gwc.z)) << 16);
      o.w = f32_to_bf16(bb.z * bf16lo(gwc.w)) | ((uint32_t)f32_to_bf16(bb.w * bf16hi(gwc.w)) << 16);
      *reinterpret_cast<uint4*>(en.xn + packed_index(m, c, d)) = o;
    }
  };
  if (regs) {
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const int c = threadIdx.x * 8 + j * 2048;
      if (c < d) one_chunk(c, gw[j]);
    }
  } else {
    for (int c = threadIdx.x * 8; c < d; c += 2048)
      one_chunk(c, en.gain ? *reinterpret_cast<const uint4*>(en.gain + c) : uint4{0u, 0u, 0u, 0u});
  }
  sq = block_sum256(sq);
  if (threadIdx.x == 0 && ss) ss[m] = sq;
  if (threadIdx.x == 0 && en.gain) en.ss[(size_t)m * en.ss_ld] = sq;
}

hipError_t launch_embed(const int32_t* tok, const u16* E, float* x, float* ss, int M, int d,
                        int V, const int32_t* n_prefix, const int32_t* depth_of, float2* rope,
                        int T, int hd, hipStream_t s, EmbedTree et, EmbedNorm en) {
  hipLaunchKernelGGL(embed_kernel, dim3(M), dim3(256), 0, s, tok, E, x, ss, d, V, n_prefix,
                     depth_of, rope, T, hd, et, en);
  return hipGetLastError();
}

// Operand of a normalised GEMM for row m of x [M][d]: the fragment-packed
// bf16 row x * g and the row's sum of squares ss[m * ss_ld] (the GEMM applies
// 1/sqrt(ss/d + 1e-5) to its accumulators).  One workgroup per row; the row
// (d <= 8192) is held in registers, so it is read once.
#define MV_NORM_MAX_CHUNKS 4          // 8 columns per thread per chunk
__global__ __launch_bounds__(256) void norm_prep_kernel(const float* __restrict__ x,
                                                        const u16* __restrict__ gain,
                                                        u16* __restrict__ outp,
                                                        float* __restrict__ ss, int ss_ld,
                                                        int d) {
  const int m = blockIdx.x;
  float v[MV_NORM_MAX_CHUNKS][8];
  float sq = 0.f;
#pragma unroll
  for (int j = 0; j < MV_NORM_MAX_CHUNKS; ++j) {
    const int c = (j * 256 + threadIdx.x) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
    if (c < d) {
      const float4 a = *reinterpret_cast<const float4*>(x + (size_t)m * d + c);
      const float4 b = *reinterpret_cast<const float4*>(x + (size_t)m * d + c + 4);
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += v[j][e] * v[j][e];
    }
  }
  sq = block_sum256(sq);
  if (threadIdx.x == 0) ss[(size_t)m * ss_ld] = sq;
#pragma unroll
  for (int j = 0; j < MV_NORM_MAX_CHUNKS; ++j) {
    const int c = (j * 256 + threadIdx.x) * 8;
    if (c >= d) continue;
    const uint4 gw = *reinterpret_cast<const uint4*>(gain + c);
    const float gv[8] = {bf16lo(gw.x), bf16hi(gw.x), bf16lo(gw.y), bf16hi(gw.y),
                         bf16lo(gw.z), bf16hi(gw.z), bf16lo(gw.w), bf16hi(gw.w)};
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const u16 lo = f32_to_bf16(v[j][2 * e] * gv[2 * e]);
      const u16 hi = f32_to_bf16(v[j][2 * e + 1] * gv[2 * e + 1]);
      pk[e] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *reinterpret_cast<uint4*>(outp + packed_index(m, c, d)) = uint4{pk[0], pk[1], pk[2], pk[3]};
  }
}

hipError_t launch_norm_prep(const float* x, const u16* g, u16* xn_packed, float* ss, int ss_ld,
                            int M, int d, hipStream_t s) {
  if (d > MV_NORM_MAX_CHUNKS * 2048) return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_prep_kernel, dim3(M), dim3(256), 0, s, x, g, xn_packed, ss, ss_ld, d);
  return hipGetLastError();
}

// (cos, sin) tables for all B*T rows (see embed_kernel).
__global__ void rope_table_kernel(const int32_t* __restrict__ n_prefix,
                                  const int32_t* __restrict__ depth_of, float2* __restrict__ rope,
                                  int B, int T, int hd) {
  const int half = hd >> 1;
  const int total = B * T * half;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
    const int m = e / half, i = e % half;
    const double pos = (double)(n_prefix[m / T] + depth_of[m]);
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
// slot n + m <- slot n + path[m], for K and V.  Each thread owns one dim of
// one (layer, b, head) and reads every source row before writing any row, so
// overlapping sources and destinations are safe.
#define MV_MAX_PATH (MV_MAX_DEPTH + 1)
__global__ void compact_kernel(u16* __restrict__ kc, u16* __restrict__ vc, int L, int B, int H,
                               int hd, int cap, const int32_t* __restrict__ path, int path_stride,
                               const int32_t* __restrict__ accept_len,
                               const int32_t* __restrict__ n_prefix, int advanced,
                               int32_t* __restrict__ u_index) {
  // advanced: n_prefix already holds n + accept_len + 1 (the acceptance
  // kernel moved it on); the step's draw counter is bumped here
  if (advanced && u_index && blockIdx.x == 0 && threadIdx.x == 0) u_index[0] += 1;
  const size_t total = (size_t)L * B * H * hd;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int dim = (int)(e % hd);
    const size_t lbh = e / hd;                    // (l*B + b)*H + h
    const int b = (int)((lbh / H) % B);
    const int n = max(n_prefix[b] - (advanced ? accept_len[b] + 1 : 0), 0);
    int cnt = accept_len[b] + 1;
    cnt = cnt > path_stride ? path_stride : (cnt < 1 ? 1 : cnt);
    const int32_t* pb = path + (size_t)b * path_stride;
    u16 kv[MV_MAX_PATH], vv[MV_MAX_PATH];
    u16* kp = kc + lbh * (size_t)cap * hd;
    u16* vp = vc + lbh * (size_t)cap * hd;
    if (n + cnt > cap) continue;                  // out of contract: leave the cache alone
    for (int m = 0; m < cnt; ++m) {
      const int s = min(n + max(pb[m], 0), cap - 1);
      kv[m] = kp[kv_k_off(s, dim, hd)];
      vv[m] = vp[kv_v_off(s, dim, hd)];
    }
    for (int m = 0; m < cnt; ++m) {
      const int s = n + m;
      kp[kv_k_off(s, dim, hd)] = kv[m];
      vp[kv_v_off(s, dim, hd)] = vv[m];
    }
  }
}

// Streaming-read probe (measurement only): workgroup i sums the i-th slice
// of buf with 16 16-byte loads in flight per lane; the sum is written only if
// it equals a sentinel, so the reads cannot be dropped.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         float* __restrict__ out) {
  constexpr int U = 16;
  const size_t per = n16 / gridDim.x;
  const uint4* q = p + per * blockIdx.x;
  float s = 0.f;
  for (size_t i = threadIdx.x; i + (U - 1) * 256 < per; i += U * 256) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = q[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) s += __uint_as_float(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  if (s == 1.2345f) out[0] = s;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(4096), dim3(256), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_compact(u16* kc, u16* vc, int L, int B, int H, int hd, int cap,
                          const int32_t* path, int path_stride, const int32_t* accept_len,
                          const int32_t* n_prefix, hipStream_t s, int advanced,
                          int32_t* u_index) {
  const size_t total = (size_t)L * B * H * hd;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(compact_kernel, dim3(blocks), dim3(256), 0, s, kc, vc, L, B, H, hd, cap,
                     path, path_stride, accept_len, n_prefix, advanced, u_index);
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
