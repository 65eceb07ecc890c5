// Shared device/host helpers of the gfx950 Medusa tree-verify library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <algorithm>

#include "medusa_verify.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

#define MV_WAVE 64

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is kept as raw 16-bit patterns in memory.  Widening is
// exact (append 16 zero bits); narrowing rounds to nearest, ties to even
// (the hardware v_cvt_pk_bf16_f32 conversion on gfx950).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(u16 b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(u16, h);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Fragment-packed bf16 matrices.
//
// A matrix [R][C] (R % 16 == 0, C % 32 == 0) is cut into blocks of 16 rows x
// 32 columns; inside a block, lane l (0..63) owns row (l % 16) and columns
// 8*(l/16) .. 8*(l/16)+7, and the 64 lanes' 16-byte pieces are consecutive
// (1 KiB per block).  This is the operand layout of
// v_mfma_f32_16x16x32_bf16 for both A (rows = M) and B (rows = N).
//  * activations: row-block-major (block (rb, cb) at rb * C/32 + cb)
//  * weights:     k-block-major   (block (rb, cb) at cb * R/16 + rb)
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ size_t packed_index(int r, int c, int C) {
  const int rb = r >> 4, cb = c >> 5;
  const int lane = (r & 15) + 16 * ((c & 31) >> 3);
  return ((((size_t)rb * (C >> 5) + cb) * 64 + lane) << 3) + (c & 7);
}
__host__ __device__ __forceinline__ size_t packed_index_kmajor(int r, int c, int R) {
  const int rb = r >> 4, cb = c >> 5;
  const int lane = (r & 15) + 16 * ((c & 31) >> 3);
  return ((((size_t)cb * (R >> 4) + rb) * 64 + lane) << 3) + (c & 7);
}

// ---------------------------------------------------------------------------
// KV cache layouts.  Each (layer, sequence, head) owns cap * hd elements
// (cap % 64 == 0, hd % 8 == 0):
//  * K: [cap/32][hd/8][32][8] -- per 32-slot group and 8-dim piece, 32 rows
//    of 16 bytes; slot offset o (0..31) in its group sits at row
//    16*((o>>2)&1) + 4*(o>>3) + (o&3).  The tree-attention K operand of
//    16 keys x 32 dims is then four 256-byte runs (whole cache lines), and
//    the keys it holds match the probabilities' register order.
//  * V: [cap/8][hd][8] -- 8 consecutive slots per dim (one 16-byte load per
//    lane for the P*V operand).
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int kv_krow(int o) {
  return ((o >> 2) & 1) * 16 + (o >> 3) * 4 + (o & 3);
}
__host__ __device__ __forceinline__ size_t kv_k_off(int slot, int dim, int hd) {
  return (((size_t)(slot >> 5) * (hd >> 3) + (dim >> 3)) * 32 + kv_krow(slot & 31)) * 8 + (dim & 7);
}
__host__ __device__ __forceinline__ size_t kv_v_off(int slot, int dim, int hd) {
  return ((size_t)(slot >> 3) * hd + dim) * 8 + (slot & 7);
}

// Order-preserving 64-bit key of (value, column) for an argmax by atomic max:
// larger values win, and among equal values the lower column (0 = no entry).
__device__ __forceinline__ unsigned long long argmax_key(float v, int col) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)col;
}
__device__ __forceinline__ int argmax_key_col(unsigned long long k) {
  return (int)~(uint32_t)(k & 0xffffffffull);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double warp_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------
// Internal launchers (defined in the .hip files; called by api.cpp).
// All return hipError_t of the launch.
// ---------------------------------------------------------------------------
namespace mvk {

enum GemmEpi {
  EPI_STORE = 0,     // out_f32[m][n] = y
  EPI_ADD = 1,       // out_f32[m][n] += y (residual stream)
  EPI_SWIGLU = 2,    // tile = [gate cols | up cols]; out_bf16 packed h = SiLU(g) * u
  EPI_QKV = 3,       // RoPE on q,k; q -> bf16 [M][d]; k,v -> KV cache slots
};

struct QkvArgs {
  u16* q;                 // bf16 [M][d] row-major, RoPE'd
  u16* kcache;            // bf16 K of this layer, [B][H] blocks (kv_k_off inside)
  u16* vcache;            // bf16 V of this layer, [B][H] blocks (kv_v_off inside)
  const int32_t* n_prefix;   // device [B]
  const float2* rope;     // (cos, sin) [B*T][hd/2] at each row's position
  int B, T, H, hd, cap, d;
};

struct GemmArgs {
  const u16* A;      // fragment-packed bf16 activations [Mp][K] (row-block-major)
  const u16* W;      // k-major packed weights [K/32][N/16] blocks (SWIGLU: gate)
  const u16* W2;     // SWIGLU: up weights (same layout)
  int M, Mp, N, K;   // SWIGLU: N = F (features)
  int w, nbw;        // waves per workgroup, 16-column blocks per wave (SWIGLU, QKV: 2)
  int splits;        // K splits across workgroups
  int epi;
  const float* ss;   // nullable: rows' partial sums of squares [Mp][ss_ld] (first
  int ss_tiles;      //   ss_tiles entries of a row used; ss_ld % 4 == 0) of the
  int ss_ld;         //   un-normalised input; accumulators scaled by 1/sqrt(sum/K + 1e-5)
  float* out_f32;    // STORE / ADD target [M][N]
  u16* out_bf16;     // SWIGLU target (packed [Mp][N])
  const u16* next_gain;  // ADD, nullable: gain of the norm that reads x next
  u16* xn_out;           // ADD: packed bf16 [Mp][N] = x * next_gain
  float* ss_out;         // ADD: [Mp][ss_ld] rows' sums of squares of x per column tile
  unsigned long long* amax_key;   // STORE, nullable: per row, atomic max of
                     //   argmax_key(value, column) over the row's columns; must
                     //   hold 0 before the launch (the consumer clears it)
  int* status;       // STORE, nullable: MV_STATUS_NONFINITE OR-ed in when a
                     //   stored value (rows < M) is not finite
  float* partial;    // split-K partial tiles
  int* counters;     // split-K arrival counters [tiles], zero between launches
  QkvArgs qkv;
  int wide;          // 0, or the wide-tile kernel's column blocks per wave (4 or
                     //   5; more than 128 rows): tiles of 256 rows x 32*wide columns
  int prefetch;      // QKV: extra grid columns of workgroups that read this
                     //   layer's cached prefix K/V ahead of the attention launch,
  int pf_budget16;   //   at most this many 16-byte pieces each
};

int gemm_mb(int Mp);                                  // 16-row blocks per tile
int gemm_kc(int MB);                                  // k-blocks per chunk
int gemm_ntiles(int epi, int N, int w, int nbw);      // column tiles
int gemm_wide_ntiles(int epi, int N, int nbh);        // column tiles of the wide kernel
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);
hipError_t launch_pack(const u16* src, u16* dst, int R, int C, int rope_hd, int rope_rows,
                       hipStream_t s);
// Embedding options: tree tokens from the heads' top-s lists (top_ids
// [B][D][s_top], root [B], rank [B*T]; tokens written to tok_out), and the
// first norm's GEMM operand (packed bf16(x * gain) [Mp][d], sums of squares at
// ss[m * ss_ld]).  Null top_ids / gain: off.
struct EmbedTree {
  const int32_t* top_ids;
  const int32_t* root;
  const int32_t* rank;
  int D, s_top;
  int32_t* tok_out;
};
struct EmbedNorm {
  const u16* gain;
  u16* xn;
  float* ss;
  int ss_ld;
};
hipError_t launch_embed(const int32_t* tok, const u16* E, float* x, float* ss, int M, int d,
                        int V, const int32_t* n_prefix, const int32_t* depth_of, float2* rope,
                        int T, int hd, hipStream_t s, EmbedTree et = {}, EmbedNorm en = {});
hipError_t launch_norm_prep(const float* x, const u16* g, u16* xn_packed, float* ss, int ss_ld,
                            int M, int d, hipStream_t s);
hipError_t launch_rope_table(const int32_t* n_prefix, const int32_t* depth_of, float2* rope,
                             int B, int T, int hd, hipStream_t s);
// Tree attention with the key range of each (sequence, head) split over up
// to attention_splits(B, H, T) workgroups; with more than one split the
// partial states go to part_o [B*H][S][round16(T)][hd] fp32 and part_ml
// [B*H][S][T] in the caller's workspace, and a second launch merges them.
int attention_splits(int B, int H, int T);
// Whether a launch of this shape splits key ranges (else one workgroup per
// 16 queries of a (sequence, head) reads the pair's whole cache).
bool attention_uses_splits(int B, int H, int T, int cap);
hipError_t launch_attention(const u16* q, const u16* kc, const u16* vc, const int32_t* n_prefix,
                            const uint64_t* anc, int B, int T, int H, int hd, int cap, int mw,
                            u16* out, int packed, float* part_o, float2* part_ml, hipStream_t s);
hipError_t launch_heads_w1(const u16* h, const u16* w1, float* u, int B, int D, int d,
                           hipStream_t s);
hipError_t launch_heads_w2(const float* u, const u16* w2, float* z, int B, int D, int d, int V,
                           hipStream_t s);
int topk_waves(int V);   // stage-1 waves per row (candidate slots = waves * s)
hipError_t launch_topk(const float* z, int rows, int V, int s_top, int32_t* ids, float* vals,
                       float* cand_v, int* cand_i, hipStream_t s);
hipError_t launch_tree_fill(const int32_t* top_ids, const int32_t* root, const int32_t* depth_of,
                            const int32_t* rank, int32_t* tok, int B, int T, int D, int s_top,
                            hipStream_t s);
hipError_t launch_row_stats(const float* logits, int rows, int V, int mode, double temperature,
                            int32_t* argmax, double* stats, hipStream_t s, double* bsum = nullptr);
// Capacity check of a step, done by its acceptance kernel: with status
// non-null, MV_STATUS_CAPACITY is OR-ed into *status when a sequence's prefix
// length at the start of the step (before the kernel moves it on) was
// negative or left fewer than T free slots below cap.
struct StepGuard {
  int* status;
  int cap, T;
};
hipError_t launch_accept_finish(const float* logits, const int32_t* argmax, unsigned long long* amax_key,
                                const double* stats,
                                const int32_t* parent, const int32_t* depth_of,
                                const int32_t* tok, int B, int T, int V, int depth, int mode,
                                int root_mode, double temperature, double eps, double delta,
                                const double* u, const int32_t* u_index, int u_stride,
                                int32_t* accept_len, int32_t* path, int32_t* best,
                                int32_t* next_root, int32_t* emitted, double* margin,
                                const float* x, const u16* final_norm, u16* h_last, int d,
                                hipStream_t s, int32_t* n_advance = nullptr,
                                const double* bsum = nullptr, StepGuard guard = {});
hipError_t launch_prefill_select(const float* logits, const int32_t* amax, const int32_t* cnt,
                                 int B, int T, int V, int root_mode, double temperature,
                                 const double* u, int u_bstride, int32_t* root, int32_t* n_prefix,
                                 const float* x, const u16* final_norm, u16* h_last, int d,
                                 hipStream_t s);
hipError_t launch_reject_accept(const float* logits, const int32_t* argmax, const double* stats,
                                const int32_t* parent, const int32_t* tok, int B, int T, int V,
                                int depth, double temperature, const float* draft,
                                const double* dstats, const double* u, const int32_t* u_index,
                                long long u_stride, double* resid, int32_t* accept_len,
                                int32_t* path, int32_t* best, int32_t* next_root,
                                int32_t* emitted, double* margin, const float* x,
                                const u16* final_norm, u16* h_last, int d, hipStream_t s,
                                int32_t* n_advance = nullptr, const double* bsum = nullptr,
                                StepGuard guard = {});
hipError_t launch_compact(u16* kc, u16* vc, int L, int B, int H, int hd, int cap,
                          const int32_t* path, int path_stride, const int32_t* accept_len,
                          const int32_t* n_prefix, hipStream_t s, int advanced = 0,
                          int32_t* u_index = nullptr);
hipError_t launch_advance(int32_t* n_prefix, const int32_t* accept_len, int B,
                          int32_t* counter, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

// train.hip: Medusa-1 head loss and gradients
hipError_t launch_gemm_nt(const u16* A, int lda, size_t sa, const u16* B, int ldb, size_t sb,
                          float* C, int ldc, size_t sc, int M, int N, int K, int batch,
                          hipStream_t s);
hipError_t launch_gemm_nt_splitk(const u16* A, int lda, const u16* B, int ldb, float* C, int M,
                                 int N, int K, float* part, size_t part_elems, hipStream_t s);
hipError_t launch_transpose_bf16(const u16* in, size_t s_in, u16* out, size_t s_out, int R, int C,
                                 int batch, hipStream_t s);
hipError_t launch_medusa1_act(const float* a, const u16* h, u16* s, size_t n, hipStream_t st);
hipError_t launch_medusa1_dact(const float* ds, const float* a, u16* da, size_t n, hipStream_t st);
hipError_t launch_medusa1_ce(const float* z, const int32_t* labels, int ldl, int k, float lambda,
                             int N, int V, float* loss_tk, u16* g, hipStream_t st);
hipError_t launch_medusa1_sum(const float* v, int n, double* out, hipStream_t st);

}  // namespace mvk
