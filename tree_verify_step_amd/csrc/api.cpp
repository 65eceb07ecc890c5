// C ABI of the Medusa tree-verify library: argument validation, workspace
// carving, kernel sequencing for each operation, and the step driver that
// captures one whole decoding step into a hipGraph.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "common.hpp"
#include "internal.hpp"
#include "medusa_verify.h"

namespace mvk {
hipError_t launch_prefill_select(const float* logits, const int32_t* amax, const int32_t* cnt,
                                 int B, int T, int V, int root_mode, float temperature,
                                 const double* u, int32_t* root, int32_t* n_prefix, const u16* hn,
                                 u16* h_last, int d, hipStream_t s);
}

namespace mv {

static thread_local char g_err[512];
char* last_error_buf() { return g_err; }

#define MV_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return fail(MV_EHIP, "%s: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
  } while (0)

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int round16(int x) { return (x + 15) & ~15; }

static int check_dims(const mv_dims* D) {
  if (!D) return fail(MV_EINVAL, "dims is NULL");
  if (D->L < 1 || D->d < 64 || D->H < 1 || D->hd < 1 || D->F < 32 || D->V < 64 || D->K < 1)
    return fail(MV_EINVAL, "dims out of range (L=%d d=%d H=%d hd=%d F=%d V=%d K=%d)", D->L, D->d,
                D->H, D->hd, D->F, D->V, D->K);
  if (D->H * D->hd != D->d) return fail(MV_EUNSUPPORTED, "H*hd (%d) != d (%d)", D->H * D->hd, D->d);
  if (D->d % 64 || D->F % 32 || D->V % 64)
    return fail(MV_EUNSUPPORTED, "need d%%64==0, F%%32==0, V%%64==0 (d=%d F=%d V=%d)", D->d, D->F, D->V);
  if (D->hd != 16 && D->hd != 32 && D->hd != 64 && D->hd != 128)
    return fail(MV_EUNSUPPORTED, "head dim %d not in {16,32,64,128}", D->hd);
  if (D->K > MV_MAX_DEPTH) return fail(MV_EUNSUPPORTED, "K=%d > %d", D->K, MV_MAX_DEPTH);
  return MV_OK;
}

static int check_tree(const mv_tree* t, bool need_anc) {
  if (!t) return fail(MV_EINVAL, "tree is NULL");
  if (t->T < 1 || t->T > MV_MAX_T) return fail(MV_EUNSUPPORTED, "tree T=%d outside [1,%d]", t->T, MV_MAX_T);
  if (t->depth < 0 || t->depth > MV_MAX_DEPTH || t->depth > t->T - 1)
    return fail(MV_ETREE, "tree depth %d invalid for T=%d", t->depth, t->T);
  if (t->mask_words != (t->T + 63) / 64)
    return fail(MV_EINVAL, "mask_words %d != ceil(T/64)", t->mask_words);
  if (!t->parent || !t->depth_of || !t->rank || (need_anc && !t->anc))
    return fail(MV_EINVAL, "tree arrays must be non-NULL");
  return MV_OK;
}

static int check_batch(int B) {
  if (B < 1 || B > MV_MAX_BATCH) return fail(MV_EUNSUPPORTED, "batch %d outside [1,%d]", B, MV_MAX_BATCH);
  return MV_OK;
}

// ---------------------------------------------------------------------------
// Launch configuration and workspace
// ---------------------------------------------------------------------------
static int attn_nsplit(int B, int H, int T) {
  const int QG = (T + 63) / 64;
  int ns = 512 / (B * H * QG) - 1;
  return std::max(1, std::min(ns, 31));
}

static int gemm_splits(int ntiles, int K) {
  const int KB = K / 32;
  int s = (320 + ntiles - 1) / ntiles;
  s = std::min(s, std::max(1, KB / 8));
  return std::max(1, std::min(s, 16));
}

struct Gemms {
  int qkv, o, gu, down, lm;
};
static Gemms gemm_plan(const mv_dims& D) {
  Gemms g;
  g.qkv = gemm_splits(3 * D.d / 64, D.d);
  g.o = gemm_splits(D.d / 64, D.d);
  g.gu = gemm_splits(D.F / 32, D.d);
  g.down = gemm_splits(D.d / 64, D.F);
  g.lm = 1;
  return g;
}

struct Ws {
  size_t x, xa, ha, q, rope, po, pml, part, hu, hz, topi, topv, amax, stats, hn, cnt, total;
  int nsplit;
};

static Ws ws_layout(const mv_dims& D, int B, int T) {
  Ws w;
  const int M = B * T, Mp = round16(M);
  const Gemms g = gemm_plan(D);
  w.nsplit = attn_nsplit(B, D.H, T);
  size_t part = 0;
  auto upd = [&](int s, size_t ncols) {
    if (s > 1) part = std::max(part, (size_t)s * M * ncols * 4);
  };
  upd(g.qkv, 3 * (size_t)D.d);
  upd(g.o, D.d);
  upd(g.gu, 2 * (size_t)D.F);
  upd(g.down, D.d);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 16));
    return o;
  };
  w.x = take((size_t)M * D.d * 4);
  w.xa = take((size_t)Mp * D.d * 2);
  w.ha = take((size_t)Mp * D.F * 2);
  w.q = take((size_t)M * D.d * 2);
  w.rope = take((size_t)M * (D.hd / 2) * 8);
  w.po = take((size_t)(w.nsplit + 1) * M * D.d * 4);
  w.pml = take((size_t)(w.nsplit + 1) * M * D.H * 8);
  w.part = take(part);
  w.hu = take((size_t)B * D.K * D.d * 4);
  w.hz = take((size_t)B * D.K * D.V * 4);
  w.topi = take((size_t)B * D.K * MV_MAX_TOPK * 4);
  w.topv = take((size_t)B * D.K * MV_MAX_TOPK * 4);
  w.amax = take((size_t)M * 4);
  w.stats = take((size_t)M * 3 * 8);
  w.hn = take((size_t)M * D.d * 2);
  w.cnt = take((size_t)B * 4);
  w.total = off;
  return w;
}

template <class T>
static inline T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

static size_t kv_layer_elems(const mv_kv& kv) { return (size_t)kv.B * kv.H * kv.cap * kv.hd; }

static hipError_t gemm(const mvk::GemmArgs& g, hipStream_t s) {
  hipError_t e = mvk::launch_gemm(g, s);
  if (e == hipSuccess && g.splits > 1) e = mvk::launch_gemm_reduce(g, s);
  return e;
}

// ---------------------------------------------------------------------------
// Optional per-launch timing of an eagerly enqueued step: a pair of HIP
// events around each launch group, tagged with its kind (mv_step_profile).
// ---------------------------------------------------------------------------
struct Prof {
  hipEvent_t* ev;       // 2 * cap events
  int cap, n;
  int kind[1024];
};
static thread_local Prof* g_prof = nullptr;

static inline void prof_begin(hipStream_t s) {
  if (g_prof && g_prof->n < g_prof->cap) (void)hipEventRecord(g_prof->ev[2 * g_prof->n], s);
}
static inline void prof_end(int kind, hipStream_t s) {
  if (g_prof && g_prof->n < g_prof->cap) {
    (void)hipEventRecord(g_prof->ev[2 * g_prof->n + 1], s);
    g_prof->kind[g_prof->n++] = kind;
  }
}

// ---------------------------------------------------------------------------
// Enqueue helpers (no validation)
// ---------------------------------------------------------------------------
static int enq_rope(const mv_dims& D, int B, const mv_tree& t, const int32_t* n_prefix, void* ws,
                    const Ws& L, hipStream_t s) {
  MV_HIP(mvk::launch_rope_table(n_prefix, t.depth_of, at<float2>(ws, L.rope), B, t.T, D.hd, s));
  return MV_OK;
}

static int enq_attention(const mv_dims& D, int B, const mv_tree& t, const int32_t* n_prefix,
                         const u16* q, const mv_kv& kv, int layer, u16* out, int packed, void* ws,
                         const Ws& L, hipStream_t s) {
  const size_t le = kv_layer_elems(kv);
  const u16* kc = static_cast<const u16*>(kv.k) + (size_t)layer * le;
  const u16* vc = static_cast<const u16*>(kv.v) + (size_t)layer * le;
  MV_HIP(mvk::launch_attention(q, kc, vc, n_prefix, t.anc, B, t.T, D.H, D.hd, kv.cap,
                               t.mask_words, L.nsplit, at<float>(ws, L.po), at<float>(ws, L.pml), s));
  MV_HIP(mvk::launch_attn_combine(at<float>(ws, L.po), at<float>(ws, L.pml), out, packed, B, t.T,
                                  D.H, D.hd, L.nsplit, round16(B * t.T), s));
  return MV_OK;
}

static int enq_layer(const mv_dims& D, int B, const mv_tree& t, const int32_t* n_prefix,
                     const mv_layer_weights& w, const mv_kv& kv, int layer, float* x, void* ws,
                     const Ws& L, hipStream_t s) {
  const int M = B * t.T, Mp = round16(M);
  const Gemms plan = gemm_plan(D);
  u16* xa = at<u16>(ws, L.xa);
  u16* ha = at<u16>(ws, L.ha);
  u16* q = at<u16>(ws, L.q);
  float* part = at<float>(ws, L.part);
  const size_t le = kv_layer_elems(kv);

  prof_begin(s);
  MV_HIP(mvk::launch_rmsnorm_pack(x, static_cast<const u16*>(w.attn_norm), xa, nullptr, M, Mp, D.d, s));
  prof_end(MV_K_NORM, s);
  mvk::GemmArgs g{};
  g.A = xa;
  g.W = static_cast<const u16*>(w.wqkv);
  g.M = M;
  g.Mp = Mp;
  g.N = 3 * D.d;
  g.K = D.d;
  g.splits = plan.qkv;
  g.epi = mvk::EPI_QKV;
  g.partial = part;
  g.qkv.q = q;
  g.qkv.kcache = static_cast<u16*>(kv.k) + (size_t)layer * le;
  g.qkv.vcache = static_cast<u16*>(kv.v) + (size_t)layer * le;
  g.qkv.n_prefix = n_prefix;
  g.qkv.depth_of = t.depth_of;
  g.qkv.rope = at<float2>(ws, L.rope);
  g.qkv.B = B;
  g.qkv.T = t.T;
  g.qkv.H = D.H;
  g.qkv.hd = D.hd;
  g.qkv.cap = kv.cap;
  g.qkv.d = D.d;
  prof_begin(s);
  MV_HIP(gemm(g, s));
  prof_end(MV_K_QKV, s);

  prof_begin(s);
  int rc = enq_attention(D, B, t, n_prefix, q, kv, layer, xa, 1, ws, L, s);
  if (rc) return rc;
  prof_end(MV_K_ATTN, s);

  mvk::GemmArgs o{};
  o.A = xa;
  o.W = static_cast<const u16*>(w.wo);
  o.M = M;
  o.Mp = Mp;
  o.N = D.d;
  o.K = D.d;
  o.splits = plan.o;
  o.epi = mvk::EPI_ADD;
  o.out_f32 = x;
  o.partial = part;
  prof_begin(s);
  MV_HIP(gemm(o, s));
  prof_end(MV_K_O, s);

  prof_begin(s);
  MV_HIP(mvk::launch_rmsnorm_pack(x, static_cast<const u16*>(w.ffn_norm), xa, nullptr, M, Mp, D.d, s));
  prof_end(MV_K_NORM, s);
  mvk::GemmArgs gu{};
  gu.A = xa;
  gu.W = static_cast<const u16*>(w.wgate);
  gu.W2 = static_cast<const u16*>(w.wup);
  gu.M = M;
  gu.Mp = Mp;
  gu.N = D.F;
  gu.K = D.d;
  gu.splits = plan.gu;
  gu.epi = mvk::EPI_SWIGLU;
  gu.out_bf16 = ha;
  gu.partial = part;
  prof_begin(s);
  MV_HIP(gemm(gu, s));
  prof_end(MV_K_GATE_UP, s);

  mvk::GemmArgs dn{};
  dn.A = ha;
  dn.W = static_cast<const u16*>(w.wdown);
  dn.M = M;
  dn.Mp = Mp;
  dn.N = D.d;
  dn.K = D.F;
  dn.splits = plan.down;
  dn.epi = mvk::EPI_ADD;
  dn.out_f32 = x;
  dn.partial = part;
  prof_begin(s);
  MV_HIP(gemm(dn, s));
  prof_end(MV_K_DOWN, s);
  return MV_OK;
}

static int enq_lm_head(const mv_dims& D, int M, const float* x, const void* final_norm,
                       const void* lm, float* logits, u16* hn_rows, void* ws, const Ws& L,
                       hipStream_t s) {
  const int Mp = round16(M);
  u16* xa = at<u16>(ws, L.xa);
  MV_HIP(mvk::launch_rmsnorm_pack(x, static_cast<const u16*>(final_norm), xa, hn_rows, M, Mp, D.d, s));
  mvk::GemmArgs g{};
  g.A = xa;
  g.W = static_cast<const u16*>(lm);
  g.M = M;
  g.Mp = Mp;
  g.N = D.V;
  g.K = D.d;
  g.splits = 1;
  g.epi = mvk::EPI_STORE;
  g.out_f32 = logits;
  MV_HIP(gemm(g, s));
  return MV_OK;
}

static int enq_heads(const mv_dims& D, int B, int Dn, int s_top, const void* h, const void* w1,
                     const void* w2, const mv_tree* tree, const int32_t* root, int32_t* top_ids,
                     float* top_vals, int32_t* tree_tok, float* z, void* ws, const Ws& L,
                     hipStream_t s) {
  float* u = at<float>(ws, L.hu);
  MV_HIP(mvk::launch_heads_w1(static_cast<const u16*>(h), static_cast<const u16*>(w1), u, B, Dn,
                              D.d, s));
  MV_HIP(mvk::launch_heads_w2(u, static_cast<const u16*>(w2), z, B, Dn, D.d, D.V, s));
  MV_HIP(mvk::launch_topk(z, B * Dn, D.V, s_top, top_ids, top_vals, s));
  if (tree && tree_tok)
    MV_HIP(mvk::launch_tree_fill(top_ids, root, tree->depth_of, tree->rank, tree_tok, B, tree->T,
                                 Dn, s_top, s));
  return MV_OK;
}

static int enq_accept(int B, int T, int V, int d, const float* logits, const mv_tree& t,
                      const int32_t* tok, const mv_accept_params& p, const double* u,
                      const int32_t* u_index, int u_stride, int32_t* accept_len, int32_t* path,
                      int32_t* best, int32_t* next_root, int32_t* emitted, double* margin,
                      const void* hn, void* h_last, void* ws, const Ws& L, hipStream_t s) {
  int32_t* amax = at<int32_t>(ws, L.amax);
  double* stats = at<double>(ws, L.stats);
  MV_HIP(mvk::launch_row_stats(logits, B * T, V, p.mode, p.temperature, amax, stats, s));
  MV_HIP(mvk::launch_accept_finish(logits, amax, stats, t.parent, t.depth_of, tok, B, T, V,
                                   t.depth, p.mode, p.root_mode, p.temperature, p.eps, p.delta, u,
                                   u_index, u_stride, accept_len, path, best, next_root, emitted,
                                   margin, static_cast<const u16*>(hn), static_cast<u16*>(h_last),
                                   d, s));
  return MV_OK;
}

}  // namespace mv

using namespace mv;

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

MV_API const char* mv_strerror(int status) {
  switch (status) {
    case MV_OK: return "ok";
    case MV_EINVAL: return "invalid argument";
    case MV_EUNSUPPORTED: return "unsupported shape";
    case MV_ECAPACITY: return "KV cache capacity exceeded";
    case MV_EWORKSPACE: return "workspace too small";
    case MV_EHIP: return "HIP runtime error";
    case MV_ETREE: return "invalid tree";
    default: return "unknown status";
  }
}

MV_API const char* mv_last_error(void) { return g_err; }

MV_API int mv_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols, int32_t layout,
                          int32_t hd, void* stream) {
  if (!src || !dst) return fail(MV_EINVAL, "mv_pack_weight: NULL buffer");
  if (rows < 16 || cols < 32 || rows % 16 || cols % 32)
    return fail(MV_EUNSUPPORTED, "mv_pack_weight: rows %d / cols %d not multiples of 16 / 32", rows, cols);
  if (src == dst) return fail(MV_EINVAL, "mv_pack_weight: src and dst overlap");
  int rope_hd = 0, rope_rows = 0;
  if (layout == MV_PACK_QKV) {
    if (rows != 3 * cols || (hd != 16 && hd != 32 && hd != 64 && hd != 128) || cols % hd)
      return fail(MV_EINVAL, "mv_pack_weight: QKV layout needs rows = 3*cols and a valid hd");
    rope_hd = hd;
    rope_rows = 2 * cols;
  } else if (layout != MV_PACK_PLAIN) {
    return fail(MV_EINVAL, "mv_pack_weight: unknown layout %d", layout);
  }
  MV_HIP(mvk::launch_pack(static_cast<const u16*>(src), static_cast<u16*>(dst), rows, cols, rope_hd,
                          rope_rows, (hipStream_t)stream));
  return MV_OK;
}

MV_API int mv_workspace_size(const mv_dims* dims, int32_t B, int32_t T, int32_t cap, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_batch(B))) return rc;
  if (T < 1 || T > MV_MAX_T) return fail(MV_EUNSUPPORTED, "T=%d outside [1,%d]", T, MV_MAX_T);
  if (!bytes) return fail(MV_EINVAL, "bytes is NULL");
  (void)cap;
  *bytes = ws_layout(*dims, B, T).total;
  return MV_OK;
}

static int check_ws(const mv_dims* dims, int B, int T, size_t ws_bytes, const void* ws) {
  const size_t need = ws_layout(*dims, B, T).total;
  if (!ws || ws_bytes < need)
    return fail(MV_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return MV_OK;
}

static int check_kv(const mv_kv* kv, const mv_dims* D, int B, int T) {
  if (!kv || !kv->k || !kv->v) return fail(MV_EINVAL, "kv buffers must be non-NULL");
  if (kv->L != D->L || kv->B != B || kv->H != D->H || kv->hd != D->hd)
    return fail(MV_EINVAL, "kv shape (L=%d B=%d H=%d hd=%d) does not match", kv->L, kv->B, kv->H, kv->hd);
  if (kv->cap < T || kv->cap % 64) return fail(MV_ECAPACITY, "kv cap %d must be a multiple of 64 >= T", kv->cap);
  return MV_OK;
}

MV_API int mv_medusa_heads(const mv_dims* dims, int32_t B, int32_t D, int32_t s, const void* h,
                           const void* w1, const void* w2, const mv_tree* tree,
                           const int32_t* root_tok, int32_t* top_ids, float* top_vals,
                           int32_t* tree_tok, float* head_logits, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_batch(B))) return rc;
  if (D < 1 || D > dims->K) return fail(MV_EINVAL, "heads used D=%d outside [1,K=%d]", D, dims->K);
  if (s < 1 || s > MV_MAX_TOPK || s > dims->V) return fail(MV_EUNSUPPORTED, "s=%d outside [1,%d]", s, MV_MAX_TOPK);
  if (!h || !w1 || !w2 || !top_ids || !top_vals) return fail(MV_EINVAL, "mv_medusa_heads: NULL pointer");
  if (tree) {
    if ((rc = check_tree(tree, false))) return rc;
    if (tree->depth > D) return fail(MV_ETREE, "tree depth %d > heads used %d", tree->depth, D);
    if (!root_tok || !tree_tok) return fail(MV_EINVAL, "root_tok and tree_tok needed with a tree");
  }
  if ((size_t)B * dims->d * 4 > 160 * 1024) return fail(MV_EUNSUPPORTED, "B*d too large for the head GEMV");
  if ((rc = check_ws(dims, B, tree ? tree->T : 1, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, tree ? tree->T : 1);
  float* z = head_logits ? head_logits : at<float>(ws, L.hz);
  return enq_heads(*dims, B, D, s, h, w1, w2, tree, root_tok, top_ids, top_vals, tree_tok, z, ws,
                   L, (hipStream_t)stream);
}

MV_API int mv_tree_attention(const mv_dims* dims, int32_t B, const mv_tree* tree,
                             const int32_t* n_prefix, const void* q, const mv_kv* kv,
                             int32_t layer, void* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_batch(B))) return rc;
  if ((rc = check_tree(tree, true))) return rc;
  if ((rc = check_kv(kv, dims, B, tree->T))) return rc;
  if (layer < 0 || layer >= dims->L) return fail(MV_EINVAL, "layer %d outside [0,%d)", layer, dims->L);
  if (!n_prefix || !q || !out) return fail(MV_EINVAL, "mv_tree_attention: NULL pointer");
  if ((rc = check_ws(dims, B, tree->T, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, tree->T);
  return enq_attention(*dims, B, *tree, n_prefix, static_cast<const u16*>(q), *kv, layer,
                       static_cast<u16*>(out), 0, ws, L, (hipStream_t)stream);
}

MV_API int mv_decoder_layer(const mv_dims* dims, int32_t B, const mv_tree* tree,
                            const int32_t* n_prefix, const mv_layer_weights* w, const mv_kv* kv,
                            int32_t layer, float* x, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_batch(B))) return rc;
  if ((rc = check_tree(tree, true))) return rc;
  if ((rc = check_kv(kv, dims, B, tree->T))) return rc;
  if (layer < 0 || layer >= dims->L) return fail(MV_EINVAL, "layer %d outside [0,%d)", layer, dims->L);
  if (!w || !w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm || !w->wgate || !w->wup ||
      !w->wdown || !x || !n_prefix)
    return fail(MV_EINVAL, "mv_decoder_layer: NULL pointer");
  if ((rc = check_ws(dims, B, tree->T, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, tree->T);
  if ((rc = enq_rope(*dims, B, *tree, n_prefix, ws, L, (hipStream_t)stream))) return rc;
  return enq_layer(*dims, B, *tree, n_prefix, *w, *kv, layer, x, ws, L, (hipStream_t)stream);
}

MV_API int mv_embed(const mv_dims* dims, int32_t M, const int32_t* tokens, const void* embed,
                    float* x, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1) return fail(MV_EINVAL, "M=%d", M);
  if (!tokens || !embed || !x) return fail(MV_EINVAL, "mv_embed: NULL pointer");
  MV_HIP(mvk::launch_embed(tokens, static_cast<const u16*>(embed), x, M, dims->d, dims->V,
                           (hipStream_t)stream));
  return MV_OK;
}

MV_API int mv_lm_head(const mv_dims* dims, int32_t M, const float* x, const void* final_norm,
                      const void* lm_head, float* logits, void* hn_rows, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1 || M > MV_MAX_BATCH * MV_MAX_T) return fail(MV_EUNSUPPORTED, "M=%d", M);
  if (!x || !final_norm || !lm_head || !logits) return fail(MV_EINVAL, "mv_lm_head: NULL pointer");
  // any (B, T) with B*T >= M gives a large enough xa; use B=1, T=M when M fits
  const int B = (M + MV_MAX_T - 1) / MV_MAX_T, T = (M + B - 1) / B;
  if ((rc = check_ws(dims, B, T, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, T);
  return enq_lm_head(*dims, M, x, final_norm, lm_head, logits, static_cast<u16*>(hn_rows), ws, L,
                     (hipStream_t)stream);
}

MV_API int mv_accept(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                     const mv_tree* tree, const int32_t* tree_tok, const mv_accept_params* p,
                     const double* u, int32_t* accept_len, int32_t* path, int32_t* best,
                     int32_t* next_root, int32_t* emitted, double* margin, const void* hn,
                     void* h_last, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_batch(B);
  if (rc) return rc;
  if ((rc = check_tree(tree, false))) return rc;
  if (tree->T != T) return fail(MV_EINVAL, "T=%d != tree T=%d", T, tree->T);
  if (V < 64 || V % 64) return fail(MV_EUNSUPPORTED, "V=%d", V);
  if (!p || !logits || !tree_tok || !accept_len || !path || !best || !next_root)
    return fail(MV_EINVAL, "mv_accept: NULL pointer");
  if (p->mode != MV_ACCEPT_GREEDY && p->mode != MV_ACCEPT_TYPICAL) return fail(MV_EINVAL, "accept mode %d", p->mode);
  if (p->root_mode != MV_ROOT_ARGMAX && p->root_mode != MV_ROOT_SAMPLE) return fail(MV_EINVAL, "root mode %d", p->root_mode);
  if ((p->mode == MV_ACCEPT_TYPICAL || p->root_mode == MV_ROOT_SAMPLE) && !(p->temperature > 0.f))
    return fail(MV_EINVAL, "temperature must be > 0 for typical acceptance or sampled roots");
  if (p->root_mode == MV_ROOT_SAMPLE && !u) return fail(MV_EINVAL, "sampled root needs u");
  if ((hn == nullptr) != (h_last == nullptr)) return fail(MV_EINVAL, "hn and h_last go together");
  if (hn && (d < 1 || d % 8)) return fail(MV_EINVAL, "d=%d", d);
  // workspace: amax [B*T] int32 + stats [B*T][3] double
  const size_t need = align256((size_t)B * T * 4) + (size_t)B * T * 24;
  if (!ws || ws_bytes < need) return fail(MV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  Ws L{};
  L.amax = 0;
  L.stats = align256((size_t)B * T * 4);
  return enq_accept(B, T, V, d, logits, *tree, tree_tok, *p, u, nullptr, B, accept_len, path, best,
                    next_root, emitted, margin, hn, h_last, ws, L, (hipStream_t)stream);
}

MV_API int mv_kv_compact(const mv_kv* kv, const int32_t* path, int32_t path_stride,
                         const int32_t* accept_len, int32_t* n_prefix, void* stream) {
  if (!kv || !kv->k || !kv->v || !path || !accept_len || !n_prefix)
    return fail(MV_EINVAL, "mv_kv_compact: NULL pointer");
  if (kv->L < 1 || kv->B < 1 || kv->B > MV_MAX_BATCH || kv->H < 1 || kv->hd < 1 || kv->cap % 64)
    return fail(MV_EINVAL, "mv_kv_compact: bad kv shape");
  if (path_stride < 1 || path_stride > MV_MAX_DEPTH + 1)
    return fail(MV_EINVAL, "path_stride %d outside [1,%d]", path_stride, MV_MAX_DEPTH + 1);
  const hipStream_t s = (hipStream_t)stream;
  MV_HIP(mvk::launch_compact(static_cast<u16*>(kv->k), static_cast<u16*>(kv->v), kv->L, kv->B,
                             kv->H, kv->hd, kv->cap, path, path_stride, accept_len, n_prefix, s));
  MV_HIP(mvk::launch_advance(n_prefix, accept_len, kv->B, nullptr, s));
  return MV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Step context
// ---------------------------------------------------------------------------
struct mv_ctx {
  mv_step_desc d;
  std::vector<mv_layer_weights> layers;
  Ws L;
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  // chain tree for prefill [B][T]
  int32_t* chain = nullptr;      // parent | depth | rank  (3 * B * T int32)
  uint64_t* chain_anc = nullptr; // [B][T][mask_words]
  int32_t* chunk_tok = nullptr;  // [B][T]
  std::vector<hipEvent_t> prof_ev;
};

static int enq_step(mv_ctx* c, hipStream_t s) {
  const mv_step_desc& d = c->d;
  const mv_dims& D = d.dims;
  const int B = d.B, T = d.T, M = B * T;
  void* ws = d.ws;
  const Ws& L = c->L;
  int rc;
  const int Dn = d.tree.depth;
  prof_begin(s);
  if (Dn > 0) {
    rc = enq_heads(D, B, Dn, d.s, d.h_last, d.w1, d.w2, &d.tree, d.root_tok,
                   d.top_ids ? d.top_ids : at<int32_t>(ws, L.topi), at<float>(ws, L.topv),
                   d.tree_tok, d.head_logits ? d.head_logits : at<float>(ws, L.hz), ws, L, s);
    if (rc) return rc;
  } else {
    MV_HIP(mvk::launch_tree_fill(at<int32_t>(ws, L.topi), d.root_tok, d.tree.depth_of, d.tree.rank,
                                 d.tree_tok, B, T, 1, d.s, s));
  }
  prof_end(MV_K_HEADS, s);
  float* x = at<float>(ws, L.x);
  prof_begin(s);
  MV_HIP(mvk::launch_embed(d.tree_tok, static_cast<const u16*>(d.embed), x, M, D.d, D.V, s));
  if ((rc = enq_rope(D, B, d.tree, d.n_prefix, ws, L, s))) return rc;
  prof_end(MV_K_EMBED, s);
  for (int l = 0; l < D.L; ++l)
    if ((rc = enq_layer(D, B, d.tree, d.n_prefix, c->layers[l], d.kv, l, x, ws, L, s))) return rc;
  u16* hn = at<u16>(ws, L.hn);
  prof_begin(s);
  if ((rc = enq_lm_head(D, M, x, d.final_norm, d.lm_head, d.logits, hn, ws, L, s))) return rc;
  prof_end(MV_K_LM_HEAD, s);
  prof_begin(s);
  if ((rc = enq_accept(B, T, D.V, D.d, d.logits, d.tree, d.tree_tok, d.accept, d.u_draws,
                       d.u_index, B, d.accept_len, d.path, d.best, d.root_tok, d.emitted, nullptr,
                       hn, d.h_last, ws, L, s)))
    return rc;
  prof_end(MV_K_ACCEPT, s);
  prof_begin(s);
  MV_HIP(mvk::launch_compact(static_cast<u16*>(d.kv.k), static_cast<u16*>(d.kv.v), D.L, B, D.H,
                             D.hd, d.kv.cap, d.path, d.tree.depth + 1, d.accept_len, d.n_prefix, s));
  MV_HIP(mvk::launch_advance(d.n_prefix, d.accept_len, B, d.u_index, s));
  prof_end(MV_K_COMPACT, s);
  return MV_OK;
}

extern "C" {

MV_API int mv_ctx_create(mv_ctx** out, const mv_step_desc* desc) {
  if (!out || !desc) return fail(MV_EINVAL, "mv_ctx_create: NULL pointer");
  const mv_step_desc& d = *desc;
  int rc = check_dims(&d.dims);
  if (rc) return rc;
  if ((rc = check_batch(d.B))) return rc;
  if ((rc = check_tree(&d.tree, true))) return rc;
  if (d.tree.T != d.T) return fail(MV_EINVAL, "desc T=%d != tree T=%d", d.T, d.tree.T);
  if (d.tree.depth > d.dims.K) return fail(MV_ETREE, "tree depth %d > K=%d", d.tree.depth, d.dims.K);
  if (d.s < 1 || d.s > MV_MAX_TOPK || d.s > d.dims.V) return fail(MV_EUNSUPPORTED, "s=%d", d.s);
  if ((rc = check_kv(&d.kv, &d.dims, d.B, d.T))) return rc;
  if (!d.layers || !d.embed || !d.final_norm || !d.lm_head || !d.w1 || !d.w2 || !d.n_prefix ||
      !d.root_tok || !d.h_last || !d.tree_tok || !d.logits || !d.accept_len || !d.path ||
      !d.emitted || !d.best)
    return fail(MV_EINVAL, "mv_ctx_create: NULL pointer in desc");
  for (int l = 0; l < d.dims.L; ++l) {
    const mv_layer_weights& w = d.layers[l];
    if (!w.attn_norm || !w.wqkv || !w.wo || !w.ffn_norm || !w.wgate || !w.wup || !w.wdown)
      return fail(MV_EINVAL, "layer %d has a NULL weight", l);
  }
  const mv_accept_params& p = d.accept;
  if (p.mode != MV_ACCEPT_GREEDY && p.mode != MV_ACCEPT_TYPICAL) return fail(MV_EINVAL, "accept mode");
  if (p.root_mode != MV_ROOT_ARGMAX && p.root_mode != MV_ROOT_SAMPLE) return fail(MV_EINVAL, "root mode");
  if ((p.mode == MV_ACCEPT_TYPICAL || p.root_mode == MV_ROOT_SAMPLE) && !(p.temperature > 0.f))
    return fail(MV_EINVAL, "temperature must be > 0");
  if (p.root_mode == MV_ROOT_SAMPLE && (!d.u_draws || !d.u_index || d.n_draws < 1))
    return fail(MV_EINVAL, "sampled roots need u_draws, u_index and n_draws");
  if ((size_t)d.B * d.dims.d * 4 > 160 * 1024) return fail(MV_EUNSUPPORTED, "B*d too large");
  if ((rc = check_ws(&d.dims, d.B, d.T, d.ws_bytes, d.ws))) return rc;

  mv_ctx* c = new mv_ctx();
  c->d = d;
  c->layers.assign(d.layers, d.layers + d.dims.L);
  c->d.layers = nullptr;
  c->L = ws_layout(d.dims, d.B, d.T);
  const int B = d.B, T = d.T, mw = d.tree.mask_words;
  std::vector<int32_t> ch(3 * (size_t)B * T);
  std::vector<uint64_t> ca((size_t)B * T * mw, 0);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < T; ++i) {
      ch[(size_t)b * T + i] = i - 1;
      ch[(size_t)B * T + b * T + i] = i;
      ch[(size_t)2 * B * T + b * T + i] = 0;
      for (int a = 0; a <= i; ++a) ca[((size_t)b * T + i) * mw + (a >> 6)] |= 1ull << (a & 63);
    }
  hipError_t e = hipMalloc(&c->chain, ch.size() * 4);
  if (e == hipSuccess) e = hipMalloc(&c->chain_anc, ca.size() * 8);
  if (e == hipSuccess) e = hipMalloc(&c->chunk_tok, (size_t)B * T * 4);
  if (e == hipSuccess) e = hipMemcpy(c->chain, ch.data(), ch.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->chain_anc, ca.data(), ca.size() * 8, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(c->chunk_tok, 0, (size_t)B * T * 4);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) {
    mv_ctx_destroy(c);
    return fail(MV_EHIP, "mv_ctx_create: %s", hipGetErrorString(e));
  }
  *out = c;
  return MV_OK;
}

MV_API void mv_ctx_destroy(mv_ctx* c) {
  if (!c) return;
  if (c->exec) (void)hipGraphExecDestroy(c->exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->chain) (void)hipFree(c->chain);
  if (c->chain_anc) (void)hipFree(c->chain_anc);
  if (c->chunk_tok) (void)hipFree(c->chunk_tok);
  for (auto e : c->prof_ev) (void)hipEventDestroy(e);
  delete c;
}

MV_API int mv_prefill(mv_ctx* c, const int32_t* ids, int32_t ld, const int32_t* n_ids,
                      void* stream) {
  if (!c || !ids || !n_ids) return fail(MV_EINVAL, "mv_prefill: NULL pointer");
  const mv_step_desc& d = c->d;
  const mv_dims& D = d.dims;
  const int B = d.B, T = d.T, M = B * T;
  int nmax = 0;
  for (int b = 0; b < B; ++b) {
    if (n_ids[b] < 1 || n_ids[b] > d.kv.cap - T || n_ids[b] > ld)
      return fail(MV_ECAPACITY, "prefix length %d of sequence %d outside [1, min(cap-T=%d, ld=%d)]",
                  n_ids[b], b, d.kv.cap - T, ld);
    nmax = std::max(nmax, (int)n_ids[b]);
  }
  const hipStream_t s = (hipStream_t)stream;
  void* ws = d.ws;
  const Ws& L = c->L;
  mv_tree chain{T, T - 1, d.tree.mask_words, c->chain, c->chain + (size_t)B * T,
                c->chain + (size_t)2 * B * T, c->chain_anc};
  MV_HIP(mvk::launch_fill_i32(d.n_prefix, 0, B, s));
  float* x = at<float>(ws, L.x);
  u16* hn = at<u16>(ws, L.hn);
  int32_t* cnt = at<int32_t>(ws, L.cnt);
  const int chunks = (nmax + T - 1) / T;
  std::vector<int32_t> hc(B);
  int rc;
  for (int ci = 0; ci < chunks; ++ci) {
    for (int b = 0; b < B; ++b) {
      const int m = std::max(0, std::min(T, n_ids[b] - ci * T));
      hc[b] = m;
      if (m > 0)
        MV_HIP(hipMemcpyAsync(c->chunk_tok + (size_t)b * T, ids + (size_t)b * ld + (size_t)ci * T,
                              (size_t)m * 4, hipMemcpyDeviceToDevice, s));
    }
    MV_HIP(hipMemcpyAsync(cnt, hc.data(), (size_t)B * 4, hipMemcpyHostToDevice, s));
    MV_HIP(mvk::launch_embed(c->chunk_tok, static_cast<const u16*>(d.embed), x, M, D.d, D.V, s));
    if ((rc = enq_rope(D, B, chain, d.n_prefix, ws, L, s))) return rc;
    for (int l = 0; l < D.L; ++l)
      if ((rc = enq_layer(D, B, chain, d.n_prefix, c->layers[l], d.kv, l, x, ws, L, s))) return rc;
    if ((rc = enq_lm_head(D, M, x, d.final_norm, d.lm_head, d.logits, hn, ws, L, s))) return rc;
    MV_HIP(mvk::launch_row_stats(d.logits, M, D.V, MV_ACCEPT_GREEDY, 1.f, at<int32_t>(ws, L.amax),
                                 at<double>(ws, L.stats), s));
    MV_HIP(mvk::launch_prefill_select(d.logits, at<int32_t>(ws, L.amax), cnt, B, T, D.V,
                                      d.accept.root_mode, d.accept.temperature, d.u_draws,
                                      d.root_tok, d.n_prefix, hn, static_cast<u16*>(d.h_last), D.d,
                                      s));
    // the host-side counts buffer is reused next chunk: wait for the copy
    MV_HIP(hipStreamSynchronize(s));
  }
  if (d.u_index) MV_HIP(mvk::launch_fill_i32(d.u_index, 1, 1, s));
  return MV_OK;
}

MV_API int mv_step(mv_ctx* c, int32_t use_graph, void* stream) {
  if (!c) return fail(MV_EINVAL, "mv_step: NULL context");
  const hipStream_t s = (hipStream_t)stream;
  if (!use_graph) return enq_step(c, s);
  if (!c->exec) {
    MV_HIP(hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    const int rc = enq_step(c, c->cap_stream);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cap_stream, &g);
    if (rc) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return fail(MV_EHIP, "graph capture: %s", hipGetErrorString(e));
    c->graph = g;
    MV_HIP(hipGraphInstantiate(&c->exec, c->graph, nullptr, nullptr, 0));
  }
  MV_HIP(hipGraphLaunch(c->exec, s));
  return MV_OK;
}

MV_API int mv_step_profile(mv_ctx* c, float* ms, int32_t* count, void* stream) {
  if (!c || !ms || !count) return fail(MV_EINVAL, "mv_step_profile: NULL pointer");
  const hipStream_t s = (hipStream_t)stream;
  if (c->prof_ev.empty()) {
    c->prof_ev.resize(2 * 1024);
    for (auto& e : c->prof_ev) MV_HIP(hipEventCreate(&e));
  }
  Prof p;
  p.ev = c->prof_ev.data();
  p.cap = 1024;
  p.n = 0;
  g_prof = &p;
  const int rc = enq_step(c, s);
  g_prof = nullptr;
  if (rc) return rc;
  MV_HIP(hipEventSynchronize(p.ev[2 * p.n - 1]));
  for (int k = 0; k < MV_K_COUNT; ++k) {
    ms[k] = 0.f;
    count[k] = 0;
  }
  for (int i = 0; i < p.n; ++i) {
    float t = 0.f;
    MV_HIP(hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]));
    ms[p.kind[i]] += t;
    count[p.kind[i]] += 1;
  }
  return MV_OK;
}

}  // extern "C"
