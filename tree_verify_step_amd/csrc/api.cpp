// C ABI of the Medusa tree-verify library: argument validation, workspace
// carving, kernel sequencing for each operation, and the step driver that
// captures one whole decoding step into a hipGraph.
//
// A decoder layer is five launches, six when the attention merges split
// key ranges: QKV GEMM (row-norm scale, RoPE and KV-cache write in its
// epilogue), tree attention (and its merge), O-projection GEMM (residual
// add; writes the FFN norm's operand and the rows' sums of squares), gate/up
// GEMM (row-norm scale, SwiGLU), down GEMM (residual add; writes the next
// norm's operand and sums of squares).  RMSNorm never runs as a kernel of
// its own inside a step; split-K partials are reduced inside the GEMMs.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "internal.hpp"
#include "medusa_verify.h"

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
  if (D->V > MV_MAX_VOCAB) return fail(MV_EUNSUPPORTED, "V=%d > %d", D->V, MV_MAX_VOCAB);
  if (D->d % 64 || D->F % 32 || D->V % 64)
    return fail(MV_EUNSUPPORTED, "need d%%64==0, F%%32==0, V%%64==0 (d=%d F=%d V=%d)", D->d, D->F, D->V);
  if (D->hd != 16 && D->hd != 32 && D->hd != 64 && D->hd != 128)
    return fail(MV_EUNSUPPORTED, "head dim %d not in {16,32,64,128}", D->hd);
  if (D->K > MV_MAX_DEPTH) return fail(MV_EUNSUPPORTED, "K=%d > %d", D->K, MV_MAX_DEPTH);
  if (D->d > 8192) return fail(MV_EUNSUPPORTED, "d=%d > 8192", D->d);
  return MV_OK;
}

// max_depth: MV_MAX_DEPTH where a depth indexes heads or paths; the forward
// itself (attention, decoder layer) takes any depth < T (e.g. chain trees).
static int check_tree(const mv_tree* t, bool need_anc, int max_depth = MV_MAX_DEPTH) {
  if (!t) return fail(MV_EINVAL, "tree is NULL");
  if (t->T < 1 || t->T > MV_MAX_T) return fail(MV_EUNSUPPORTED, "tree T=%d outside [1,%d]", t->T, MV_MAX_T);
  if (t->depth < 0 || t->depth > max_depth || t->depth > t->T - 1)
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
enum GemmKind { G_QKV = 0, G_O, G_GU, G_DOWN, G_LM, G_KINDS };

struct GemmCfg {
  int w, nbw, splits, ntiles, mtiles, MB, N, K, epi;
  int wide;     // 0, or the wide-tile kernel's column blocks per wave
};

// Waves per workgroup and column blocks per wave per GEMM (measured on
// MI355X at M = 64 for the 7B shapes); K is split until the tiles cover the
// 256 compute units, keeping at least two activation chunks per split.
static GemmCfg gemm_cfg(const mv_dims& D, int kind, int Mp) {
  GemmCfg c;
  c.MB = mvk::gemm_mb(Mp);
  switch (kind) {
    case G_QKV: {   // one block per wave, RoPE partners in neighbouring waves: 8-wave tiles
                    // at 128 and 256 rows; up to 64 rows 4-wave tiles of 64 columns, whose
                    // count covers the chip without a K split (7B: 192 tiles)
      const bool split = c.MB >= 8 && (3 * D.d / 16 + 7) / 8 <= 256;
      c.w = split ? 8 : 4; c.nbw = split || c.MB <= 4 ? 1 : 2; c.N = 3 * D.d; c.K = D.d;
      c.epi = mvk::EPI_QKV;
      break;
    }
    case G_O: c.w = 4; c.nbw = 1; c.N = D.d; c.K = D.d; c.epi = mvk::EPI_ADD; break;
    case G_GU: {
      // 128- and 256-row tiles: gate and up blocks in separate waves of 8-
      // or 10-wave workgroups (4 or 5 feature blocks a tile; deeper weight
      // ring) while those tiles fit the compute units in one round;
      // otherwise two blocks per wave
      const int fw = (D.F / 16 + 3) / 4 <= 256 ? 4 : (D.F / 16 + 4) / 5 <= 256 ? 5 : 0;
      const bool split = c.MB >= 8 && fw > 0;
      c.w = split ? 2 * fw : 4; c.nbw = split ? 1 : 2; c.N = D.F; c.K = D.d;
      c.epi = mvk::EPI_SWIGLU;
      break;
    }
    case G_DOWN: c.w = 4; c.nbw = 1; c.N = D.d; c.K = D.F; c.epi = mvk::EPI_ADD; break;
    default:
      c.w = D.V % 128 == 0 ? 8 : 4; c.nbw = 1; c.N = D.V; c.K = D.d; c.epi = mvk::EPI_STORE;
      break;
  }
  c.mtiles = (Mp / 16 + c.MB - 1) / c.MB;
  const int KB = c.K / 32;
  c.wide = 0;
  // More than 128 rows: the wide-tile kernel (256 rows x 128 columns, or x
  // 160 for gate/up when 64-feature tiles would not fit the compute units in
  // one round), whose range-checked operand loads need each operand below
  // 2 GiB.  It takes the launches where it measured faster at 256 rows: K of
  // 6144 and more with fewer than 8 K splits (every 33B GEMM, 13B down:
  // 90 against 137 us at 33B down), gate/up from K = 5120 (13B: 95 against
  // 104 us) and gate/up in the narrow tiles below (7B); the 16-row-block
  // tiles keep the other 7B shapes (prefill 14.7 against 15.7 ms) and 13B
  // QKV and O (67 against 71 us, 37.5 against 40).
  if (c.MB == 16 && (size_t)c.N * c.K * 2 < (1ull << 31) && (size_t)Mp * c.K * 2 < (1ull << 31)) {
    GemmCfg w = c;
    w.wide = 4;
    if (w.epi == mvk::EPI_SWIGLU && mvk::gemm_wide_ntiles(w.epi, w.N, 4) * w.mtiles > 256) w.wide = 5;
    // QKV and gate/up: tiles of 3 column blocks a wave (96 columns; 48
    // features) when those of 4 would leave more than 30% of the compute
    // units idle and the narrower ones still fit in one round (33B QKV: 116
    // against 111 us; 7B gate/up at 256 rows: 77 against 69.5 us)
    bool narrow = false;
    if ((w.epi == mvk::EPI_QKV || w.epi == mvk::EPI_SWIGLU) &&
        mvk::gemm_wide_ntiles(w.epi, w.N, 4) * w.mtiles < 180 &&
        mvk::gemm_wide_ntiles(w.epi, w.N, 3) * w.mtiles <= 256) {
      w.wide = 3;
      narrow = true;
    }
    w.w = 8;
    w.nbw = 1;
    w.ntiles = mvk::gemm_wide_ntiles(w.epi, w.N, w.wide);
    // K splits while the tiles leave compute units idle, each split at least
    // four 2-k-block stages
    w.splits = std::max(1, std::min(256 / (w.ntiles * w.mtiles), KB / 8));
    if ((c.K >= 6144 && w.splits < 8) || (c.epi == mvk::EPI_SWIGLU && (c.K >= 5120 || narrow)))
      return w;
  }
  c.ntiles = mvk::gemm_ntiles(c.epi, c.N, c.w, c.nbw);
  const int KC = mvk::gemm_kc(c.MB);
  c.splits = std::max(1, 256 / (c.ntiles * c.mtiles));
  c.splits = std::max(1, std::min(c.splits, KB / (2 * KC)));
  return c;
}

// Bytes of one K split's partial tile.
static size_t gemm_partial_bytes(const GemmCfg& c) {
  if (c.wide) return (size_t)c.wide * 32768;     // 8 waves x 4 x wide accumulators of 1 KiB
  return (size_t)c.w * c.MB * c.nbw * 256 * sizeof(float);
}

struct Ws {
  size_t x, xa, ao, ha, ss, q, rope, part, counters, apo, apml, hu, hz, topi, topv, tcv,
      tci, amax, amaxp, stats, bsum, cnt, plog, total;
  int ss_ld;    // floats per row of the sums-of-squares buffer
};

// Row stride of the sums of squares: the residual GEMMs' column tiles, rounded to 4.
static int ss_ld_of(const mv_dims& D, int Mp) {
  int t = 1;
  for (int k = 0; k < G_KINDS; ++k) {
    const GemmCfg c = gemm_cfg(D, k, Mp);
    if (c.epi == mvk::EPI_ADD) t = std::max(t, c.ntiles);
  }
  return (t + 3) & ~3;
}

// Row buffers hold B * max(T, P) rows: the step's T-row trees and, when it is
// larger, the prefill's P-row chunks (P <= T: prefill uses T-row chunks).
static Ws ws_layout(const mv_dims& D, int B, int T, int P = 0) {
  Ws w;
  const int R = std::max(T, P);
  const int M = B * R, Mp = round16(M);
  size_t part = 0, max_tiles = 1;
  w.ss_ld = 1;
  for (const int Mq : {round16(B * T), P > T ? Mp : 0}) {
    if (!Mq) continue;
    for (int k = 0; k < G_KINDS; ++k) {
      const GemmCfg c = gemm_cfg(D, k, Mq);
      const size_t tiles = (size_t)c.ntiles * c.mtiles;
      if (c.splits > 1) part = std::max(part, tiles * c.splits * gemm_partial_bytes(c));
      max_tiles = std::max(max_tiles, tiles);
    }
    w.ss_ld = std::max(w.ss_ld, ss_ld_of(D, Mq));
  }
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + std::max<size_t>(bytes, 16));
    return o;
  };
  w.x = take((size_t)M * D.d * 4);
  w.xa = take((size_t)Mp * D.d * 2);
  w.ao = take((size_t)Mp * D.d * 2);
  w.ha = take((size_t)Mp * D.F * 2);
  w.ss = take((size_t)w.ss_ld * Mp * 4);
  w.q = take((size_t)M * D.d * 2);
  w.rope = take((size_t)M * (D.hd / 2) * 8);
  w.part = take(part);
  w.counters = take(max_tiles * 4);
  // tree attention's split states (the step's T-row trees and the prefill's
  // R-row chains)
  size_t apo = 0, apml = 0;
  for (const int Tq : {T, R}) {
    const size_t ps = (size_t)B * D.H * mvk::attention_splits(B, D.H, Tq);
    apo = std::max(apo, ps * (size_t)round16(Tq) * D.hd * 4);
    apml = std::max(apml, ps * Tq * 8);
  }
  w.apo = take(apo);
  w.apml = take(apml);
  w.hu = take((size_t)B * D.K * D.d * 4);
  w.hz = take((size_t)B * D.K * D.V * 4);
  w.topi = take((size_t)B * D.K * MV_MAX_TOPK * 4);
  w.topv = take((size_t)B * D.K * MV_MAX_TOPK * 4);
  w.tcv = take((size_t)B * D.K * mvk::topk_waves(D.V) * MV_MAX_TOPK * 4);
  w.tci = take((size_t)B * D.K * mvk::topk_waves(D.V) * MV_MAX_TOPK * 4);
  w.amax = take((size_t)M * 4);
  w.amaxp = take((size_t)M * 8);
  w.stats = take((size_t)M * 3 * 8);
  w.bsum = take((size_t)M * ((D.V + 255) / 256) * 8);   // rows' 256-id block sums
  w.cnt = take((size_t)B * 4);
  w.plog = P > T ? take((size_t)B * P * D.V * 4) : 0;   // prefill chunks' logits
  w.total = off;
  return w;
}

template <class T>
static inline T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

static size_t kv_layer_elems(const mv_kv& kv) { return (size_t)kv.B * kv.H * kv.cap * kv.hd; }

static mvk::GemmArgs gemm_args(const mv_dims& D, int kind, int M, void* ws, const Ws& L) {
  mvk::GemmArgs g{};
  const int Mp = round16(M);
  const GemmCfg c = gemm_cfg(D, kind, Mp);
  g.M = M;
  g.Mp = Mp;
  g.N = c.N;
  g.K = c.K;
  g.w = c.w;
  g.nbw = c.nbw;
  g.splits = c.splits;
  g.epi = c.epi;
  g.wide = c.wide;
  g.ss_ld = L.ss_ld;
  g.partial = at<float>(ws, L.part);
  g.counters = at<int>(ws, L.counters);
  return g;
}

// Column tiles of a residual GEMM = entries per row of the sums of squares it writes.
static int ss_tiles_of(const mv_dims& D, int kind, int M) {
  return gemm_cfg(D, kind, round16(M)).ntiles;
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
static int enq_attention(const mv_dims& D, int B, const mv_tree& t, const int32_t* n_prefix,
                         const u16* q, const mv_kv& kv, int layer, u16* out, int packed,
                         void* ws, const Ws& L, hipStream_t s) {
  const size_t le = kv_layer_elems(kv);
  const u16* kc = static_cast<const u16*>(kv.k) + (size_t)layer * le;
  const u16* vc = static_cast<const u16*>(kv.v) + (size_t)layer * le;
  MV_HIP(mvk::launch_attention(q, kc, vc, n_prefix, t.anc, B, t.T, D.H, D.hd, kv.cap,
                               t.mask_words, out, packed, at<float>(ws, L.apo),
                               at<float2>(ws, L.apml), s));
  return MV_OK;
}

// Normalised-GEMM operand of x: xa = bf16(x * gain) packed, ss[0][m] = sum x^2.
static int enq_norm_prep(const mv_dims& D, int M, const float* x, const void* gain, void* ws,
                         const Ws& L, hipStream_t s) {
  MV_HIP(mvk::launch_norm_prep(x, static_cast<const u16*>(gain), at<u16>(ws, L.xa),
                               at<float>(ws, L.ss), L.ss_ld, M, D.d, s));
  return MV_OK;
}

// One decoder layer over the B*T rows of x.  On entry ws.xa holds
// bf16(x * attn_norm) and ws.ss the rows' sums of squares in ss_tiles_in
// entries (ws.rope the RoPE tables).  With next_gain the down GEMM leaves the
// same for the next norm (entries: ss_tiles_of(G_DOWN)).
static int enq_layer(const mv_dims& D, int B, const mv_tree& t, const int32_t* n_prefix,
                     const mv_layer_weights& w, const mv_kv& kv, int layer, float* x,
                     int ss_tiles_in, const void* next_gain, void* ws, const Ws& L,
                     hipStream_t s, int only_kind = -1) {
  auto want = [&](int kind) { return only_kind < 0 || only_kind == kind; };
  const int M = B * t.T;
  u16* xa = at<u16>(ws, L.xa);
  u16* ao = at<u16>(ws, L.ao);
  u16* ha = at<u16>(ws, L.ha);
  u16* q = at<u16>(ws, L.q);
  float* ss = at<float>(ws, L.ss);
  const size_t le = kv_layer_elems(kv);

  mvk::GemmArgs g = gemm_args(D, G_QKV, M, ws, L);
  g.A = xa;
  g.W = static_cast<const u16*>(w.wqkv);
  g.ss = ss;
  g.ss_tiles = ss_tiles_in;
  g.qkv.q = q;
  g.qkv.kcache = static_cast<u16*>(kv.k) + (size_t)layer * le;
  g.qkv.vcache = static_cast<u16*>(kv.v) + (size_t)layer * le;
  g.qkv.n_prefix = n_prefix;
  g.qkv.rope = at<float2>(ws, L.rope);
  g.qkv.B = B;
  g.qkv.T = t.T;
  g.qkv.H = D.H;
  g.qkv.hd = D.hd;
  g.qkv.cap = kv.cap;
  g.qkv.d = D.d;
  {   // compute units the QKV tiles leave idle read the prefix K/V ahead
    const GemmCfg c = gemm_cfg(D, G_QKV, round16(M));
    g.prefetch = c.wide ? 0 : std::max(0, (256 - c.ntiles * c.splits * c.mtiles) / (c.splits * c.mtiles));
    // half the weight bytes one tile workgroup streams
    g.pf_budget16 = (int)((size_t)c.N * c.K * 2 / ((size_t)c.ntiles * c.splits * c.mtiles) / 2 / 16);
  }
  if (want(MV_K_QKV)) {
    prof_begin(s);
    MV_HIP(mvk::launch_gemm(g, s));
    prof_end(MV_K_QKV, s);
  }

  if (want(MV_K_ATTN)) {
    prof_begin(s);
    const int rc = enq_attention(D, B, t, n_prefix, q, kv, layer, ao, 1, ws, L, s);
    if (rc) return rc;
    prof_end(MV_K_ATTN, s);
  }

  mvk::GemmArgs o = gemm_args(D, G_O, M, ws, L);
  o.A = ao;
  o.W = static_cast<const u16*>(w.wo);
  o.out_f32 = x;
  o.next_gain = static_cast<const u16*>(w.ffn_norm);
  o.xn_out = xa;
  o.ss_out = ss;
  if (want(MV_K_O)) {
    prof_begin(s);
    MV_HIP(mvk::launch_gemm(o, s));
    prof_end(MV_K_O, s);
  }

  mvk::GemmArgs gu = gemm_args(D, G_GU, M, ws, L);
  gu.A = xa;
  gu.W = static_cast<const u16*>(w.wgate);
  gu.W2 = static_cast<const u16*>(w.wup);
  gu.ss = ss;
  gu.ss_tiles = ss_tiles_of(D, G_O, M);
  gu.out_bf16 = ha;
  if (want(MV_K_GATE_UP)) {
    prof_begin(s);
    MV_HIP(mvk::launch_gemm(gu, s));
    prof_end(MV_K_GATE_UP, s);
  }

  mvk::GemmArgs dn = gemm_args(D, G_DOWN, M, ws, L);
  dn.A = ha;
  dn.W = static_cast<const u16*>(w.wdown);
  dn.out_f32 = x;
  dn.next_gain = static_cast<const u16*>(next_gain);
  dn.xn_out = xa;
  dn.ss_out = ss;
  if (want(MV_K_DOWN)) {
    prof_begin(s);
    MV_HIP(mvk::launch_gemm(dn, s));
    prof_end(MV_K_DOWN, s);
  }
  return MV_OK;
}

// LM head: logits [M][V] fp32 of rmsnorm(x) * final_norm.  With ss_tiles > 0
// ws.xa / ws.ss already hold the final norm's operand (left by the last
// layer); otherwise it is prepared from x here.
static int enq_lm_head(const mv_dims& D, int M, const float* x, const void* final_norm,
                       const void* lm, float* logits, int ss_tiles, void* ws, const Ws& L,
                       hipStream_t s, unsigned long long* amax_key = nullptr,
                       int32_t* status = nullptr) {
  if (ss_tiles <= 0) {
    const int rc = enq_norm_prep(D, M, x, final_norm, ws, L, s);
    if (rc) return rc;
    ss_tiles = 1;
  }
  mvk::GemmArgs g = gemm_args(D, G_LM, M, ws, L);
  g.A = at<u16>(ws, L.xa);
  g.W = static_cast<const u16*>(lm);
  g.ss = at<float>(ws, L.ss);
  g.ss_tiles = ss_tiles;
  g.out_f32 = logits;
  g.amax_key = amax_key;
  g.status = status;
  MV_HIP(mvk::launch_gemm(g, s));
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
  MV_HIP(mvk::launch_topk(z, B * Dn, D.V, s_top, top_ids, top_vals, at<float>(ws, L.tcv),
                          at<int>(ws, L.tci), s));
  if (tree && tree_tok)
    MV_HIP(mvk::launch_tree_fill(top_ids, root, tree->depth_of, tree->rank, tree_tok, B, tree->T,
                                 Dn, s_top, s));
  return MV_OK;
}

static int enq_accept(int B, int T, int V, int d, const float* logits, const mv_tree& t,
                      const int32_t* tok, const mv_accept_params& p, const double* u,
                      const int32_t* u_index, int u_stride, int32_t* accept_len, int32_t* path,
                      int32_t* best, int32_t* next_root, int32_t* emitted, double* margin,
                      const float* x, const void* final_norm, void* h_last, int32_t* amax,
                      double* stats, double* bsum, hipStream_t s,
                      unsigned long long* amax_key = nullptr, int32_t* n_advance = nullptr,
                      mvk::StepGuard guard = {}) {
  if (p.mode == MV_ACCEPT_REJECT) {
    MV_HIP(mvk::launch_row_stats(logits, B * T, V, p.mode, p.temperature, amax, stats, s, bsum));
    MV_HIP(mvk::launch_reject_accept(logits, amax, stats, t.parent, tok, B, T, V, t.depth,
                                     p.temperature, nullptr, nullptr, u, u_index, (long long)u_stride,
                                     nullptr, accept_len, path, best, next_root, emitted, margin,
                                     x, static_cast<const u16*>(final_norm),
                                     static_cast<u16*>(h_last), d, s, n_advance, bsum, guard));
    return MV_OK;
  }
  // greedy acceptance with the LM head's argmax keys needs no pass over the
  // logits; otherwise the rows' argmax (and typical statistics)
  if (!(amax_key && p.mode == MV_ACCEPT_GREEDY)) {
    amax_key = nullptr;
    MV_HIP(mvk::launch_row_stats(logits, B * T, V, p.mode, p.temperature, amax, stats, s,
                                 p.mode == MV_ACCEPT_GREEDY ? nullptr : bsum));
  }
  MV_HIP(mvk::launch_accept_finish(logits, amax, amax_key, stats, t.parent, t.depth_of, tok, B, T, V,
                                   t.depth, p.mode, p.root_mode, p.temperature, p.eps, p.delta, u,
                                   u_index, u_stride, accept_len, path, best, next_root, emitted,
                                   margin, x, static_cast<const u16*>(final_norm),
                                   static_cast<u16*>(h_last), d, s, n_advance,
                                   p.mode == MV_ACCEPT_GREEDY ? nullptr : bsum, guard));
  return MV_OK;
}

}  // namespace mv

namespace mvk {
// heads.hip: calibration counts of the heads' ranks
hipError_t launch_head_accuracy(const int32_t* top_ids, const int32_t* labels, int N, int K, int s,
                                int32_t* counts, hipStream_t st);
// Streaming read of buf (rows.hip: 4096 workgroups, each its own contiguous
// slice; the bytes of the last partial 64 KiB of a slice are skipped).
hipError_t launch_read_probe(const void* buf, size_t bytes, float* sink, hipStream_t s);
}  // namespace mvk

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

MV_API int mv_workspace_size_prefill(const mv_dims* dims, int32_t B, int32_t T,
                                     int32_t prefill_rows, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_batch(B))) return rc;
  if (T < 1 || T > MV_MAX_T) return fail(MV_EUNSUPPORTED, "T=%d outside [1,%d]", T, MV_MAX_T);
  if (prefill_rows != 0 && (prefill_rows < T || prefill_rows > MV_MAX_T))
    return fail(MV_EUNSUPPORTED, "prefill_rows=%d outside {0} or [T=%d, %d]", prefill_rows, T, MV_MAX_T);
  if (!bytes) return fail(MV_EINVAL, "bytes is NULL");
  *bytes = ws_layout(*dims, B, T, prefill_rows).total;
  return MV_OK;
}

static int check_ws(const mv_dims* dims, int B, int T, size_t ws_bytes, const void* ws, int P = 0) {
  const size_t need = ws_layout(*dims, B, T, P).total;
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

MV_API int mv_head_accuracy(int32_t N, int32_t K, int32_t s, const int32_t* top_ids,
                            const int32_t* labels, int32_t* counts, void* stream) {
  if (N < 0 || K < 1 || K > MV_MAX_DEPTH || s < 1 || s > MV_MAX_TOPK)
    return fail(MV_EINVAL, "mv_head_accuracy: N=%d K=%d s=%d", N, K, s);
  if ((int64_t)N * K > ((int64_t)1 << 30)) return fail(MV_EINVAL, "N*K too large");
  if (N > 0 && (!top_ids || !labels || !counts))
    return fail(MV_EINVAL, "mv_head_accuracy: NULL pointer");
  MV_HIP(mvk::launch_head_accuracy(top_ids, labels, N, K, s, counts, (hipStream_t)stream));
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
  if ((size_t)B * dims->d * 4 > MV_HEADS_LDS_MAX) return fail(MV_EUNSUPPORTED, "B*d too large for the head GEMV");
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
  if ((rc = check_tree(tree, true, MV_MAX_T - 1))) return rc;
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
  if ((rc = check_tree(tree, true, MV_MAX_T - 1))) return rc;
  if ((rc = check_kv(kv, dims, B, tree->T))) return rc;
  if (layer < 0 || layer >= dims->L) return fail(MV_EINVAL, "layer %d outside [0,%d)", layer, dims->L);
  if (!w || !w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm || !w->wgate || !w->wup ||
      !w->wdown || !x || !n_prefix)
    return fail(MV_EINVAL, "mv_decoder_layer: NULL pointer");
  if ((rc = check_ws(dims, B, tree->T, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, tree->T);
  const hipStream_t s = (hipStream_t)stream;
  MV_HIP(mvk::launch_rope_table(n_prefix, tree->depth_of, at<float2>(ws, L.rope), B, tree->T,
                                dims->hd, s));
  if ((rc = enq_norm_prep(*dims, B * tree->T, x, w->attn_norm, ws, L, s))) return rc;
  return enq_layer(*dims, B, *tree, n_prefix, *w, *kv, layer, x, 1, nullptr, ws, L, s);
}

MV_API int mv_embed(const mv_dims* dims, int32_t M, const int32_t* tokens, const void* embed,
                    float* x, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1) return fail(MV_EINVAL, "M=%d", M);
  if (!tokens || !embed || !x) return fail(MV_EINVAL, "mv_embed: NULL pointer");
  MV_HIP(mvk::launch_embed(tokens, static_cast<const u16*>(embed), x, nullptr, M, dims->d, dims->V,
                           nullptr, nullptr, nullptr, 1, dims->hd, (hipStream_t)stream));
  return MV_OK;
}

MV_API int mv_lm_head(const mv_dims* dims, int32_t M, const float* x, const void* final_norm,
                      const void* lm_head, float* logits, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (M < 1 || M > MV_MAX_BATCH * MV_MAX_T) return fail(MV_EUNSUPPORTED, "M=%d", M);
  if (!x || !final_norm || !lm_head || !logits) return fail(MV_EINVAL, "mv_lm_head: NULL pointer");
  // any (B, T) with B*T >= M gives large enough buffers; use the smallest B
  const int B = (M + MV_MAX_T - 1) / MV_MAX_T, T = (M + B - 1) / B;
  if ((rc = check_ws(dims, B, T, ws_bytes, ws))) return rc;
  const Ws L = ws_layout(*dims, B, T);
  const hipStream_t s = (hipStream_t)stream;
  return enq_lm_head(*dims, M, x, final_norm, lm_head, logits, 0, ws, L, s);
}

// ---------------------------------------------------------------------------
// Acceptance without a caller workspace (mv_accept_noalloc): the scratch
// lives in a static device array of this library, one per GPU, found by its
// symbol address once per device.  Host code passes only that address to the
// kernels (the array's name is a host-side stand-in, not a device address).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MV_NOALLOC_SCRATCH_BYTES];

#define MV_NOALLOC_MAX_DEVICES 64
static std::once_flag g_scratch_once[MV_NOALLOC_MAX_DEVICES];
static void* g_scratch_ptr[MV_NOALLOC_MAX_DEVICES];
static hipError_t g_scratch_err[MV_NOALLOC_MAX_DEVICES];

// Bytes of acceptance scratch: row argmax int32 [B*T] and row stats double
// [B*T][3] (each part 256-aligned), then for typical acceptance and
// rejection sampling the rows' 256-id block sums double [B*T][ceil(V/256)].
static size_t accept_ws_need(int B, int T, int V, int mode) {
  const size_t head = align256((size_t)B * T * 4) + align256((size_t)B * T * 24);
  const size_t sums = (size_t)B * T * ((V + 255) / 256) * 8;
  if (mode == MV_ACCEPT_GREEDY) return head;
  return head + (mode == MV_ACCEPT_REJECT ? align256(sums) : sums);
}

MV_API int mv_accept(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                     const mv_tree* tree, const int32_t* tree_tok, const mv_accept_params* p,
                     const double* u, int32_t* accept_len, int32_t* path, int32_t* best,
                     int32_t* next_root, int32_t* emitted, double* margin, const float* x,
                     const void* final_norm, void* h_last, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_batch(B);
  if (rc) return rc;
  if ((rc = check_tree(tree, false))) return rc;
  if (tree->T != T) return fail(MV_EINVAL, "T=%d != tree T=%d", T, tree->T);
  if (V < 64 || V % 64 || V > MV_MAX_VOCAB) return fail(MV_EUNSUPPORTED, "V=%d", V);
  if (!p || !logits || !tree_tok || !accept_len || !path || !best || !next_root)
    return fail(MV_EINVAL, "mv_accept: NULL pointer");
  if (p->mode == MV_ACCEPT_REJECT)
    return mv_accept_reject(B, T, V, d, logits, tree, tree_tok, p->temperature, nullptr, u,
                            accept_len, path, best, next_root, emitted, margin, x, final_norm,
                            h_last, ws, ws_bytes, stream);
  if (p->mode != MV_ACCEPT_GREEDY && p->mode != MV_ACCEPT_TYPICAL) return fail(MV_EINVAL, "accept mode %d", p->mode);
  if (p->root_mode != MV_ROOT_ARGMAX && p->root_mode != MV_ROOT_SAMPLE) return fail(MV_EINVAL, "root mode %d", p->root_mode);
  if ((p->mode == MV_ACCEPT_TYPICAL || p->root_mode == MV_ROOT_SAMPLE) && !(p->temperature > 0.0))
    return fail(MV_EINVAL, "temperature must be > 0 for typical acceptance or sampled roots");
  if (p->root_mode == MV_ROOT_SAMPLE && !u) return fail(MV_EINVAL, "sampled root needs u");
  if ((x == nullptr) != (h_last == nullptr) || (x && !final_norm))
    return fail(MV_EINVAL, "x, final_norm and h_last go together");
  if (x && (d < 1 || d % 4)) return fail(MV_EINVAL, "d=%d", d);
  // workspace: amax [B*T] int32, stats [B*T][3] double, then (typical)
  // the rows' 256-id block sums [B*T][ceil(V/256)] double
  const size_t o_stats = align256((size_t)B * T * 4);
  const size_t o_bsum = o_stats + align256((size_t)B * T * 24);
  const bool sums = p->mode == MV_ACCEPT_TYPICAL;
  const size_t need = o_bsum + (sums ? (size_t)B * T * ((V + 255) / 256) * 8 : 0);
  if (!ws || ws_bytes < need) return fail(MV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  return enq_accept(B, T, V, d, logits, *tree, tree_tok, *p, u, nullptr, B, accept_len, path, best,
                    next_root, emitted, margin, x, final_norm, h_last, at<int32_t>(ws, 0),
                    at<double>(ws, o_stats), sums ? at<double>(ws, o_bsum) : nullptr,
                    (hipStream_t)stream);
}

MV_API int mv_accept_noalloc(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                             const mv_tree* tree, const int32_t* tree_tok,
                             const mv_accept_params* p, const double* u, int32_t* accept_len,
                             int32_t* path, int32_t* best, int32_t* next_root, int32_t* emitted,
                             double* margin, const float* x, const void* final_norm,
                             void* h_last, void* stream) {
  int rc = check_batch(B);
  if (rc) return rc;
  if (!p) return fail(MV_EINVAL, "mv_accept_noalloc: NULL params");
  if (T < 1 || T > MV_MAX_T) return fail(MV_EUNSUPPORTED, "T=%d outside [1,%d]", T, MV_MAX_T);
  if (V < 64 || V % 64 || V > MV_MAX_VOCAB) return fail(MV_EUNSUPPORTED, "V=%d", V);
  if (p->mode != MV_ACCEPT_GREEDY && p->mode != MV_ACCEPT_TYPICAL && p->mode != MV_ACCEPT_REJECT)
    return fail(MV_EINVAL, "accept mode %d", p->mode);
  const size_t need = accept_ws_need(B, T, V, p->mode);
  if (need > MV_NOALLOC_SCRATCH_BYTES)
    return fail(MV_EWORKSPACE,
                "mv_accept_noalloc: B=%d T=%d V=%d needs %zu bytes of scratch, more than the "
                "library's static %u bytes (use mv_accept with a workspace)",
                B, T, V, need, (unsigned)MV_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  MV_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= MV_NOALLOC_MAX_DEVICES)
    return fail(MV_EUNSUPPORTED, "mv_accept_noalloc: device %d >= %d", dev, MV_NOALLOC_MAX_DEVICES);
  // once per device, with that device current: the array's device address
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(MV_EHIP, "mv_accept_noalloc: hipGetSymbolAddress: %s",
                hipGetErrorString(g_scratch_err[dev]));
  return mv_accept(B, T, V, d, logits, tree, tree_tok, p, u, accept_len, path, best, next_root,
                   emitted, margin, x, final_norm, h_last, g_scratch_ptr[dev],
                   MV_NOALLOC_SCRATCH_BYTES, stream);
}

MV_API int mv_accept_reject(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                            const mv_tree* tree, const int32_t* tree_tok, double temperature,
                            const float* draft_logits, const double* u, int32_t* accept_len,
                            int32_t* path, int32_t* best, int32_t* next_root, int32_t* emitted,
                            double* margin, const float* x, const void* final_norm, void* h_last,
                            void* ws, size_t ws_bytes, void* stream) {
  int rc = check_batch(B);
  if (rc) return rc;
  if ((rc = check_tree(tree, false))) return rc;
  if (tree->T != T) return fail(MV_EINVAL, "T=%d != tree T=%d", T, tree->T);
  if (V < 64 || V % 64 || V > MV_MAX_VOCAB) return fail(MV_EUNSUPPORTED, "V=%d", V);
  if (!logits || !tree_tok || !u || !accept_len || !path || !best || !next_root)
    return fail(MV_EINVAL, "mv_accept_reject: NULL pointer");
  if (!(temperature > 0.0)) return fail(MV_EINVAL, "temperature must be > 0");
  if (draft_logits && tree->depth < 1) return fail(MV_EINVAL, "draft logits need a tree of depth >= 1");
  if ((x == nullptr) != (h_last == nullptr) || (x && !final_norm))
    return fail(MV_EINVAL, "x, final_norm and h_last go together");
  if (x && (d < 1 || d % 4)) return fail(MV_EINVAL, "d=%d", d);
  // workspace: row argmax and stats of the tree rows, then (draft logits)
  // those of the draft rows and two residual rows per sequence
  const int Dr = draft_logits ? B * tree->depth : 0;
  const size_t o_stats = align256((size_t)B * T * 4);
  const size_t o_bsum = o_stats + align256((size_t)B * T * 24);
  const size_t o_damax = o_bsum + align256((size_t)B * T * ((V + 255) / 256) * 8);
  const size_t o_dstats = o_damax + align256((size_t)Dr * 4);
  const size_t o_res = o_dstats + align256((size_t)Dr * 24);
  const size_t need = draft_logits ? o_res + (size_t)B * 2 * V * 8 : o_damax;
  if (!ws || ws_bytes < need) return fail(MV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  const hipStream_t s = (hipStream_t)stream;
  MV_HIP(mvk::launch_row_stats(logits, B * T, V, MV_ACCEPT_REJECT, temperature, at<int32_t>(ws, 0),
                               at<double>(ws, o_stats), s, at<double>(ws, o_bsum)));
  if (draft_logits)
    MV_HIP(mvk::launch_row_stats(draft_logits, Dr, V, MV_ACCEPT_REJECT, temperature,
                                 at<int32_t>(ws, o_damax), at<double>(ws, o_dstats), s));
  MV_HIP(mvk::launch_reject_accept(logits, at<int32_t>(ws, 0), at<double>(ws, o_stats), tree->parent,
                                   tree_tok, B, T, V, tree->depth, temperature, draft_logits,
                                   draft_logits ? at<double>(ws, o_dstats) : nullptr, u,
                                   nullptr, 0, draft_logits ? at<double>(ws, o_res) : nullptr,
                                   accept_len, path, best, next_root, emitted, margin, x,
                                   static_cast<const u16*>(final_norm), static_cast<u16*>(h_last),
                                   d, s, nullptr, at<double>(ws, o_bsum)));
  return MV_OK;
}

// ---------------------------------------------------------------------------
// Medusa-1 head loss and gradients (train.hip)
// ---------------------------------------------------------------------------
struct TrainWs {
  size_t a, s, z, g, gt, st, w2t, ds, da, dat, ht, ltk, total;
};

static TrainWs train_ws(const mv_dims& D, int N) {
  TrainWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t Nd = (size_t)N * D.d, NV = (size_t)N * D.V;
  w.a = take(Nd * 4);                     // a = H W1^T (fp32)
  w.s = take(Nd * 2);                     // s = SiLU(a) + H (bf16)
  w.z = take(NV * 4);                     // logits (fp32)
  w.g = take(NV * 2);                     // logits' gradient (bf16)
  w.gt = take(NV * 2);                    // ... transposed [V][N]
  w.st = take(Nd * 2);                    // s transposed [d][N]
  w.w2t = take((size_t)D.V * D.d * 2);    // W2 transposed [d][V]
  w.ds = take(Nd * 4);                    // ds (fp32)
  w.da = take(Nd * 2);                    // da (bf16)
  w.dat = take(Nd * 2);                   // da transposed [d][N]
  w.ht = take(Nd * 2);                    // H transposed [d][N]
  w.ltk = take((size_t)N * D.K * 4);      // per-position losses when the caller keeps none
  w.total = off;
  return w;
}

static int check_train(const mv_dims* dims, int N) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (N < 64 || N % 64 || N > (1 << 20))
    return fail(MV_EUNSUPPORTED, "positions N=%d: need a multiple of 64 in [64, 2^20]", N);
  return MV_OK;
}

MV_API int mv_medusa1_workspace_size(const mv_dims* dims, int32_t N, size_t* bytes) {
  int rc = check_train(dims, N);
  if (rc) return rc;
  if (!bytes) return fail(MV_EINVAL, "bytes is NULL");
  *bytes = train_ws(*dims, N).total;
  return MV_OK;
}

MV_API int mv_medusa1_loss(const mv_dims* dims, int32_t N, int32_t K, const void* h,
                           const int32_t* labels, const double* lambda, const void* w1,
                           const void* w2, double* loss, float* loss_tk, float* dw1, float* dw2,
                           void* ws, size_t ws_bytes, void* stream) {
  int rc = check_train(dims, N);
  if (rc) return rc;
  const mv_dims& D = *dims;
  if (K < 1 || K > D.K) return fail(MV_EINVAL, "heads K=%d outside [1, dims.K=%d]", K, D.K);
  if (!h || !labels || !w1 || !w2 || !loss) return fail(MV_EINVAL, "mv_medusa1_loss: NULL pointer");
  double lam[MV_MAX_DEPTH];
  for (int k = 0; k < K; ++k) {
    lam[k] = lambda ? lambda[k] : 0.8;
    if (!lambda)
      for (int j = 0; j < k; ++j) lam[k] *= 0.8;        // 0.8^(k+1) for head k+1
    if (!(lam[k] >= 0.0) || !(lam[k] < 1e30)) return fail(MV_EINVAL, "lambda[%d] = %g", k, lam[k]);
  }
  const TrainWs L = train_ws(D, N);
  if (!ws || ws_bytes < L.total)
    return fail(MV_EWORKSPACE, "workspace %zu < %zu", ws_bytes, L.total);
  const hipStream_t s = (hipStream_t)stream;
  const int d = D.d, V = D.V;
  const u16* H = static_cast<const u16*>(h);
  float* a = at<float>(ws, L.a);
  u16* sb = at<u16>(ws, L.s);
  float* z = at<float>(ws, L.z);
  u16* g = at<u16>(ws, L.g);
  float* ltk = loss_tk ? loss_tk : at<float>(ws, L.ltk);
  if (dw1) MV_HIP(mvk::launch_transpose_bf16(H, 0, at<u16>(ws, L.ht), 0, N, d, 1, s));
  for (int k = 0; k < K; ++k) {
    const u16* W1 = static_cast<const u16*>(w1) + (size_t)k * d * d;
    const u16* W2 = static_cast<const u16*>(w2) + (size_t)k * V * d;
    // forward: a = H W1^T, s = SiLU(a) + H, z = s W2^T, loss and dL/dz
    MV_HIP(mvk::launch_gemm_nt_splitk(H, d, W1, d, a, N, d, d, z, (size_t)N * V, s));
    MV_HIP(mvk::launch_medusa1_act(a, H, sb, (size_t)N * d, s));
    MV_HIP(mvk::launch_gemm_nt(sb, d, 0, W2, d, 0, z, V, 0, N, V, d, 1, s));
    MV_HIP(mvk::launch_medusa1_ce(z, labels, K, k, (float)lam[k], N, V, ltk, g, s));
    if (dw2) {   // dW2 = g^T s: (g^T [V][N]) (s^T [d][N])^T
      MV_HIP(mvk::launch_transpose_bf16(g, 0, at<u16>(ws, L.gt), 0, N, V, 1, s));
      MV_HIP(mvk::launch_transpose_bf16(sb, 0, at<u16>(ws, L.st), 0, N, d, 1, s));
      MV_HIP(mvk::launch_gemm_nt(at<u16>(ws, L.gt), N, 0, at<u16>(ws, L.st), N, 0,
                                 dw2 + (size_t)k * V * d, d, 0, V, d, N, 1, s));
    }
    if (dw1) {   // ds = g W2 = g (W2^T [d][V])^T; da = ds SiLU'(a); dW1 = (da^T) (H^T)^T
      MV_HIP(mvk::launch_transpose_bf16(W2, 0, at<u16>(ws, L.w2t), 0, V, d, 1, s));
      MV_HIP(mvk::launch_gemm_nt_splitk(g, V, at<u16>(ws, L.w2t), V, at<float>(ws, L.ds), N, d, V,
                                        z, (size_t)N * V, s));     // z is free after the loss
      MV_HIP(mvk::launch_medusa1_dact(at<float>(ws, L.ds), a, at<u16>(ws, L.da), (size_t)N * d, s));
      MV_HIP(mvk::launch_transpose_bf16(at<u16>(ws, L.da), 0, at<u16>(ws, L.dat), 0, N, d, 1, s));
      MV_HIP(mvk::launch_gemm_nt(at<u16>(ws, L.dat), N, 0, at<u16>(ws, L.ht), N, 0,
                                 dw1 + (size_t)k * d * d, d, 0, d, d, N, 1, s));
    }
  }
  MV_HIP(mvk::launch_medusa1_sum(ltk, N * K, loss, s));
  return MV_OK;
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
  int P = 0;                     // prefill chunk rows (>= T)
  int64_t draws_used = 1;        // draws of u_draws consumed (draw 0: the prefill's root)
  // host-side upper bound on the device prefix lengths: the largest n after
  // mv_prefill / mv_ctx_resume plus depth + 1 per step enqueued since
  bool have_state = false;
  int64_t n_hi = 0;
};

// A step that draws (sampled roots, rejection sampling) takes the next row of
// u_draws: refuse to run past the last one.  The row counts as used once the
// step is enqueued (note_draw).
static bool draws_rows(const mv_ctx* c) {
  const mv_accept_params& p = c->d.accept;
  return p.root_mode == MV_ROOT_SAMPLE || p.mode == MV_ACCEPT_REJECT;
}
static int check_draw(const mv_ctx* c) {
  if (draws_rows(c) && c->draws_used >= c->d.n_draws)
    return fail(MV_ECAPACITY, "all %d rows of u_draws are used (prefill again or pass more)",
                c->d.n_draws);
  return MV_OK;
}
static int note_draw(mv_ctx* c, int rc) {
  if (rc == MV_OK && draws_rows(c)) ++c->draws_used;
  return rc;
}

// A step writes the tree's K/V at slots n .. n+T-1 of every sequence: refuse
// it while the host-side bound on n leaves fewer than T free slots.
static int check_capacity(const mv_ctx* c) {
  if (!c->have_state)
    return fail(MV_EINVAL, "no decode state: call mv_prefill or mv_ctx_resume first");
  if (c->n_hi + c->d.T > c->d.kv.cap)
    return fail(MV_ECAPACITY, "KV capacity: prefix length may reach %lld, + T=%d > cap=%d",
                (long long)c->n_hi, c->d.T, c->d.kv.cap);
  return MV_OK;
}
// A step moves n on by at most depth + 1 (the root and its accepted path).
static int note_step(mv_ctx* c, int rc) {
  if (rc == MV_OK) c->n_hi += c->d.tree.depth + 1;
  return note_draw(c, rc);
}

// All L layers; the last one leaves the final norm's operand in ws.xa / ws.ss.
static int enq_layers(mv_ctx* c, const mv_tree& tree, float* x, hipStream_t s,
                      int only_kind = -1) {
  const mv_step_desc& d = c->d;
  const mv_dims& D = d.dims;
  const int M = d.B * tree.T;
  int rc;
  for (int l = 0; l < D.L; ++l) {
    const void* next_gain = l + 1 < D.L ? c->layers[l + 1].attn_norm : d.final_norm;
    const int ss_in = l == 0 ? 1 : ss_tiles_of(D, G_DOWN, M);
    if ((rc = enq_layer(D, d.B, tree, d.n_prefix, c->layers[l], d.kv, l, x, ss_in, next_gain,
                        d.ws, c->L, s, only_kind)))
      return rc;
  }
  return MV_OK;
}

static int enq_step(mv_ctx* c, hipStream_t s) {
  const mv_step_desc& d = c->d;
  const mv_dims& D = d.dims;
  const int B = d.B, T = d.T, M = B * T;
  void* ws = d.ws;
  const Ws& L = c->L;
  int rc;
  const int Dn = d.tree.depth;
  int32_t* top_ids = d.top_ids ? d.top_ids : at<int32_t>(ws, L.topi);
  prof_begin(s);
  if (Dn > 0) {
    // the tree's tokens are filled in by the embedding launch below
    rc = enq_heads(D, B, Dn, d.s, d.h_last, d.w1, d.w2, nullptr, d.root_tok, top_ids,
                   at<float>(ws, L.topv), nullptr,
                   d.head_logits ? d.head_logits : at<float>(ws, L.hz), ws, L, s);
    if (rc) return rc;
  }
  prof_end(MV_K_HEADS, s);
  float* x = at<float>(ws, L.x);
  prof_begin(s);
  // tree tokens, embedding rows, RoPE tables and the first norm's operand
  const mvk::EmbedTree et{top_ids, d.root_tok, d.tree.rank, Dn > 0 ? Dn : 1, d.s, d.tree_tok};
  const mvk::EmbedNorm en{static_cast<const u16*>(c->layers[0].attn_norm), at<u16>(ws, L.xa),
                          at<float>(ws, L.ss), L.ss_ld};
  MV_HIP(mvk::launch_embed(nullptr, static_cast<const u16*>(d.embed), x, nullptr, M, D.d, D.V,
                           d.n_prefix, d.tree.depth_of, at<float2>(ws, L.rope), T, D.hd, s, et, en));
  prof_end(MV_K_EMBED, s);
  if ((rc = enq_layers(c, d.tree, x, s))) return rc;
  prof_begin(s);
  const bool greedy = d.accept.mode == MV_ACCEPT_GREEDY;
  unsigned long long* amaxp = greedy ? at<unsigned long long>(ws, L.amaxp) : nullptr;
  if ((rc = enq_lm_head(D, M, x, d.final_norm, d.lm_head, d.logits, ss_tiles_of(D, G_DOWN, M),
                        ws, L, s, amaxp, d.status)))
    return rc;
  prof_end(MV_K_LM_HEAD, s);
  prof_begin(s);
  const int u_stride = d.accept.mode == MV_ACCEPT_REJECT ? B * T : B;
  if ((rc = enq_accept(B, T, D.V, D.d, d.logits, d.tree, d.tree_tok, d.accept, d.u_draws,
                       d.u_index, u_stride, d.accept_len, d.path, d.best, d.root_tok, d.emitted, nullptr,
                       x, d.final_norm, d.h_last, at<int32_t>(ws, L.amax), at<double>(ws, L.stats),
                       at<double>(ws, L.bsum), s, amaxp, d.n_prefix,
                       mvk::StepGuard{d.status, d.kv.cap, T})))
    return rc;
  prof_end(MV_K_ACCEPT, s);
  prof_begin(s);
  // n_prefix was moved on by the acceptance kernel; the compaction bumps the
  // draw counter
  MV_HIP(mvk::launch_compact(static_cast<u16*>(d.kv.k), static_cast<u16*>(d.kv.v), D.L, B, D.H,
                             D.hd, d.kv.cap, d.path, d.tree.depth + 1, d.accept_len, d.n_prefix, s,
                             1, d.u_index));
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
  if (p.mode != MV_ACCEPT_GREEDY && p.mode != MV_ACCEPT_TYPICAL && p.mode != MV_ACCEPT_REJECT)
    return fail(MV_EINVAL, "accept mode");
  if (p.root_mode != MV_ROOT_ARGMAX && p.root_mode != MV_ROOT_SAMPLE) return fail(MV_EINVAL, "root mode");
  const bool draws = p.root_mode == MV_ROOT_SAMPLE || p.mode == MV_ACCEPT_REJECT;
  if ((p.mode != MV_ACCEPT_GREEDY || p.root_mode == MV_ROOT_SAMPLE) && !(p.temperature > 0.0))
    return fail(MV_EINVAL, "temperature must be > 0");
  if (draws && (!d.u_draws || !d.u_index || d.n_draws < 1))
    return fail(MV_EINVAL, "sampled roots and rejection sampling need u_draws, u_index and n_draws");
  if ((size_t)d.B * d.dims.d * 4 > MV_HEADS_LDS_MAX) return fail(MV_EUNSUPPORTED, "B*d too large");
  if (d.prefill_rows != 0 && (d.prefill_rows < d.T || d.prefill_rows > MV_MAX_T))
    return fail(MV_EUNSUPPORTED, "prefill_rows=%d outside {0} or [T=%d, %d]", d.prefill_rows, d.T,
                MV_MAX_T);
  const int Pr = std::max(d.T, (int)d.prefill_rows);
  if (d.kv.cap < Pr) return fail(MV_ECAPACITY, "kv cap %d < prefill rows %d", d.kv.cap, Pr);
  if ((rc = check_ws(&d.dims, d.B, d.T, d.ws_bytes, d.ws, Pr))) return rc;

  mv_ctx* c = new mv_ctx();
  c->d = d;
  c->layers.assign(d.layers, d.layers + d.dims.L);
  c->d.layers = nullptr;
  c->L = ws_layout(d.dims, d.B, d.T, Pr);
  c->P = Pr;
  // the prefill chain tree: P rows per sequence
  const int B = d.B, T = Pr, mw = (Pr + 63) / 64;
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
  // the GEMMs' arrival counters and the LM head's argmax keys must start at
  // zero (their consumers reset them)
  if (e == hipSuccess) e = hipMemset(at<char>(d.ws, c->L.counters), 0, c->L.hu - c->L.counters);
  if (e == hipSuccess) e = hipMemset(at<char>(d.ws, c->L.amaxp), 0, c->L.stats - c->L.amaxp);
  if (e == hipSuccess) e = hipDeviceSynchronize();
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
  // chunks of P rows (P = T unless a larger prefill chunk was asked for)
  const int B = d.B, T = c->P, M = B * T;
  const bool reject = d.accept.mode == MV_ACCEPT_REJECT;   // draws [n][B][T]: root from [0][b][0]
  int nmax = 0;
  for (int b = 0; b < B; ++b) {
    if (n_ids[b] < 1 || n_ids[b] > d.kv.cap - T || n_ids[b] > ld)
      return fail(MV_ECAPACITY, "prefix length %d of sequence %d outside [1, min(cap-P=%d, ld=%d)]",
                  n_ids[b], b, d.kv.cap - T, ld);
    nmax = std::max(nmax, (int)n_ids[b]);
  }
  const hipStream_t s = (hipStream_t)stream;
  void* ws = d.ws;
  const Ws& L = c->L;
  mv_tree chain{T, T - 1, (T + 63) / 64, c->chain, c->chain + (size_t)B * T,
                c->chain + (size_t)2 * B * T, c->chain_anc};
  float* logits = T > d.T ? at<float>(ws, L.plog) : d.logits;   // larger chunks: logits in ws
  c->have_state = false;          // until the whole prefill is enqueued
  MV_HIP(mvk::launch_fill_i32(d.n_prefix, 0, B, s));
  float* x = at<float>(ws, L.x);
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
    MV_HIP(mvk::launch_embed(c->chunk_tok, static_cast<const u16*>(d.embed), x,
                             nullptr, M, D.d, D.V, d.n_prefix, chain.depth_of,
                             at<float2>(ws, L.rope), T, D.hd, s));
    if ((rc = enq_norm_prep(D, M, x, c->layers[0].attn_norm, ws, L, s))) return rc;
    if ((rc = enq_layers(c, chain, x, s))) return rc;
    if ((rc = enq_lm_head(D, M, x, d.final_norm, d.lm_head, logits, ss_tiles_of(D, G_DOWN, M),
                          ws, L, s)))
      return rc;
    MV_HIP(mvk::launch_row_stats(logits, M, D.V, MV_ACCEPT_GREEDY, 1.0, at<int32_t>(ws, L.amax),
                                 at<double>(ws, L.stats), s));
    MV_HIP(mvk::launch_prefill_select(logits, at<int32_t>(ws, L.amax), cnt, B, T, D.V,
                                      reject ? MV_ROOT_SAMPLE : d.accept.root_mode,
                                      d.accept.temperature, d.u_draws, reject ? d.T : 1, d.root_tok, d.n_prefix, x,
                                      static_cast<const u16*>(d.final_norm),
                                      static_cast<u16*>(d.h_last), D.d, s));
    // the host-side counts buffer is reused next chunk: wait for the copy
    MV_HIP(hipStreamSynchronize(s));
  }
  if (d.u_index) MV_HIP(mvk::launch_fill_i32(d.u_index, 1, 1, s));
  c->draws_used = 1;
  c->have_state = true;
  c->n_hi = nmax;
  return MV_OK;
}

MV_API int mv_ctx_resume(mv_ctx* c, const int32_t* n_host, int32_t draws_used) {
  if (!c || !n_host) return fail(MV_EINVAL, "mv_ctx_resume: NULL pointer");
  const mv_step_desc& d = c->d;
  if (draws_used < 0 || (draws_rows(c) ? draws_used > d.n_draws : draws_used > 1))
    return fail(MV_EINVAL, "mv_ctx_resume: draws_used %d outside [0, %d]", draws_used,
                draws_rows(c) ? d.n_draws : 1);
  int64_t nmax = 0;
  for (int b = 0; b < d.B; ++b) {
    if (n_host[b] < 0 || n_host[b] > d.kv.cap - d.T)
      return fail(MV_ECAPACITY, "mv_ctx_resume: n[%d] = %d outside [0, cap - T = %d]", b,
                  n_host[b], d.kv.cap - d.T);
    nmax = std::max<int64_t>(nmax, n_host[b]);
  }
  c->draws_used = draws_used;
  c->have_state = true;
  c->n_hi = nmax;
  return MV_OK;
}

MV_API int mv_step(mv_ctx* c, int32_t use_graph, void* stream) {
  if (!c) return fail(MV_EINVAL, "mv_step: NULL context");
  const hipStream_t s = (hipStream_t)stream;
  if (int rc = check_capacity(c)) return rc;
  if (int rc = check_draw(c)) return rc;
  if (!use_graph) return note_step(c, enq_step(c, s));
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
  return note_step(c, MV_OK);
}

MV_API const float* mv_ctx_residual(const mv_ctx* c) {
  return c ? at<const float>(c->d.ws, c->L.x) : nullptr;
}

MV_API int mv_step_profile(mv_ctx* c, float* ms, int32_t* count, void* stream) {
  if (!c || !ms || !count) return fail(MV_EINVAL, "mv_step_profile: NULL pointer");
  const hipStream_t s = (hipStream_t)stream;
  if (int rc = check_capacity(c)) return rc;
  if (int rc = check_draw(c)) return rc;
  if (c->prof_ev.empty()) {
    c->prof_ev.resize(2 * 1024);
    for (auto& e : c->prof_ev) MV_HIP(hipEventCreate(&e));
  }
  Prof p;
  p.ev = c->prof_ev.data();
  p.cap = 1024;
  p.n = 0;
  g_prof = &p;
  const int rc = note_step(c, enq_step(c, s));
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

MV_API int mv_read_probe(const void* buf, size_t bytes, int32_t reps, float* sink, float* us,
                         void* stream) {
  if (!buf || !sink || !us) return fail(MV_EINVAL, "mv_read_probe: NULL pointer");
  if (reps < 1 || bytes < ((size_t)16 << 20))
    return fail(MV_EINVAL, "mv_read_probe: reps %d < 1 or bytes %zu < 16 MiB", reps, bytes);
  const hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  MV_HIP(hipEventCreate(&e0));
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(MV_EHIP, "mv_read_probe: event create");
  }
  hipError_t e = mvk::launch_read_probe(buf, bytes, sink, s);   // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = mvk::launch_read_probe(buf, bytes, sink, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return fail(MV_EHIP, "mv_read_probe: %s", hipGetErrorString(e));
  *us = 1000.f * ms / (float)reps;
  return MV_OK;
}

MV_API int mv_time_kernel(mv_ctx* c, int32_t kind, int32_t reps, float* us, void* stream) {
  if (!c || !us) return fail(MV_EINVAL, "mv_time_kernel: NULL pointer");
  if (reps < 1) return fail(MV_EINVAL, "mv_time_kernel: reps %d < 1", reps);
  if (kind != MV_K_QKV && kind != MV_K_ATTN && kind != MV_K_O && kind != MV_K_GATE_UP &&
      kind != MV_K_DOWN && kind != MV_K_LM_HEAD)
    return fail(MV_EINVAL, "mv_time_kernel: kind %d is not a per-layer GEMM, attention or LM head",
                kind);
  if (int rc = check_capacity(c)) return rc;   // the kernels write the tree's K/V slots
  const hipStream_t s = (hipStream_t)stream;
  const mv_step_desc& d = c->d;
  const mv_dims& D = d.dims;
  const int M = d.B * d.T;
  float* x = at<float>(d.ws, c->L.x);
  hipEvent_t e0, e1;
  MV_HIP(hipEventCreate(&e0));
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(MV_EHIP, "mv_time_kernel: event create");
  }
  int rc = MV_OK, launches = 0;
  hipError_t e = hipEventRecord(e0, s);
  for (int r = 0; r < reps && rc == MV_OK && e == hipSuccess; ++r) {
    if (kind == MV_K_LM_HEAD) {
      rc = enq_lm_head(D, M, x, d.final_norm, d.lm_head, d.logits, ss_tiles_of(D, G_DOWN, M),
                       d.ws, c->L, s);
      launches += 1;
    } else {
      rc = enq_layers(c, d.tree, x, s, kind);
      launches += D.L;
    }
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc) return rc;
  if (e != hipSuccess) return fail(MV_EHIP, "mv_time_kernel: %s", hipGetErrorString(e));
  *us = 1000.f * ms / (float)launches;
  return MV_OK;
}

}  // extern "C"
