/*
 * medusa_verify.h -- C ABI of the gfx950 (MI355X) Medusa tree-verify step.
 *
 * One Medusa decoding step (Medusa paper digest, "Algorithm: Medusa decoding
 * step", steps 1-6; Method items 1-5):
 *   1. root token t0 from the LM-head logits at the last accepted position;
 *      each Medusa head k takes its top-s_k tokens           -> mv_medusa_heads
 *   2. the tree's nodes get their tokens (root: t0)           -> mv_medusa_heads
 *   3. all tree nodes go through one backbone forward with the
 *      ancestor-only mask, position id = prefix length + depth -> mv_embed,
 *                                   mv_decoder_layer x L (uses mv_tree_attention),
 *                                   mv_lm_head
 *   4-5. greedy or typical acceptance, longest accepted prefix -> mv_accept
 *   6. the accepted path's KV moved into contiguous slots       -> mv_kv_compact
 * mv_step runs the whole step from device-resident state (one hipGraph).
 *
 * Conventions (all entry points):
 *  - Every pointer argument marked "device" is device memory owned by the
 *    caller; the library never allocates or frees caller memory and keeps no
 *    pointer beyond the call (except inside an mv_ctx, see mv_ctx_create).
 *  - bf16 tensors are raw 16-bit bf16 patterns; fp32 is IEEE float.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it and never synchronise; device faults
 *    surface at the caller's next synchronisation.
 *  - Every call validates its scalar arguments (and, where stated, host-side
 *    tree arrays) before enqueuing anything.  On failure it returns a
 *    negative mv_status, enqueues nothing and leaves every output untouched;
 *    mv_last_error() then describes the failure (thread-local string).
 *  - Device pointers must be 16-byte aligned.
 *
 * Data layouts:
 *  - Rows of the verify pass: m = b * T + v for sequence b and tree node v.
 *  - Fragment-packed bf16 weight [R][C] (R % 16 == 0, C % 32 == 0): blocks of
 *    16 rows x 32 columns in k-block-major order (all row blocks of column
 *    block 0 first), each block 64 pieces of 8 consecutive columns, piece
 *    l = row (l % 16), columns 8 * (l / 16) ..; element (r, c) sits at
 *      ((((c/32) * (R/16) + r/16) * 64 + (r%16) + 16*((c%32)/8)) * 8 + c%8.
 *    Weights of the backbone GEMMs are passed packed (see mv_pack_weight).
 *  - Workspace: caller-owned device memory of mv_workspace_size() bytes,
 *    zero-filled before its first use; the library keeps its internal
 *    arrival counters at zero between calls.  Calls sharing a workspace must
 *    be ordered on one stream.
 *  - KV cache (one buffer for K, one for V, all layers): one block of
 *    cap*hd bf16 elements per (l, b, h), at ((l*B + b)*H + h)*cap*hd.
 *    Inside a block, with o = slot % 32:
 *      K: [cap/32][hd/8][32][8]: element (slot, i) at
 *         (((slot/32)*(hd/8) + i/8)*32 + row(o))*8 + i%8,
 *         row(o) = 16*((o/4)%2) + 4*(o/8) + o%4   (whole-line attention loads)
 *      V: [cap/8][hd][8]: element (slot, i) at ((slot/8)*hd + i)*8 + slot%8
 *    cap % 64 == 0, hd % 8 == 0.  Slots >= n + T may hold anything.
 *  - Tree (per sequence, T nodes, root = node 0, parents before children):
 *    parent[T] (root: -1), depth_of[T] (root: 0), rank[T] (rank of the node's
 *    token within its head's top-s list; root: 0), and the ancestor bitmask
 *    anc[T][mask_words] (bit a of node v's words set iff a == v or a is an
 *    ancestor of v).  Node v's K/V sit at slot n + v, its position id is
 *    n + depth_of[v] (Medusa paper digest, Method 3 and Pitfalls).
 */
#ifndef MEDUSA_VERIFY_H
#define MEDUSA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MV_API __attribute__((visibility("default")))

typedef enum {
  MV_OK = 0,
  MV_EINVAL = -1,        /* bad scalar argument or null required pointer */
  MV_EUNSUPPORTED = -2,  /* shape outside what the kernels implement */
  MV_ECAPACITY = -3,     /* n + T would exceed the cache capacity, or u_draws ran out */
  MV_EWORKSPACE = -4,    /* workspace smaller than mv_workspace_size() */
  MV_EHIP = -5,          /* a HIP runtime call failed (detail in mv_last_error) */
  MV_ETREE = -6          /* invalid tree (not prefix-closed, too deep, ...) */
} mv_status;

#define MV_MAX_T 256        /* tree nodes per sequence, root included */
#define MV_MAX_DEPTH 16     /* tree depth (<= number of Medusa heads used) */
#define MV_MAX_TOPK 16      /* candidates per head */
#define MV_MAX_BATCH 4      /* sequences per call (Medusa head GEMV) */
#define MV_MAX_VOCAB 262144 /* vocabulary (inverse-CDF draws scan 1024 blocks of 256 ids) */
#define MV_HEADS_LDS_MAX (128 * 1024)  /* head GEMV: B * d * 4 bytes of input rows in LDS */

#define MV_ACCEPT_GREEDY 0
#define MV_ACCEPT_TYPICAL 1
#define MV_ACCEPT_REJECT 2
#define MV_ROOT_ARGMAX 0
#define MV_ROOT_SAMPLE 1

#define MV_PACK_PLAIN 0
#define MV_PACK_QKV 1

/* Bits of the step's device status word (mv_step_desc.status), OR-ed in by
 * the step's kernels and never cleared by the library. */
#define MV_STATUS_NONFINITE 1  /* the LM head wrote a non-finite logit for a tree row */
#define MV_STATUS_CAPACITY 2   /* a step ran with n + T > cap on the device: its K/V
                                * writes were clamped into the cache and its outputs
                                * are not valid (only reachable when the host-side
                                * bound given to mv_ctx_resume was wrong) */

/* Backbone and head shapes.  Multi-head attention: H * hd == d.
 * Supported: d % 64 == 0, F % 32 == 0, V % 64 == 0, V <= MV_MAX_VOCAB,
 * hd in {16,32,64,128},
 * 1 <= K <= MV_MAX_DEPTH. */
typedef struct {
  int32_t L, d, H, hd, F, V, K;
} mv_dims;

/* Device-side trees of a batch: every sequence has T nodes; arrays are
 * [B][T] (anc: [B][T][mask_words]); depth = max depth over the batch;
 * mask_words = ceil(T / 64). */
typedef struct {
  int32_t T, depth, mask_words;
  const int32_t* parent;
  const int32_t* depth_of;
  const int32_t* rank;
  const uint64_t* anc;
} mv_tree;

/* The whole KV cache (layouts above). */
typedef struct {
  void* k;
  void* v;
  int32_t L, B, H, hd, cap;
} mv_kv;

/* One decoder layer's weights (device): RMSNorm gains bf16 [d]; the
 * projections fragment-packed bf16: wqkv [3d][d] packed with MV_PACK_QKV
 * (rows: q then k then v, each (out, in)), wo [d][d], wgate [F][d],
 * wup [F][d], wdown [d][F] packed with MV_PACK_PLAIN. */
typedef struct {
  const void* attn_norm;
  const void* wqkv;
  const void* wo;
  const void* ffn_norm;
  const void* wgate;
  const void* wup;
  const void* wdown;
} mv_layer_weights;

/* Acceptance rule (Medusa paper digest, Method 5 and "Paper vs code"):
 * GREEDY: candidate accepted iff it equals the argmax of its parent's row;
 * TYPICAL: iff q(x) > min(eps, delta * exp(-H(q))) with q = softmax(z /
 * temperature) of the parent's row and H(q) = -sum q log(q + 1e-5).
 * root_mode ARGMAX: next root = argmax of the best node's row; SAMPLE: the
 * smallest id whose cumulative softmax(z / temperature) mass (id order)
 * exceeds the step's uniform draw.  temperature > 0 for TYPICAL / SAMPLE.
 * REJECT: rejection sampling (speculative sampling: lecture note section
 * 二.3; speculative-decoding tutorial, Maths) with the fixed top-s
 * candidates as point-mass drafts (see mv_accept_reject); the next root is
 * the walk's final draw and root_mode is not used; temperature > 0. */
typedef struct {
  int32_t mode;
  int32_t root_mode;
  double temperature;
  double eps;
  double delta;
} mv_accept_params;

/* ---- errors -------------------------------------------------------------- */
MV_API const char* mv_strerror(int status);          /* static string */
MV_API const char* mv_last_error(void);              /* thread-local detail */

/* ---- host helpers -------------------------------------------------------- */

/* Flatten a candidate tree given as its paths of 0-based head ranks (Medusa
 * paper digest, Method 2-4; the released sparse trees are such path lists).
 * paths: host int32 [n_paths][max_len] row-major, path p = paths[p][0 ..
 * path_len[p]-1] (ranks i_1..i_k: head j's i_j-th candidate).  The list must
 * be prefix-closed, duplicate-free, with 1 <= len < MV_MAX_T (trees deeper
 * than MV_MAX_DEPTH, e.g. chains, are accepted by mv_tree_attention and
 * mv_decoder_layer only) and
 * 0 <= rank < topk.  Node order: root, then by (depth, lexicographic path).
 * Outputs (host): parent, depth_of, rank [T], anc [T][mask_words], *T_out =
 * n_paths + 1; capacity `cap_nodes` >= n_paths + 1 and mask_words >=
 * ceil(T/64).  Errors: MV_ETREE (with the offending path in mv_last_error),
 * MV_EINVAL. */
MV_API int mv_tree_compile(const int32_t* paths, const int32_t* path_len, int32_t n_paths,
                           int32_t max_len, int32_t topk, int32_t cap_nodes,
                           int32_t mask_words, int32_t* parent, int32_t* depth_of,
                           int32_t* rank, uint64_t* anc, int32_t* T_out);

/* Calibrated sparse tree (Medusa paper digest, Method 4 "Optimized sparse
 * tree", paper section 2.3.3; Pitfalls: heads taken as independent).
 * acc: host double [K][s], acc[k][i] = measured accuracy of head k+1's
 * i-th top prediction alone (see mv_head_accuracy), each in [0, 1].  A
 * node with rank path (i_1..i_k) is estimated as acc[0][i_1] * ... *
 * acc[k-1][i_k] (formed left to right); the tree grows from the root by
 * repeatedly taking the connected node with the highest estimate (ties:
 * the lexicographically smaller path) until n_nodes candidates or no node
 * of depth <= min(max_depth, K) is left.  Outputs (host): paths
 * [n_nodes][max_depth] (ranks, -1 padded) and path_len [n_nodes] in the
 * flattened tree order (depth, then path; ready for mv_tree_compile),
 * *n_out = nodes built, *expected_len (nullable) = the sum of their
 * estimates (expected accepted candidates per step).  n_nodes <= MV_MAX_T-1,
 * 1 <= max_depth <= MV_MAX_DEPTH, K <= MV_MAX_DEPTH, s <= MV_MAX_TOPK.
 * Errors: MV_EINVAL. */
MV_API int mv_tree_build_sparse(const double* acc, int32_t K, int32_t s, int32_t n_nodes,
                                int32_t max_depth, int32_t* paths, int32_t* path_len,
                                int32_t* n_out, double* expected_len);

/* Calibration of the heads (Medusa paper digest, Method 4): for N
 * calibration positions with the heads' ranked candidates top_ids (device
 * int32 [N][K][s], e.g. mv_medusa_heads' top_ids) and the true tokens
 * labels (device int32 [N][K], the token k+1 positions ahead for head
 * k+1), add to counts (device int32 [K][s], caller-zeroed, accumulated
 * across calls) the number of positions whose label equals head k+1's i-th
 * candidate.  acc[k][i] = counts[k][i] / N.  N * K <= 2^30. */
MV_API int mv_head_accuracy(int32_t N, int32_t K, int32_t s, const int32_t* top_ids,
                            const int32_t* labels, int32_t* counts, void* stream);

/* Expected acceptance length of a given tree under acc (as above): the sum
 * over its n_paths nodes (host paths [n_paths][ld], path_len [n_paths]) of
 * the products of accuracies along their rank paths.  Errors: MV_EINVAL,
 * MV_ETREE (a rank >= s or a path longer than K). */
MV_API int mv_tree_expected_length(const double* acc, int32_t K, int32_t s, const int32_t* paths,
                                   const int32_t* path_len, int32_t n_paths, int32_t ld,
                                   double* out);

/* Reorder a row-major bf16 weight [rows][cols] (out, in) into the
 * fragment-packed layout the backbone GEMMs read.  layout MV_PACK_QKV: the
 * matrix is the fused [3d][d] q|k|v projection with head size hd; q and k
 * rows are additionally permuted (head size >= 32) in groups of 32 rows: 16
 * first-half dims of a head, then their RoPE partners (dims + hd/2).  src and dst are device buffers of
 * rows*cols bf16 and must not overlap.  rows % 16 == 0, cols % 32 == 0. */
MV_API int mv_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols,
                          int32_t layout, int32_t hd, void* stream);

/* Bytes of device workspace needed by the calls below for this shape
 * (the largest of the per-call needs; one workspace serves them all). */
MV_API int mv_workspace_size(const mv_dims* dims, int32_t B, int32_t T, int32_t cap,
                             size_t* bytes);

/* Workspace bytes of a step context whose prefill runs in chunks of
 * prefill_rows rows (0, or T <= prefill_rows <= MV_MAX_T). */
MV_API int mv_workspace_size_prefill(const mv_dims* dims, int32_t B, int32_t T,
                                     int32_t prefill_rows, size_t* bytes);

/* ---- the step's operations ----------------------------------------------- */

/* Medusa heads (Medusa paper digest, Method 1-2, Algorithm steps 1-2):
 *   u_k = h + SiLU(W1_k h),  z_k = W2_k u_k,  k = 1..D (D <= dims.K),
 *   top_ids[b][k-1][0..s) = the s largest z_k (larger value first, lower id
 *   first on ties), top_vals the matching logits;
 *   tree_tok[b][v] = root_tok[b] for the root, top_ids[b][depth(v)-1][rank(v)]
 *   otherwise (skipped when tree == NULL).
 * h: device bf16 [B][d] (final-normed hidden state at the last accepted
 * position); w1: device bf16 [K][d][d], w2: device bf16 [K][V][d], both
 * row-major (out, in); head_logits: device fp32 [B][D][V] or NULL (then the
 * workspace holds them).  B <= MV_MAX_BATCH, s <= MV_MAX_TOPK, s <= V. */
MV_API int mv_medusa_heads(const mv_dims* dims, int32_t B, int32_t D, int32_t s, const void* h,
                           const void* w1, const void* w2, const mv_tree* tree,
                           const int32_t* root_tok, int32_t* top_ids, float* top_vals,
                           int32_t* tree_tok, float* head_logits, void* ws, size_t ws_bytes,
                           void* stream);

/* Tree attention of one layer (Medusa paper digest, Method 3; wq-win lecture
 * note, 二.2): for every node v of sequence b and head h,
 *   out[b][v][h] = sum_s softmax_s(q . K_s / sqrt(hd)) V_s
 * over the slots s in [0, n[b]) and s = n[b] + a for each ancestor a of v
 * (v included).  q: device bf16 [B][T][H][hd], RoPE already applied at
 * position n + depth; the tree's K/V must already sit at slots n .. n+T-1 of
 * layer `layer`; n_prefix: device int32 [B]; out: device bf16 [B][T][H][hd].
 * Requires n[b] + T <= cap (not checked on the device: the caller owns n). */
MV_API int mv_tree_attention(const mv_dims* dims, int32_t B, const mv_tree* tree,
                             const int32_t* n_prefix, const void* q, const mv_kv* kv,
                             int32_t layer, void* out, void* ws, size_t ws_bytes, void* stream);

/* One pre-norm Llama decoder layer over all B*T tree rows (the verify
 * forward of Algorithm step 3):
 *   r = RMSNorm(x) (eps 1e-5);  q,k,v = r Wq^T, r Wk^T, r Wv^T;
 *   RoPE (base 10000, pairs (i, i + hd/2)) at position n[b] + depth(v);
 *   K/V rows -> cache slots n[b] + v;  o = tree attention;
 *   x += o Wo^T;  r' = RMSNorm(x);  x += (SiLU(r' Wg^T) * (r' Wu^T)) Wd^T.
 * x: device fp32 [B*T][d], the residual stream, updated in place. */
MV_API int mv_decoder_layer(const mv_dims* dims, int32_t B, const mv_tree* tree,
                            const int32_t* n_prefix, const mv_layer_weights* w, const mv_kv* kv,
                            int32_t layer, float* x, void* ws, size_t ws_bytes, void* stream);

/* x[m] = embed[tokens[m]] widened to fp32.  tokens: device int32 [M] (values
 * clamped to [0, V)); embed: device bf16 [V][d] row-major; x: fp32 [M][d]. */
MV_API int mv_embed(const mv_dims* dims, int32_t M, const int32_t* tokens, const void* embed,
                    float* x, void* stream);

/* Final RMSNorm and LM head ("head 0"): hn = RMSNorm(x) * final_norm (bf16),
 * logits = hn W_lm^T in fp32.  x: device fp32 [M][d]; lm_head:
 * fragment-packed bf16 [V][d]; logits: device fp32 [M][V]. */
MV_API int mv_lm_head(const mv_dims* dims, int32_t M, const float* x, const void* final_norm,
                      const void* lm_head, float* logits, void* ws, size_t ws_bytes,
                      void* stream);

/* Acceptance (Algorithm steps 4-5): decisions per edge, accepted prefix,
 * best node v* = deepest accepted node (TYPICAL: then larger summed
 * log-probability of the accepted candidates; then lower index).
 * logits: device fp32 [B][T][V]; tree_tok: device int32 [B][T];
 * u: device double [B] uniform draws in [0,1) (SAMPLE only, else NULL);
 * REJECT: device double [B][T], as mv_accept_reject takes them.
 * REJECT is mv_accept_reject with no draft logits (the margin holds its
 * values, its workspace is mv_accept_reject's); eps, delta and root_mode
 * are not read.  Workspace (256-aligned parts): argmax int32 [B*T], row
 * stats double [B*T][3] and, for TYPICAL, the rows' 256-id block sums
 * double [B*T][ceil(V/256)] (used by the sampled root's draw).
 * Outputs (device): accept_len [B] (= depth of v*), path [B][depth+1] (node
 * indices root..v*, then -1), best [B], next_root [B]; optional: emitted
 * [B][depth+1] (tokens of the path, then -1), margin double [B][T+1]
 * ((q - thr)/thr per edge for TYPICAL, [T]: |cdf - u| of the sampled root),
 * and, given the verify pass's fp32 residual rows x [B*T][d] and the final
 * RMSNorm gain (bf16 [d]), the carried hidden state h_last bf16 [B][d] =
 * RMSNorm(x[b*T + v*]) * final_norm (the input of the next step's heads). */
MV_API int mv_accept(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                     const mv_tree* tree, const int32_t* tree_tok, const mv_accept_params* p,
                     const double* u, int32_t* accept_len, int32_t* path, int32_t* best,
                     int32_t* next_root, int32_t* emitted, double* margin, const float* x,
                     const void* final_norm, void* h_last, void* ws, size_t ws_bytes,
                     void* stream);

/* mv_accept for callers that cannot allocate device memory (code under
 * hipGraph capture, tight serving loops, harnesses that forbid it): the same
 * operation, arguments and outputs as mv_accept, without the workspace.  Its
 * scratch (row argmax, row statistics and, for TYPICAL and REJECT, the rows'
 * 256-id block sums: align256(4*B*T) + align256(24*B*T) [+ 8*B*T*ceil(V/256)]
 * bytes) is a static device array of MV_NOALLOC_SCRATCH_BYTES in the library,
 * one per GPU, held until the process ends; its address is looked up once
 * per device on the first call with that device current.  The call
 * allocates nothing.  Every byte of scratch it reads it first writes in the
 * same call, so nothing needs clearing, but all calls on one GPU share the
 * array: calls that overlap on one GPU (e.g. on different streams) race.
 * Errors: as mv_accept, and MV_EWORKSPACE (before anything is enqueued)
 * when the shape needs more than MV_NOALLOC_SCRATCH_BYTES. */
#define MV_NOALLOC_SCRATCH_BYTES (8u << 20)
MV_API int mv_accept_noalloc(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                             const mv_tree* tree, const int32_t* tree_tok,
                             const mv_accept_params* p, const double* u, int32_t* accept_len,
                             int32_t* path, int32_t* best, int32_t* next_root, int32_t* emitted,
                             double* margin, const float* x, const void* final_norm,
                             void* h_last, void* stream);

/* Rejection-sampling acceptance (speculative sampling: lecture note section
 * 二.3, two-word example; speculative-decoding tutorial, Concept and Maths).
 * The pages give the chain rule: a draft x drawn from q is kept against the
 * target p with probability min(1, p(x)/q(x)); the first rejection is
 * replaced by a draw from max(0, p - q) normalised and ends the pass; when
 * all are kept a bonus token is drawn from the target.  Tree reading: at
 * the current node (p = softmax(logits[node] / temperature)) the children
 * are tried in node order against the running residual r (p at first); a
 * kept child becomes the current node, a rejection sets r to the
 * correction's residual and the next sibling is tried; with no child kept
 * (or at a leaf) the next root is the inverse-CDF draw (id order) from r.
 * A residual with no mass left falls back to the node's p.  Candidate
 * tokens outside [0, V) are never kept.
 * draft_logits NULL: candidates are fixed (top-s), their draft a point mass:
 *   x is kept with probability r(x) and a rejection removes x from r.
 * draft_logits device fp32 [B][tree->depth][V]: children at depth k use
 *   q = softmax(draft_logits[b][k-1] / temperature) (candidates drawn from
 *   the heads).
 * u: device double [B][T] uniform draws in [0,1): u[b][v] decides candidate
 * v (kept iff u < keep probability), u[b][0] makes the final draw.
 * Outputs as mv_accept: accept_len [B], path [B][depth+1], best [B] (the
 * last kept node), next_root [B]; optional emitted [B][depth+1], margin
 * double [B][T+1] (u - keep probability for tested candidates, +inf
 * elsewhere; [T]: the final draw's distance to its bracketing cumulative
 * sums) and h_last (given x, final_norm) as mv_accept.
 * Workspace (each part 256-aligned): row argmax int32 [B*T], row stats
 * double [B*T][3] and the rows' 256-id block sums double
 * [B*T][ceil(V/256)]; with draft logits also argmax int32 [B*depth], stats
 * double [B*depth][3] of the draft rows and residuals double [B][2][V]:
 * align256(4*B*T) + align256(24*B*T) + align256(8*B*T*ceil(V/256)), plus
 * align256(4*B*depth) + align256(24*B*depth) + 16*B*V with draft logits.
 * temperature > 0.
 * Work is one workgroup per sequence after a pass over the T rows. */
MV_API int mv_accept_reject(int32_t B, int32_t T, int32_t V, int32_t d, const float* logits,
                            const mv_tree* tree, const int32_t* tree_tok, double temperature,
                            const float* draft_logits, const double* u, int32_t* accept_len,
                            int32_t* path, int32_t* best, int32_t* next_root, int32_t* emitted,
                            double* margin, const float* x, const void* final_norm, void* h_last,
                            void* ws, size_t ws_bytes, void* stream);

/* KV compaction (Algorithm step 6; Medusa paper digest, Pitfalls): for every
 * layer, sequence b and m = 0..accept_len[b]: slot n[b] + m <- slot n[b] +
 * path[b][m] (K and V; all sources read before any destination is written),
 * then n[b] += 1 + accept_len[b].  path: device int32 [B][path_stride];
 * accept_len, n_prefix: device int32 [B] (n_prefix updated in place). */
MV_API int mv_kv_compact(const mv_kv* kv, const int32_t* path, int32_t path_stride,
                         const int32_t* accept_len, int32_t* n_prefix, void* stream);

/* ---- Medusa-1 head training (frozen backbone) ---------------------------- */

/* Bytes of device workspace for mv_medusa1_loss over N positions. */
MV_API int mv_medusa1_workspace_size(const mv_dims* dims, int32_t N, size_t* bytes);

/* Medusa-1 head loss and its gradients (Medusa paper digest, Method 6,
 * eq. 1 with lambda_k = 0.8^k of app. B.2; wq-win lecture note, 二.1):
 *   L = sum_t sum_{k=1..K} -lambda_k log p_t^(k)(y_{t+k+1}),
 *   p_t^(k) = softmax(W2_k (SiLU(W1_k h_t) + h_t)),
 * with the backbone frozen: dL/dW1_k and dL/dW2_k.
 * h: device bf16 [N][d] (the hidden states the LM head reads, i.e. after
 * the final RMSNorm); labels: device int32 [N][K], labels[t][k-1] = the
 * token k+1 positions after t (a shift of 2 + i for 0-indexed head i, as
 * the released trainer does), -1 (or any id outside [0, V)) = no label;
 * lambda: host double [K] (NULL: 0.8^k; ones give the released trainer's
 * unweighted sum); w1: device bf16 [K'][d][d], w2: device bf16 [K'][V][d]
 * row-major (out, in), the first K of K' = dims.K heads are used.
 * Outputs (device): loss double [1] (the sum over positions and heads, in a
 * fixed order); optional: loss_tk fp32 [N][K] (each term, lambda applied),
 * dw1 fp32 [K][d][d] and dw2 fp32 [K][V][d] (NULL: not computed).
 * Requires N % 64 == 0 (64 <= N <= 2^20); workspace of
 * mv_medusa1_workspace_size bytes.  The contractions (a = h W1^T, z = s
 * W2^T, dW2 = g^T s, ds = g W2, dW1 = da^T h) run on bf16 MFMA with fp32
 * accumulation; s, the logits' gradient g and da are rounded to bf16 as
 * GEMM operands. */
MV_API int mv_medusa1_loss(const mv_dims* dims, int32_t N, int32_t K, const void* h,
                           const int32_t* labels, const double* lambda, const void* w1,
                           const void* w2, double* loss, float* loss_tk, float* dw1, float* dw2,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- whole step ---------------------------------------------------------- */

/* Everything one decode step reads and writes (all device, caller-owned).
 * State carried between steps: n_prefix [B], root_tok [B], h_last bf16
 * [B][d], the KV cache, and (SAMPLE roots, REJECT acceptance) the draw
 * counter u_index (int32, device) into u_draws: double [n_draws][B] for
 * SAMPLE roots, [n_draws][B][T] for REJECT (draw i feeds step i's
 * candidates and final draw as mv_accept_reject's u; draw 0, entry
 * [0][b][0], samples the root after prefill). */
typedef struct {
  mv_dims dims;
  int32_t B, T, s;                 /* s: candidates per head (topk) */
  const mv_layer_weights* layers;  /* host array [L] of device pointers */
  const void* embed;               /* bf16 [V][d] */
  const void* final_norm;          /* bf16 [d] */
  const void* lm_head;             /* packed bf16 [V][d] */
  const void* w1;                  /* bf16 [K][d][d] */
  const void* w2;                  /* bf16 [K][V][d] */
  mv_kv kv;
  mv_tree tree;
  mv_accept_params accept;
  int32_t* n_prefix;
  int32_t* root_tok;
  void* h_last;
  const double* u_draws;           /* SAMPLE roots or REJECT only */
  int32_t* u_index;                /* SAMPLE roots or REJECT only */
  int32_t n_draws;
  /* per-step outputs */
  int32_t* tree_tok;               /* [B][T] */
  float* logits;                   /* [B][T][V] */
  int32_t* accept_len;             /* [B] */
  int32_t* path;                   /* [B][depth+1] */
  int32_t* emitted;                /* [B][depth+1] */
  int32_t* best;                   /* [B] */
  /* optional per-step outputs (NULL: kept in the workspace) */
  float* head_logits;              /* [B][depth][V] Medusa head logits */
  int32_t* top_ids;                /* [B][depth][s] per-head candidates */
  void* ws;
  size_t ws_bytes;
  /* prefill chunk rows: 0 (chunks of T rows) or T..MV_MAX_T; a larger chunk
   * raises the GEMMs' rows per weight byte.  With prefill_rows > T the
   * workspace is mv_workspace_size_prefill's and the prefill's logits stay
   * in it (the logits buffer holds only the step's). */
  int32_t prefill_rows;
  /* optional (NULL: none): device int32 status word, MV_STATUS_* bits OR-ed
   * in by each step; the caller clears it. */
  int32_t* status;
} mv_step_desc;

typedef struct mv_ctx mv_ctx;

/* Validate the description and bind it.  The context keeps the pointers in
 * `desc` (and copies the host layer array); it owns only a captured hipGraph
 * and a few small device arrays for prefill chain trees. */
MV_API int mv_ctx_create(mv_ctx** out, const mv_step_desc* desc);
MV_API void mv_ctx_destroy(mv_ctx* ctx);

/* Prefill: run the prompts through the backbone in chunks of up to T tokens
 * (prefill_rows, when set)
 * as chain trees (parent = previous token, so the tree mask is the causal
 * mask), filling KV slots [0, n), then set h_last, root_tok (ARGMAX or SAMPLE
 * with draw 0 of u_draws; REJECT acceptance always samples) and
 * n_prefix = n.  ids: device int32 [B][ld];
 * n_ids: host int32 [B] (1 <= n <= cap - chunk rows); counter u_index is
 * set to 1. */
MV_API int mv_prefill(mv_ctx* ctx, const int32_t* ids, int32_t ld, const int32_t* n_ids,
                      void* stream);

/* Declare a decode state that the caller placed in the bound buffers
 * itself (KV cache, n_prefix, root_tok, h_last, u_index), instead of
 * mv_prefill, e.g. to resume from a saved state.  n_host: host int32 [B],
 * the values the caller wrote to n_prefix; they become the host-side bound
 * on n that mv_step checks.  draws_used: rows of u_draws already consumed
 * (the value in u_index; 1 after a prefill).  Errors: MV_EINVAL (NULL, or
 * draws_used outside [0, n_draws]), MV_ECAPACITY (some n < 0 or n + T >
 * cap); nothing is enqueued. */
MV_API int mv_ctx_resume(mv_ctx* ctx, const int32_t* n_host, int32_t draws_used);

/* One tree-verify step from the device-resident state.  graph != 0: the
 * step is captured into a hipGraph on the first call and replayed after;
 * graph == 0: the kernels are enqueued directly.
 * Capacity: n lives on the device, so the context keeps a host-side upper
 * bound on it -- the largest prefix length after mv_prefill (or
 * mv_ctx_resume), plus depth + 1 (the most a step can accept) for every
 * step enqueued since.  While bound + T > cap the call fails with
 * MV_ECAPACITY and enqueues nothing (the bound is conservative: a step may
 * be refused although the actual n would still fit).  Before the first
 * mv_prefill or mv_ctx_resume the call fails with MV_EINVAL.
 * A step that draws (SAMPLE roots, REJECT acceptance) uses the next row of
 * u_draws; once the prefill's row and one row per step have used all
 * n_draws rows, the call fails with MV_ECAPACITY and enqueues nothing. */
MV_API int mv_step(mv_ctx* ctx, int32_t graph, void* stream);

/* Device address of the verify pass's fp32 residual rows [B*T][d] inside
 * the context's workspace: after a step (and until the next call that uses
 * the workspace) they hold the rows after the last decoder layer, the input
 * of the final RMSNorm and LM head.  For inspection only; NULL for a NULL
 * context. */
MV_API const float* mv_ctx_residual(const mv_ctx* ctx);

/* Launch-group kinds reported by mv_step_profile. */
#define MV_K_HEADS 0     /* Medusa heads: W1 block, vocab projection, top-s */
#define MV_K_EMBED 1     /* tree tokens, embedding gather, RoPE table, first norm's operand */
#define MV_K_NORM 2      /* standalone norm operand (in a step the embedding writes it) */
#define MV_K_QKV 3       /* fused QKV GEMM with RoPE and KV-cache write */
#define MV_K_ATTN 4      /* tree attention */
#define MV_K_O 5         /* output projection GEMM + residual */
#define MV_K_GATE_UP 6   /* gate/up GEMM with SwiGLU */
#define MV_K_DOWN 7      /* down projection GEMM + residual */
#define MV_K_LM_HEAD 8   /* LM-head GEMM (final norm folded in) */
#define MV_K_ACCEPT 9    /* acceptance, next root, n update */
#define MV_K_COUNT 11
#define MV_K_COMPACT 10  /* KV compaction (and the draw counter) */

/* One step enqueued directly (no graph) with a pair of HIP events on
 * `stream` around every launch group; waits for the step, then reports per
 * kind the summed milliseconds ms[MV_K_COUNT] and launch-group counts
 * count[MV_K_COUNT] (host arrays).  Same kernels and launch shapes as
 * mv_step. */
MV_API int mv_step_profile(mv_ctx* ctx, float* ms, int32_t* count, void* stream);

/* Average duration in microseconds (*us, host) of one launch of one kind --
 * MV_K_QKV, MV_K_ATTN, MV_K_O, MV_K_GATE_UP, MV_K_DOWN (all L layers) or
 * MV_K_LM_HEAD -- enqueued back to back `reps` times with the step's own
 * arguments between two HIP events on `stream`, then waited for.  It reruns
 * kernels of the step on the current state: it rewrites the residual stream
 * and the workspace and the tree's KV slots past n, all of which the next
 * step writes first, so the decode state is unchanged. */
MV_API int mv_time_kernel(mv_ctx* ctx, int32_t kind, int32_t reps, float* us, void* stream);

/* Measurement helper, not part of the method: the achievable streaming-read
 * bandwidth of the device, against which the step's HBM share can be read
 * beside the 8 TB/s peak.  Reads the device buffer buf (bytes >= 16 MiB;
 * 4096 workgroups each sum a contiguous slice with sixteen 16-byte loads in
 * flight per lane) reps times back to back and stores the average
 * microseconds per pass in *us (host).  sink: device float, written only in
 * the (never taken) case that a sum equals a sentinel.  Synchronises the
 * stream.  Errors: MV_EINVAL for NULL pointers, reps < 1 or small buffers;
 * MV_EHIP for launch or event failures. */
MV_API int mv_read_probe(const void* buf, size_t bytes, int32_t reps, float* sink, float* us,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_VERIFY_H */
