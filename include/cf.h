/*
 * cf.h — C ABI of libcf: blended prefill (CacheBlend-style selective KV recompute) on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method, in the pages' terms:
 *  - QCFuse: Query-Aware Cache Fusion via Compressed View for Efficient RAG Serving, §2.1:
 *    a request is context chunks c_1..c_m (N tokens) followed by a query U (Table 1, Eq. 1);
 *    each chunk has its own cache prefilled standalone at local positions 0.. (Eq. 3); at
 *    request time the caches are position-remapped and stitched in order (Eq. 4); a set P of
 *    context positions (ratio rho = |P|/N, Eq. 6) is recomputed under the current request and
 *    replaces the stitched entries (Eq. 7).
 *  - CacheBlend: Reusing KV Caches When Your Text Isn't a Prefix: RoPE keys move by composing
 *    rotations ("Why You Can't Just Concatenate"); P is the high-KV-deviation tokens
 *    ("Quantifying the Damage"); each layer recomputes only the selected rows, scatters their
 *    K/V into the blended cache, lets them attend over the full blended K/V and updates only
 *    their hidden rows ("Selective Recompute Without Skipping"); the selection is made once on
 *    an early layer ("The Chicken-and-Egg Problem").
 *  - Request Order Matters: Cache-History Sensitivity in Selective KV-Cache Reuse for Rolling
 *    Agents: deviation d_i = ||K_i^current - K_i^cached||_2^2 (§2.2 Eq. 1), budget
 *    k = max(1, floor(r N)) (Eq. 2), one selection at a configured layer, document-aligned
 *    spans (§2.3, Eq. 3).
 *
 * General rules for every entry point
 *  - Memory: every tensor argument is a device pointer owned by the caller unless the
 *    argument says "host". The library never frees, retains or reallocates caller memory.
 *    Scratch memory is a caller-provided device workspace whose size comes from the matching
 *    *_workspace_size query; the library allocates only the RoPE tables of a cf_ctx.
 *  - Layout: row-major. A K or V cache layer is [rows][n_kv_heads][head_dim]; layer l of a
 *    multi-layer cache starts at base + l * layer_stride elements. Weight matrices are
 *    [out_features][in_features] (y = x W^T). Element type is the model dtype (CF_F32 or CF_BF16)
 *    except where an argument says fp32.
 *  - Streams: work is enqueued on `stream` (NULL = the null stream); no call synchronises the
 *    host with the device, except that cf_blend_prefill_streamed first waits for the previous
 *    streamed call of its context to finish. Calls on different streams touching disjoint buffers are
 *    independent; calls that share buffers must be ordered by the caller.
 *  - Errors: arguments are validated on the host before anything is enqueued. On failure the
 *    call returns a non-zero cf_status, enqueues nothing, and cf_last_error() describes the
 *    problem. A failed launch returns CF_EHIP. Faults inside kernels surface at the caller's
 *    next synchronisation. Device-side index arrays (sel, tokens) are clamped inside the
 *    kernels so that bad values cannot read or write out of bounds; results are then
 *    unspecified. No C++ exception crosses this interface.
 */
#ifndef CF_H
#define CF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CF_OK = 0,
  CF_EINVAL = 1,        /* bad pointer, range or ordering */
  CF_ESHAPE = 2,        /* inconsistent sizes */
  CF_EDTYPE = 3,        /* unknown element type */
  CF_EUNSUPPORTED = 4,  /* valid but not implemented here (e.g. head_dim not 64/128) */
  CF_EWORKSPACE = 5,    /* workspace missing or smaller than the size query returned */
  CF_EHIP = 6           /* a HIP runtime call failed */
} cf_status;

typedef enum { CF_F32 = 0, CF_BF16 = 1 } cf_dtype;

typedef enum {
  CF_SEL_TOKEN_TOPK = 0, /* the k tokens of largest deviation (CacheBlend HKVD top-r%) */
  CF_SEL_DOC_SPANS = 1,  /* document-aligned spans (Request Order Matters §2.3) */
  CF_SEL_ALL = 2,        /* every row at every layer: ordinary full prefill (QCFuse Eq. 2) */
  CF_SEL_RANKED_SPANS = 3, /* spans in a caller-given order, e.g. random-document (Request Order Matters §2.3) */
  CF_SEL_SPAN_HEADS = 4, /* the first tokens of every span (EPIC, as Request Order Matters §3 describes it) */
  CF_SEL_GIVEN = 5       /* cf_blend_prefill only: the caller's set, read from out_sel (e.g. the top of cf_query_scores) */
} cf_select_mode;

/* Decoder shape. Pre-norm layer: RMSNorm -> Q,K,V projections -> optional per-head RMS
 * qk-norm -> RoPE -> causal grouped-query attention (query head h reads kv head
 * h / (n_q_heads / n_kv_heads)) -> O projection + residual -> RMSNorm -> SwiGLU
 * (silu(x Wg^T) * (x Wu^T)) Wd^T + residual. RoPE rotates the pair (x_j, x_{j+hd/2}) by
 * pos * rope_theta^(-2j/hd). */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, qk_norm;
  float rope_theta, rms_eps;
  int32_t dtype; /* cf_dtype of matrices, embedding and K/V caches */
} cf_model_cfg;

/* Device pointers of one layer. Gains are fp32; matrices are the model dtype. */
typedef struct {
  const float* attn_norm; /* [d_model] */
  const void* wq;         /* [n_q_heads*head_dim][d_model] */
  const void* wk;         /* [n_kv_heads*head_dim][d_model] */
  const void* wv;         /* [n_kv_heads*head_dim][d_model] */
  const void* wo;         /* [d_model][n_q_heads*head_dim] */
  const float* mlp_norm;  /* [d_model] */
  const void* w_gate;     /* [d_ffn][d_model] */
  const void* w_up;       /* [d_ffn][d_model] */
  const void* w_down;     /* [d_model][d_ffn] */
  const float* q_norm;    /* [head_dim], used iff qk_norm, else may be NULL */
  const float* k_norm;    /* [head_dim], used iff qk_norm, else may be NULL */
} cf_layer_weights;

/* Opaque context: a copy of the model shape, the device it was created on, and RoPE cos/sin
 * tables for offsets 0..max_pos-1 (angles computed in fp64 on the host, stored fp32). */
typedef struct cf_ctx cf_ctx;

/* Create a context on `device` (a HIP device ordinal). Requires head_dim in {64, 128},
 * n_q_heads a multiple of n_kv_heads, d_model, d_ffn and head dims multiples of 8, and
 * max_pos >= the largest position or re-position offset used later. Allocates the RoPE
 * tables (the only memory the library owns); `*out` receives the context. */
cf_status cf_ctx_create(const cf_model_cfg* cfg, int32_t max_pos, int32_t device, cf_ctx** out);
void cf_ctx_destroy(cf_ctx* ctx);

/* Thread-local text of the last error on this thread ("" if none). */
const char* cf_last_error(void);

/* Library version and build string. */
const char* cf_version(void);

/* Kernel timing for diagnostics and benchmarks. While enabled (on != 0), every kernel libcf
 * enqueues is bracketed by two HIP events recorded on the stream it runs on.
 * cf_profile_report() waits for those events and returns a JSON object
 * {"name": [launches, total_ms], ...} for the launches since the previous report; the text stays
 * valid until the next call. Process-wide, not thread-safe; costs a few microseconds per launch. */
cf_status cf_profile_enable(int32_t on);
const char* cf_profile_report(void);

/* Measurement aid: enqueue a matrix-core loop with no memory traffic (blocks_per_cu x CUs
 * blocks of 256 threads, each wave issuing iters x 4 independent 32x32x16 bf16 MFMAs) to
 * measure the achievable dense bf16 rate. out: device fp32 [blocks_per_cu * CUs * 256] (the
 * sums, so the work is kept); *flops (host) receives the flop count of the launch. The caller
 * times the stream. 1 <= blocks_per_cu <= 64, 1 <= iters. */
cf_status cf_mfma_loop(int32_t device, int32_t blocks_per_cu, int32_t iters, float* out, double* flops,
                       hipStream_t stream);

/* Measurement aid: enqueue a streaming copy of `bytes` (a multiple of 16; both pointers 16-byte
 * aligned device memory, not overlapping) with 16-byte loads and stores, one contiguous 256 KB
 * range per workgroup: the reference for the achievable HBM rate of a read + write stream. The
 * caller times it. */
cf_status cf_copy_loop(int32_t device, const void* src, void* dst, int64_t bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_rope_reposition
 * QCFuse Eq. 4 (position remap Pi_i and stitching) with CacheBlend's rotation composition.
 * For each chunk i of the host table chunk_tab[m][4] = {store_row, src_pos, dst_pos, len}
 * and each layer l in [layer_begin, layer_end):
 *   K_blend[l][dst_pos + t] = R(dst_pos - src_pos) K_store[l][store_row + t]
 *   V_blend[l][dst_pos + t] = V_store[l][store_row + t]            for t < len,
 * where R(delta) rotates each pair (x_j, x_{j+hd/2}) of every kv head by delta * omega_j
 * (delta may be negative). Rows are kvd = n_kv_heads * head_dim elements wide.
 * store_rows / blend_rows bound the row indices; strides are in elements and must be at
 * least rows * kvd. |dst_pos - src_pos| must be < max_pos of the context. Chunk
 * destinations must not overlap. Up to CF_MAX_CHUNKS chunks per call. */
#define CF_MAX_CHUNKS 256
cf_status cf_rope_reposition(const cf_ctx* ctx, const void* k_store, const void* v_store,
                             int64_t store_layer_stride, int32_t store_rows, void* k_blend,
                             void* v_blend, int64_t blend_layer_stride, int32_t blend_rows,
                             const int32_t* chunk_tab /* host [m][4] */, int32_t m,
                             int32_t layer_begin, int32_t layer_end, hipStream_t stream);

/* --------------------------------------------------------------------- cf_kv_deviation
 * Request Order Matters §2.2 Eq. 1: dev[i] = sum_c (k_new[i][c] - k_ref[i][c])^2 over the
 * kv_dim entries of row i, accumulated in fp32. Rows are ld_new / ld_ref elements apart;
 * new_dtype / ref_dtype are cf_dtype values. dev: fp32 [n_tok]. */
cf_status cf_kv_deviation(const void* k_new, int32_t new_dtype, int64_t ld_new, const void* k_ref,
                          int32_t ref_dtype, int64_t ld_ref, float* dev, int32_t n_tok,
                          int32_t kv_dim, hipStream_t stream);

/* --------------------------------------------------------------------- cf_selection_deviation
 * The selection-layer step of the method as one call (Request Order Matters §2.2 Eq. 1 at the
 * configured selection layer; CacheBlend, "Quantifying the Damage"): for the N context rows of
 * hidden (fp32, row stride d_model, rows 0..N-1 at positions 0..N-1) the current keys are
 *   K_i = RoPE_i(knorm(RMSNorm(h_i; w->attn_norm) Wk^T))      (knorm only for qk_norm models)
 * and dev[i] = sum over the kvd entries of (K_i - k_ref[i])^2, accumulated in fp32; k_ref is this
 * layer's stitched cache ([>= N][kvd], model dtype, the output of cf_rope_reposition). K_i is
 * compared in fp32 and stored nowhere. The RMSNorm rows are rounded to the model dtype before the
 * projection, as in every layer. cf_blend_prefill runs exactly these launches (same plan, same
 * results bit for bit) at its selection layer.
 *  w: host struct of device pointers (wk, attn_norm and, for qk_norm, k_norm are read).
 *  dev: device fp32 [N]. ws: device workspace of cf_selection_deviation_workspace_size(ctx, N)
 *  bytes. N = 0 enqueues nothing. */
size_t cf_selection_deviation_workspace_size(const cf_ctx* ctx, int32_t N);
cf_status cf_selection_deviation(const cf_ctx* ctx, const cf_layer_weights* w /* host struct */,
                                 const float* hidden, int32_t N, const void* k_ref, float* dev, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_topk_select
 * Choose k of the n positions by their deviation dev (fp32 [n]) and write them ascending to
 * out_idx (int32 [k]).
 *  CF_SEL_TOKEN_TOPK: the k largest values (CacheBlend HKVD; Request Order Matters §2.2).
 *    Total order: value descending, then index ascending; NaN ranks as +inf, -0 equals +0.
 *  CF_SEL_DOC_SPANS: Request Order Matters §2.3, Eq. 3. span_bounds (host, [n_spans+1],
 *    strictly increasing, 0 .. n) delimit the spans. Spans rank by (fp64 sequential span sum
 *    / span length) descending, lower span index first; whole spans are taken while they fit
 *    in the remaining budget, the walk stopping at the first span that does not; the r tokens
 *    still owed are the window [a, a+r) of that span maximising P[a+r] - P[a], P being the
 *    span's fp64 running sum from its start (smallest a among equals). Exactly k tokens.
 *    Single-window is this mode with the one span {0, n}; fixed-chunk is this mode with equal
 *    spans that cross the document bounds.
 *  CF_SEL_RANKED_SPANS: random-document (Request Order Matters §2.3): span_bounds holds the
 *    n_spans + 1 bounds followed by n_spans span indices, a permutation giving the order in
 *    which spans are taken (the caller draws it); whole spans while they fit, then the first
 *    r tokens of the first span that does not fit. dev is not read.
 *  CF_SEL_SPAN_HEADS: EPIC's first tokens of every chunk (Request Order Matters §3) at the same
 *    budget: T is the smallest head length with sum over spans of min(len, T) >= k, span j
 *    gives its first min(len_j, T) tokens, and the last spans holding T give one token back each
 *    until exactly k remain. dev is not read.
 * Results are exact (bit-identical to any implementation of the same order). 0 <= k <= n.
 * n_spans <= CF_MAX_SPANS. ws: device workspace of cf_topk_workspace_size(n, mode) bytes
 * (document-aligned mode always; token mode from n = 65536 up, where the selection runs on the
 * whole GPU; the size is 0 otherwise and ws may be NULL). Token mode also runs with less, down to
 * cf_topk_workspace_min_size(n, mode) bytes (about n / 4 + 140 KB: a 2-bit map of the n values,
 * sampled keys and per-range counts): beyond that minimum the workspace holds the values left
 * undecided by a sampled band around the threshold (4 bytes each: a list of up to n / 16 first,
 * then per-range slices; the full size has room for n / 16 in each); when they do not fit, the
 * selection falls back to histogram passes over all n values, with the same result. For the other
 * modes the two sizes are equal. A call with less than the minimum fails with CF_EWORKSPACE before
 * anything is enqueued. */
#define CF_MAX_SPANS 256
size_t cf_topk_workspace_size(int32_t n, int32_t mode);
size_t cf_topk_workspace_min_size(int32_t n, int32_t mode);
cf_status cf_topk_select(const float* dev, int32_t n, int32_t k, int32_t mode,
                         const int32_t* span_bounds /* host */, int32_t n_spans, int32_t* out_idx,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_topk_select_noalloc
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): cf_topk_select with the same arguments, modes, results
 * (bit for bit) and errors, but no workspace argument. The scratch it needs lives in a fixed device
 * array of CF_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends; the call allocates and frees nothing. A selection needing more scratch than that
 * (cf_topk_workspace_min_size(n, mode) > CF_NOALLOC_SCRATCH_BYTES: document-aligned spans beyond
 * n = 524287, token mode beyond about 15.8 million values, its undecided values taking the rest of the
 * array) fails with CF_EWORKSPACE before anything is enqueued. Every
 * call on one GPU uses that GPU's one array (the current device's), and the kernels initialise what
 * they read: calls that may overlap on one GPU (other streams, other threads) race on it and must be
 * ordered by the caller, e.g. on one stream. */
#define CF_NOALLOC_SCRATCH_BYTES (4u << 20)
cf_status cf_topk_select_noalloc(const float* dev, int32_t n, int32_t k, int32_t mode,
                                 const int32_t* span_bounds /* host */, int32_t n_spans, int32_t* out_idx,
                                 hipStream_t stream);

/* --------------------------------------------------------------------- cf_blend_layer
 * One decoder layer run only on the rows sel[0..n_sel) (CacheBlend, "Selective Recompute
 * Without Skipping"): gather + RMSNorm -> Q,K,V on those rows -> qk-norm + RoPE at position
 * sel[j] -> scatter K,V into k_cache/v_cache at rows sel[j] -> each selected row attends over
 * cache rows t <= sel[j] of the full blended cache -> O projection + residual -> SwiGLU MLP +
 * residual, written back to hidden[sel[j]] only. Rows not in sel are untouched.
 *  hidden:  fp32 [L][d_model], updated in place at the selected rows.
 *  k_cache, v_cache: this layer's cache [L][n_kv_heads][head_dim] (model dtype).
 *  sel: device int32 [n_sel], strictly ascending, values in [0, L).
 *  ws: device workspace of cf_blend_layer_workspace_size(ctx, L, n_sel) bytes.
 * With sel = 0..L-1 this is one layer of ordinary causal prefill. */
size_t cf_blend_layer_workspace_size(const cf_ctx* ctx, int32_t L, int32_t n_sel);
cf_status cf_blend_layer(const cf_ctx* ctx, const cf_layer_weights* w /* host struct */,
                         float* hidden, void* k_cache, void* v_cache, const int32_t* sel,
                         int32_t n_sel, int32_t L, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_blend_prefill
 * The whole blended prefill of one request (N context tokens then U query tokens, L = N+U):
 *  1. cf_rope_reposition of layers sel_layer..n_layers-1 from the chunk store into k_out/v_out.
 *  2. hidden = embedding rows of tokens (device int32 [L]; ids outside [0, vocab) give NaN
 *     rows).
 *  3. layers l < sel_layer: every row (ordinary prefill; their K/V overwrite k_out/v_out[l]).
 *  4. layer sel_layer: current keys of the N context rows, deviation against the stitched keys
 *     (cf_kv_deviation), selection of k positions (cf_topk_select with `mode`).
 *  5. sel = those positions followed by N..L-1; layers sel_layer.. run cf_blend_layer on sel.
 *  6. out_hidden (fp32 [U][d_model]) = final RMSNorm of the U query rows.
 * mode CF_SEL_ALL runs every layer on every row instead (store arguments unused and may be
 * NULL; k ignored): this is ordinary full prefill, used both for standalone chunk caches and
 * as the baseline. Positions are 0..L-1.
 *  layers: host array [n_layers] of device-pointer structs; embed [vocab][d_model];
 *  final_norm fp32 [d_model]; chunk store as in cf_rope_reposition;
 *  k_out/v_out: [n_layers] layers of [L][kvd], out_layer_stride elements apart (>= L*kvd);
 *  out_sel: optional device int32 [k], the selected context positions ascending; with mode
 *    CF_SEL_GIVEN it is an input: the k strictly ascending context positions to recompute (the
 *    selection-layer deviation is then not measured and out_dev is left untouched);
 *  out_dev: optional device fp32 [N], the deviation at the selection layer.
 *  0 <= k <= N; 0 <= sel_layer < n_layers; ws from cf_blend_prefill_workspace_size. */
size_t cf_blend_prefill_workspace_size(const cf_ctx* ctx, int32_t N, int32_t U, int32_t k,
                                       int32_t mode);
cf_status cf_blend_prefill(const cf_ctx* ctx, const cf_layer_weights* layers, const void* embed,
                           const float* final_norm, const int32_t* tokens, int32_t N, int32_t U,
                           const void* k_store, const void* v_store, int64_t store_layer_stride,
                           int32_t store_rows, const int32_t* chunk_tab /* host [m][4] */,
                           int32_t m, int32_t sel_layer, int32_t k, int32_t mode,
                           const int32_t* span_bounds /* host */, int32_t n_spans, void* k_out,
                           void* v_out, int64_t out_layer_stride, float* out_hidden,
                           int32_t* out_sel, float* out_dev, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* --------------------------------------------------------------------- cf_query_scores
 * Query-aware token importance (QCFuse §3.2.1 Eq. 9-10; Eq. 20 for a subset of layers): the U
 * query tokens run through layers 0 .. max(layer_set) as ordinary rows at positions N .. N+U-1
 * over the stitched cache, which they only read (context rows [0, N) are never written; the
 * query rows' own K/V are written to rows [N, L) of each layer, as the blend would). At each
 * layer l in layer_set the attention weight that the query rows put on context position t
 * (each row's softmax over the rows it sees, summed over query rows and heads) is added:
 *   scores[t] = sum over l in layer_set of Attn^l(Q_U, K_C)_t,  t < N.
 * The top of these scores (cf_topk_select, token mode) is a query-aware recompute set; pass it
 * to cf_blend_prefill with mode CF_SEL_GIVEN.
 *  tokens: device int32 [L = N + U] (only the U query tokens at N.. are read).
 *  k_cache, v_cache: the stitched cache (cf_rope_reposition of every layer), [n_layers] layers
 *    of [L][kvd] out_layer_stride elements apart.
 *  layer_set: host int32 [n_set], strictly increasing layer ids.
 *  scores: device fp32 [N] (written, not accumulated across calls).
 *  ws: device workspace of cf_query_scores_workspace_size(ctx, N, U) bytes. N > 0, U > 0. */
size_t cf_query_scores_workspace_size(const cf_ctx* ctx, int32_t N, int32_t U);
cf_status cf_query_scores(const cf_ctx* ctx, const cf_layer_weights* layers, const void* embed,
                          const int32_t* tokens, int32_t N, int32_t U, void* k_cache, void* v_cache,
                          int64_t out_layer_stride, const int32_t* layer_set /* host */, int32_t n_set,
                          float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- chunk-anchor query probing
 * QCFuse's compressed token view (§3.3): a few anchor tokens per chunk stand in for the whole
 * context when the query is probed, and the resulting query states score the original context
 * positions at a few critical layers (§3.4).
 *
 * cf_key_norms: Knorm's anchor score (QCFuse §3.3.1): norms[r] = the squared L2 norm of store row
 * r's keys over layers [layer_begin, layer_end) and all kv heads (fp32), for the store_rows rows of
 * a chunk store laid out as in cf_rope_reposition (RoPE preserves the norm, so stored keys at any
 * position give the same score). norms: device fp32 [store_rows]. */
cf_status cf_key_norms(const cf_ctx* ctx, const void* k_store, int64_t store_layer_stride, int32_t store_rows,
                       int32_t layer_begin, int32_t layer_end, float* norms, hipStream_t stream);

/* Anchor positions (QCFuse §3.3.1 Eq. 14-15), host arithmetic like the policy functions below:
 * for each chunk i of the host table chunk_tab[m][4] = {store_row, src_pos, dst_pos, len}, the
 * ceil(r_a * len) chunk-local positions of highest score G_i (equal scores: the lower position;
 * r_a = ra_num / ra_den), written as request positions dst_pos + r, all chunks together in
 * ascending order into anchors (host int32 [cap]); *n_anchors receives the count even when cap is
 * too small (then CF_EINVAL).
 *  CF_ANCHOR_SINK: G_i(r) = -r, the first tokens of each chunk (scores unused, may be NULL);
 *  CF_ANCHOR_KNORM: G_i(r) = scores[store_row + r] (host fp32, e.g. cf_key_norms copied back),
 *    the largest key norms; CF_ANCHOR_KNORM_LOW: the smallest (NaN ranks as +inf in both). */
typedef enum { CF_ANCHOR_SINK = 0, CF_ANCHOR_KNORM = 1, CF_ANCHOR_KNORM_LOW = 2 } cf_anchor_rule;
cf_status cf_anchor_positions(int32_t rule, const int32_t* chunk_tab /* host [m][4] */, int32_t m, int32_t ra_num,
                              int32_t ra_den, const float* scores /* host */, int32_t store_rows,
                              int32_t* anchors /* host */, int32_t cap, int32_t* n_anchors);

/* cf_query_scores_anchored: anchor-conditioned query probing (QCFuse §3.3.2 Eq. 15-17) and
 * critical-layer scoring (§3.4 Eq. 18 and Eq. 20). The U query tokens (positions N..N+U-1) run
 * through layers 0..max(layer_set) with only the n_anchors rows of the stitched cache at the
 * given positions as their prefix (each anchor keeps its request position, its keys being the
 * re-positioned PIC entries, Eq. 16); at each layer l of layer_set the probe's query states score
 * every original context position t against the full stitched keys of that layer:
 *   scores[t] = sum over l in layer_set of the softmax weight the query rows (summed over rows and
 *   heads) put on context row t, each row's softmax running over all N context rows and the query
 *   rows up to itself (as in cf_query_scores, which this equals when every context position is an
 *   anchor).
 * The query rows' K/V of each scored layer are written to rows [N, L) of that layer of the caller's
 * cache; context rows are only read.
 *  anchors: device int32 [n_anchors], strictly increasing positions in [0, N) (values are clamped
 *    in the kernels; other arrays give unspecified results). 0 <= n_anchors <= N.
 *  Other arguments as in cf_query_scores; ws: cf_query_scores_anchored_workspace_size(ctx, N, U,
 *  n_anchors) bytes. */
size_t cf_query_scores_anchored_workspace_size(const cf_ctx* ctx, int32_t N, int32_t U, int32_t n_anchors);
cf_status cf_query_scores_anchored(const cf_ctx* ctx, const cf_layer_weights* layers, const void* embed,
                                   const int32_t* tokens, int32_t N, int32_t U, void* k_cache, void* v_cache,
                                   int64_t out_layer_stride, const int32_t* anchors, int32_t n_anchors,
                                   const int32_t* layer_set /* host */, int32_t n_set, float* scores, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_blend_prefill_streamed
 * cf_blend_prefill with the chunk store in host memory, loaded layer by layer while the
 * previous layers are recomputed (CacheBlend, "Hiding Recompute Behind I/O": selective
 * recompute of one layer runs while the next layer's cache is fetched). Layer l >= sel_layer
 * of k_store/v_store (store_rows * kvd elements each, at element offset l * store_layer_stride)
 * is copied host-to-device into one of two workspace staging slots on the context's copy
 * stream, two layers ahead, and re-positioned from its slot into k_out/v_out on that same
 * stream, which then refills the slot with layer l + 2; `stream` waits for layer l right
 * before using it. The copy stream's work begins after the work already enqueued on `stream`
 * and every part of it is waited for on `stream`, so the call stays stream-ordered; this holds
 * for a call that fails after its first copy was queued too (the error is returned after
 * `stream` has been made to wait for the copy stream). Results are those of cf_blend_prefill with the same arguments.
 *  k_store, v_store: PINNED host memory (hipHostMalloc or equivalent), same layout as in
 *    cf_blend_prefill; other memory is rejected with CF_EINVAL. The caller keeps them unchanged
 *    until the stream has passed the call.
 *  ws: device workspace of cf_blend_prefill_streamed_workspace_size(ctx, N, U, k, mode,
 *    store_rows) bytes.
 * One streamed call per context is in flight at a time: a call first waits on the host for the
 * previous streamed call of the same context to finish (copies queued behind an earlier,
 * still running call stalled the enqueueing thread inside the runtime and slowed that call).
 * The context's copy stream and events are shared by its calls: calls of this function on one
 * context must be made from one host thread at a time. */
size_t cf_blend_prefill_streamed_workspace_size(const cf_ctx* ctx, int32_t N, int32_t U, int32_t k,
                                                int32_t mode, int32_t store_rows);
cf_status cf_blend_prefill_streamed(const cf_ctx* ctx, const cf_layer_weights* layers, const void* embed,
                                    const float* final_norm, const int32_t* tokens, int32_t N, int32_t U,
                                    const void* k_store /* pinned host */, const void* v_store /* pinned host */,
                                    int64_t store_layer_stride, int32_t store_rows,
                                    const int32_t* chunk_tab /* host [m][4] */, int32_t m, int32_t sel_layer,
                                    int32_t k, int32_t mode, const int32_t* span_bounds /* host */,
                                    int32_t n_spans, void* k_out, void* v_out, int64_t out_layer_stride,
                                    float* out_hidden, int32_t* out_sel, float* out_dev, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- cf_blend_prefill_gradual
 * Blended prefill with gradual filtering (CacheBlend, "The Chicken-and-Egg Problem"): the
 * recompute set narrows layer by layer instead of staying fixed. Steps 1-4 are those of
 * cf_blend_prefill in token mode with k = k_sched[0]. Then layer sel_layer + i recomputes
 * k_sched[i] context rows (plus the U query rows):
 *  - at each layer l = sel_layer + i with 0 < i < n_layers - sel_layer - 1, the deviation of the
 *    set's fresh keys against the stitched keys they replace is measured (Request Order
 *    Matters §2.2 Eq. 1, fused into the key store: the old key is read before it is
 *    overwritten);
 *  - when k_sched[i + 1] < k_sched[i], layer l + 1 recomputes the k_sched[i + 1] rows of layer
 *    l's set with the largest deviation (ties keep the lower position); after layer sel_layer
 *    this is the top of the selection-layer ranking.
 *  k_sched: host int32 [n_layers - sel_layer], k_sched[0] <= N, non-increasing, >= 0.
 *  out_sets: optional device int32 [sum of k_sched]: each layer's set, ascending, layer by layer.
 *  out_devs: optional device fp32 [N + sum of k_sched[i] for 0 < i < n_layers - sel_layer - 1]:
 *    the selection-layer deviation over the N context rows, then each such layer's deviation
 *    over its set, in set order.
 *  ws: device workspace of cf_blend_prefill_gradual_workspace_size(ctx, N, U, sel_layer,
 *    k_sched) bytes (0 if the schedule is invalid). Other arguments, ownership and errors as in
 *    cf_blend_prefill; an invalid schedule is CF_EINVAL. */
size_t cf_blend_prefill_gradual_workspace_size(const cf_ctx* ctx, int32_t N, int32_t U, int32_t sel_layer,
                                               const int32_t* k_sched /* host */);
cf_status cf_blend_prefill_gradual(const cf_ctx* ctx, const cf_layer_weights* layers, const void* embed,
                                   const float* final_norm, const int32_t* tokens, int32_t N, int32_t U,
                                   const void* k_store, const void* v_store, int64_t store_layer_stride,
                                   int32_t store_rows, const int32_t* chunk_tab /* host [m][4] */, int32_t m,
                                   int32_t sel_layer, const int32_t* k_sched /* host */, void* k_out,
                                   void* v_out, int64_t out_layer_stride, float* out_hidden, int32_t* out_sets,
                                   float* out_devs, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------------------- policy arithmetic (host)
 * The integer and scalar bookkeeping of the method. These functions read and write host memory
 * only, take no context or stream, never touch the device, and return CF_EINVAL (with
 * cf_last_error text) on a bad argument, leaving outputs untouched unless stated otherwise.
 * Ratios are exact rationals num/den with 0 <= num <= den and den > 0. */

/* Recompute budget (Request Order Matters §2.2 Eq. 2; ratio as in QCFuse §2.1.3 Eq. 6):
 * *k = max(1, floor(n_ctx * num / den)) when num > 0 and n_ctx > 0, else 0 (the direct-reuse
 * endpoint). Integer arithmetic: floating point puts 0.15 * 3072 and 0.29 * 100 just below the
 * integer. n_ctx >= 0 counts context tokens only (the query is never ranked). */
cf_status cf_budget(int32_t n_ctx, int32_t rho_num, int32_t rho_den, int32_t* k);

/* Gradual-filtering schedule (CacheBlend, "The Chicken-and-Egg Problem": the recompute ratio
 * narrows r_1 > r_2 > ... toward r, each layer keeping part of the previous layer's set):
 * k_sched[0] = budget(n_ctx, first), then k_sched[i+1] = max(budget(n_ctx, final),
 * max(1, floor(k_sched[i] * keep))) while k_sched[i] > 0 (0 stays 0). Writes n_sched counts to
 * k_sched (host int32 [n_sched]), the layout cf_blend_prefill_gradual reads. The final ratio
 * must not exceed the first. */
cf_status cf_gradual_schedule(int32_t n_ctx, int32_t n_sched, int32_t first_num, int32_t first_den,
                              int32_t keep_num, int32_t keep_den, int32_t final_num, int32_t final_den,
                              int32_t* k_sched);

/* Loading controller (CacheBlend, "Hiding Recompute Behind I/O"): among the n candidate ratios
 * ratios[i] = {num, den} (host int32 [n][2]) whose measured per-layer recompute time
 * recompute_ms[i] (host double [n]) is at most the per-layer cache load time load_ms, take the
 * largest (the first among equal ratios), then clamp it from below at the floor r* = floor_num /
 * floor_den: r = max(r_load, r*). With no candidate fitting, r = r*. */
cf_status cf_loading_ratio(double load_ms, const int32_t* ratios, const double* recompute_ms, int32_t n,
                           int32_t floor_num, int32_t floor_den, int32_t* out_num, int32_t* out_den);

/* Span bounds of the span-policy ablations (Request Order Matters §2.3 and §4.4), for
 * cf_topk_select / cf_blend_prefill in CF_SEL_DOC_SPANS mode. bounds: host int32 [cap]; *n_bounds
 * receives the number of bounds (spans + 1) even when cap is too small (then CF_EINVAL).
 *  single-window: the one span {0, n_ctx}, so the document-aligned rule takes the k-token window
 *    of largest total deviation anywhere in the context.
 *  fixed-chunk: spans of `size` tokens that cross document bounds, shifted by `offset`
 *    (0 <= offset < size; the page's offset is unstated): 0, offset, offset + size, ..., n_ctx
 *    (offset 0 gives 0, size, 2 size, ...). n_ctx = 0 gives {0, 0}. */
cf_status cf_single_window_bounds(int32_t n_ctx, int32_t* bounds, int32_t cap, int32_t* n_bounds);
cf_status cf_fixed_chunk_bounds(int32_t n_ctx, int32_t size, int32_t offset, int32_t* bounds, int32_t cap,
                                int32_t* n_bounds);

/* Selection diagnostics of Request Order Matters §4.4 Table 2 for k distinct positions sel (host
 * int32 [k], any order, each in [0, n)) and the selection-layer deviation dev (host fp32 [n]):
 * *segments = the number of maximal runs of consecutive selected positions; *captured = the share
 * of the total deviation that the selected positions carry, both totals summed in fp64 with NaN
 * counted as +inf (0 when the total is 0). */
cf_status cf_selection_stats(const int32_t* sel, int32_t k, const float* dev, int32_t n, int32_t* segments,
                             double* captured);

#ifdef __cplusplus
}
#endif
#endif /* CF_H */
