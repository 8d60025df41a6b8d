// Host-side launchers of the libcf kernels (internal; the public interface is include/cf.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cf {

enum Dt { F32 = 0, BF16 = 1 };

// ----------------------------------------------------------------- row kernels (rows.hip)
constexpr int CHUNKS_PER_LAUNCH = 64;
struct ChunkBatch {
  int n;
  int row[CHUNKS_PER_LAUNCH];
  int dst[CHUNKS_PER_LAUNCH];
  int len[CHUNKS_PER_LAUNCH];
  int delta[CHUNKS_PER_LAUNCH];
  int blk0[CHUNKS_PER_LAUNCH + 1];  // first block of each chunk (prefix sums of row blocks)
};
constexpr int REPOS_ROWS_PER_BLOCK = 4;

hipError_t launch_reposition(Dt dt, const void* ks, const void* vs, int64_t sls, void* kb, void* vb,
                             int64_t bls, const ChunkBatch& cb, int kvd, int hd, const float* cos_t,
                             const float* sin_t, int layer_begin, int n_layers, hipStream_t st);
hipError_t launch_embed(Dt dt, const int* tok, int L, const void* emb, int vocab, int d, float* h,
                        hipStream_t st);
// out[j] = RMSNorm(x[rows ? rows[j] : j]) * g, written as `out_dt` with row stride ldo.
hipError_t launch_rmsnorm_rows(Dt out_dt, const float* x, const int* rows, int n, int L, int d,
                               const float* g, float eps, void* out, int64_t ldo, hipStream_t st);
// Post-process fp32 projection rows: qk-norm, RoPE at pos = rows[j], Q -> q_out (model dtype),
// K/V scattered into the cache at row pos. With dev != nullptr, only K is present (ld = kvd),
// positions are j, and dev[j] = sum (rope(k) - k_ref[j])^2; nothing is stored. With dev_heads
// (store mode, hd 64 or 128), rows j < n_dev also get dev_heads[j * hkv + h] = sum over head h
// of (rope(k) - the cached key it replaces)^2, read before the store.
struct QkvPost {
  const float* qkv; int64_t ld;
  const int* rows; int n; int L;
  int hq, hkv, hd; int qk_norm; const float* qn; const float* kn; float eps;
  const float* cos_t; const float* sin_t;
  void* q_out; void* k_cache; void* v_cache;
  float* dev; const void* k_ref;
  int splits; int64_t split_stride;    // qkv holds `splits` partial sums, split_stride floats apart
  float* dev_heads; int n_dev;
  int rope_off;                        // RoPE position = stored row + rope_off (0: the row itself)
};
hipError_t launch_qkv_post(Dt dt, const QkvPost& p, hipStream_t st);
// dev[j] = sum over h < hkv of dev_heads[j * hkv + h], in head order (j < n).
hipError_t launch_dev_rows(const float* dev_heads, int n, int hkv, float* dev, hipStream_t st);
// Narrowed recompute set: sel[j] = prev[sel[j]] for j < k (sel holds indices into prev on entry),
// then sel[k + u] = n_ctx + u for u < U (the query rows).
hipError_t launch_sel_map(int* sel, const int* prev, int k, int U, int n_ctx, hipStream_t st);
hipError_t launch_iota(int* out, int n, int start, hipStream_t st);
hipError_t launch_copy_i32(int* dst, const int* src, int n, hipStream_t st);
hipError_t launch_copy_f32(float* dst, const float* src, int n, hipStream_t st);
// out[out_rows[m]][c] = resid[resid_rows[m]][c] + sum_s part[s][m][c]   (rows may be null)
hipError_t launch_splitk_reduce(const float* part, int splits, int M, int N, const float* resid,
                                const int* resid_rows, float* out, const int* out_rows, int L,
                                hipStream_t st);
// Split-K reduction fused with the residual and the next RMSNorm:
// out[out_rows[m]] = resid[resid_rows[m]] + sum_s part[s][m]; x[m] = RMSNorm(that row) * g (model
// dtype); null row maps are the identity.
hipError_t launch_reduce_resid_norm(Dt dt, const float* part, int splits, int M, int d, const float* resid,
                                    const int* resid_rows, float* out, const int* out_rows, int L, const float* g,
                                    float eps, void* x, hipStream_t st);
// act[m][c] = silu(gu[m][c]) * gu[m][F + c]  (fp32 path)
hipError_t launch_swiglu(Dt dt, const float* gu, int M, int F, void* act, hipStream_t st);
hipError_t launch_deviation(Dt dn, const void* a, int64_t lda, Dt dr, const void* b, int64_t ldb,
                            float* dev, int n, int kvd, hipStream_t st);
// dst[j] = src[idx ? idx[j] (clamped to [0, src_rows)) : j] for j < n; rows of row_elems elements
// (row_elems * element size a multiple of 16 bytes), leading dimensions in elements.
hipError_t launch_gather_rows(Dt dt, const void* src, int64_t src_ld, int src_rows, const int* idx, int n,
                              int row_elems, void* dst, int64_t dst_ld, hipStream_t st);
// norms[r] = sum over layers [lb, le) of the squared entries of K[l][r] (rows of kvd elements,
// layers sls elements apart), fp32.
hipError_t launch_key_norms(Dt dt, const void* k, int64_t sls, int rows, int kvd, int lb, int le, float* norms,
                            hipStream_t st);

// ----------------------------------------------------------------- measurement (probe.hip)
// Launches blocks x 256 threads of the MFMA loop; returns its flop count.
double launch_mfma_loop(int blocks, int iters, float* out, hipStream_t st);
void launch_copy_loop(const void* src, void* dst, int64_t n16, hipStream_t st);

// ----------------------------------------------------------------- GEMM (gemm.hip)
enum Epi { EPI_F32 = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_PARTIAL = 3 };
struct GemmArgs {
  Dt dt;
  int cfg;                             // kernel / tile configuration (GemmCfgId), from gemm_plan
  const void* A; int64_t lda;          // [M][K]
  const void* B[3]; int nb0, nb1;      // weights [n][K] (row stride K): cols [0,nb0) from B[0],
                                       // [nb0,nb1) from B[1], [nb1,N) from B[2]
  int M, N, K;
  int splits;                          // split-K factor (>= 1); EPI_PARTIAL writes part[s]
  int epi;
  float* C; int64_t ldc;               // EPI_F32 / EPI_PARTIAL destination ([splits][M][ldc])
  void* act; int64_t ld_act;           // EPI_SWIGLU: N = d_ffn, B[0] = gate, B[1] = up
  const float* resid; const int* resid_rows; float* out; const int* out_rows; int L;  // EPI_RESID
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
enum GemmCfgId {
  GEMM_SMALL = 0, GEMM_DTL128 = 1, GEMM_DTL96 = 2, GEMM_DTL64 = 3, GEMM_DTL256 = 4, GEMM_DTL128N = 5, GEMM_DTL64N = 6,
  GEMM_DTL224 = 7
};
struct GemmPlan { int cfg; int splits; };
// Kernel, block height and split-K factor for an M x N x K product: a direct-to-LDS kernel when
// K % 64 == 0 (else the register-staged one), choosing the pair that minimises (rounds of
// resident blocks) x (work per block) / (per-CU rate of that block shape). Split-K is only
// considered when allow_split (the epilogue is linear in the accumulator).
GemmPlan gemm_plan(Dt dt, int M, int N, int K, bool swiglu, bool allow_split, int n_cu);

// ----------------------------------------------------------------- attention (attn.hip)
// Work-balanced key pieces for the selected rows: query tile qt (128 / G consecutive rows) has c
// key blocks of 64 up to its last row's position; it is cut into pieces of `chunk` key blocks,
// pieces [off[qt], off[qt + 1]); T <= P pieces in all, chunk the smallest for which they fit.
// Built on the device from the positions. piece[t] holds what the block running piece t needs, in
// one record: its tile's first row, its key range [kbeg, kend) and its partial-sum slot (t when
// the tile has several pieces, else -1).
constexpr int ATTN_MAXQ = 256, ATTN_MAXP = 256;
struct AttnSched {
  int4 piece[ATTN_MAXP];
  int T; int off[ATTN_MAXQ + 1];
};
struct AttnArgs {
  Dt dt;
  const void* q; int64_t ldq;          // [n][hq*hd]
  const int* pos; int n;               // absolute positions, ascending
  const void* k; const void* v; int L; // cache [L][hkv*hd]
  int hq, hkv, hd;
  void* out; int64_t ldo;              // [n][hq*hd] (model dtype)
  float* o_part; float* ml_part;       // pieces' partial sums: [hkv][P][128][hd], [hkv][P][128][2]
  const AttnSched* sched; int P;       // balanced pieces (bf16): P blocks per kv head, else null
                                       // (whole query tiles)
  float* ml_out;                       // optional [n][hq][2]: each row's softmax max and sum (log2
                                       // units: weights are exp2(s log2(e) / sqrt(hd) - m) / l)
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);        // main pass
hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t st);  // merge of the pieces
hipError_t launch_attention_sched(const AttnArgs& a, AttnSched* s, hipStream_t st);  // pieces for a.pos
// *P > 0: balanced pieces with P blocks per kv head; 0: whole query tiles
void attn_plan(Dt dt, int n, int hq, int hkv, int n_cu, int* P);

// ----------------------------------------------------------------- query-aware scores (qmass.hip)
// Attention mass of n query rows (Q [n][hq*hd] with row stride ldq, softmax max/sum ml [n][hq][2]
// from the layer's attention) on the context keys k [0, n_ctx) (cache [.][hkv*hd]): part [hkv][n_ctx]
// scratch, score[t] = (first ? 0 : score[t]) + the mass on t summed over rows and heads.
struct QMassArgs {
  const void* q; int64_t ldq; int n;
  const void* k; int n_ctx;
  int hq, hkv, hd;
  const float* ml; float* part; float* score;
};
hipError_t launch_query_mass(Dt dt, const QMassArgs& a, int first, hipStream_t st);

// ----------------------------------------------------------------- selection (topk.hip)
constexpr int MAX_SPANS = 256;
// Span selections: mode 1 document-aligned (rank by mean deviation, best window in the first span
// that does not fit), 3 ranked by order[] (deviation unused, head of the first span that does not
// fit), 4 heads of every span (deviation unused, the budget shared evenly).
enum SpanMode { SPAN_DOC = 1, SPAN_RANKED = 3, SPAN_HEADS = 4 };
struct SpanArgs { int n_spans; int mode; int b[MAX_SPANS + 1]; int order[MAX_SPANS]; };
// ws: topk_token_ws_bytes(n) bytes (none below the large-n threshold, where one workgroup runs). At
// least topk_token_ws_min_bytes(n) are required (state, sampled keys, per-range counts and a 2-bit
// map of the n keys); what lies beyond them holds the undecided keys (4 bytes each: a list of up to
// n / 16, then per-range slices), and with less room the selection falls back to histogram passes
// over all n keys (same result).
size_t topk_token_ws_bytes(int n);
size_t topk_token_ws_min_bytes(int n);
hipError_t launch_topk_token(const float* dev, int n, int k, int* out, void* ws, size_t ws_bytes, hipStream_t st);
hipError_t launch_topk_spans(const float* dev, int n, int k, const SpanArgs& sp, int* out,
                             double* ws, hipStream_t st);

// ----------------------------------------------------------------- fixed scratch (noalloc.hip)
// Device address of the library's fixed scratch array (CF_NOALLOC_SCRATCH_BYTES) on the current
// device, looked up with that device current on the first call per device and kept.
hipError_t noalloc_scratch(void** out);

}  // namespace cf
