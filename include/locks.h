/*
 * locks.h -- C ABI of the LOCKS decode hot path on MI355X (gfx950).
 *
 * LOCKS ("LOCKS: Page-Local Compact Key Summaries for Efficient Long-Context
 * Decoding"; gist.science explainer, technical summary sec. 2, and the
 * paper's abstract) keeps the full paged KV cache, gives every page a small
 * spectral summary of its keys, estimates each page's attention mass from the
 * summaries alone, and runs attention over only the top pages.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *    memory; the library allocates nothing, never synchronizes and never
 *    reads device memory on the host, so every call may be captured in a
 *    HIP graph.
 *  - `stream` is a hipStream_t passed as void*.  Work is enqueued on it and
 *    the call returns at once.
 *  - Arguments are validated on the host before anything is launched; on
 *    failure a negative status is returned and nothing is launched.  A launch
 *    error returns LOCKS_ERR_LAUNCH.  Faults inside kernels surface at the
 *    caller's next synchronization.
 *  - Supported shape: head_dim 128, page_size 16, rank 4, 8 or 16 (8 is the
 *    pages' setting; 4 and 16 are the same method at other state sizes), and
 *    num_q_heads a multiple of num_kv_heads with a GQA group G = Hq / Hkv of
 *    1, 2, 4 or 8 query heads per KV head (sec. 2 group-shared selection: the
 *    G heads of a group share one page table); anything else returns
 *    LOCKS_ERR_UNSUPPORTED.
 *  - bf16 tensors are raw bfloat16 bit patterns (uint16).
 *  - Alignment: q, k_cache, v_cache and summaries 16 bytes; every other array
 *    (int32 and fp32 arrays, the bf16 output) 4 bytes; a misaligned one
 *    returns LOCKS_ERR_SHAPE.  Workspaces 16 bytes, else LOCKS_ERR_WORKSPACE.
 *  - Device-side data (seq_lens, block tables, selections) is range-checked
 *    in the kernels: a sequence length is clamped to max_pages * 16, and a
 *    block id outside [0, num_blocks) makes that page count as absent.
 *  - The library keeps no state and is safe to call from several threads.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t locks_status;
#define LOCKS_OK 0
#define LOCKS_ERR_NULL (-1)        /* a required pointer is NULL            */
#define LOCKS_ERR_SHAPE (-2)       /* a size or stride is out of range     */
#define LOCKS_ERR_UNSUPPORTED (-3) /* dims outside the supported shape     */
#define LOCKS_ERR_WORKSPACE (-4)   /* workspace missing or too small       */
#define LOCKS_ERR_LAUNCH (-5)      /* the HIP runtime refused a launch     */

typedef struct {
  int32_t num_q_heads;  /* Hq                                      */
  int32_t num_kv_heads; /* Hkv; Hq / Hkv is the GQA group size G   */
  int32_t head_dim;     /* d (128)                                 */
  int32_t page_size;    /* B, tokens per KV page (16)              */
  int32_t rank;         /* r, basis vectors per page summary (4, 8 or 16) */
  int32_t newest_page_pending; /* 0 or 1, see below                  */
} locks_dims;

/* Summarized pages.  With newest_page_pending = 0 the summarized (finalized)
 * pages of a sequence of n tokens are its n / 16 full pages, and the n % 16
 * tokens after them (the partial tail page) are attended in full, outside
 * the budget.  With newest_page_pending = 1 the page that holds the newest
 * token is not summarized yet even when it is full: the summarized pages are
 * the first (n - 1) / 16, and the 1 to 16 tokens after them are attended in
 * full.  This is the decode step whose pages are summarized off its critical
 * path (sec. 2 implementation): a page completed by the step's token is
 * summarized after the step (locks_finalize_pages on the new lengths) and
 * selected from the next step on.  Every call that scores, selects or
 * attends reads the flag the same way; the builders ignore it. */

/* Element strides (bf16 elements) of one layer's paged K or V cache:
 * element (block, kv_head, token, dim) sits at
 *   block*block_stride + kv_head*head_stride + token*token_stride + dim. */
typedef struct {
  int64_t block_stride;
  int64_t head_stride;
  int64_t token_stride;
} locks_kv_layout;

/* Bytes of one summary record per (page, KV head): 84r + 130 bytes of fields
 * padded to a multiple of 64: 832 at r=8 (codes 768 B + 17 fp16 scales; about
 * 10% of the page-head's 8192 K+V bytes, sec. 2 quantization paragraph), 512
 * at r=4, 1536 at r=16.  Returns 0 for unsupported dims. */
size_t locks_summary_bytes(const locks_dims* dims);

/* Workspace sizes (bytes).  max_pages is the block-table row length; the
 * budget is in pages.  Workspace contents need no initialization; a
 * workspace must not be shared by calls that may run concurrently.
 *
 * locks_workspace_bytes: one size that serves every decode-path call with
 * these sizes -- the `workspace` of locks_score_pages, locks_select_pages,
 * locks_score_select and locks_sparse_attend (sparse or dense), and the
 * single workspace of locks_decode_layer when its attend_ws is NULL.
 * Returns 0 for unsupported dims or sizes (budget_pages must be >= 1).
 *
 * locks_score_workspace_bytes / locks_attend_workspace_bytes: the smaller
 * sizes of the scoring-and-selection part and of the attention part alone
 * (max_attended_pages = budget_pages + 1 for a sparse pass, max_pages + 1 for
 * a dense one). */
size_t locks_workspace_bytes(const locks_dims* dims, int32_t batch, int32_t max_pages,
                             int32_t budget_pages);
size_t locks_score_workspace_bytes(const locks_dims* dims, int32_t batch,
                                   int32_t max_pages, int32_t budget_pages);
size_t locks_attend_workspace_bytes(const locks_dims* dims, int32_t batch,
                                    int32_t max_attended_pages);

/* Build the summaries of whole pages ("page finalization", sec. 2 core
 * mechanism: centroid, a small eigendecomposition of the centered keys, the
 * top-r eigenvectors and one coefficient vector per token; int4 basis, int8
 * coefficients and centroid).
 *   k_cache    : bf16 K of one layer, strides `layout`.
 *   block_ids  : [n_blocks] physical blocks to summarize (all KV heads).
 *   num_blocks : physical blocks in the layer (record array extent).
 *   summaries  : [Hkv][num_blocks][locks_summary_bytes] records, written for
 *                the listed blocks only.
 *   raw_debug  : nullable; fp32 [n_blocks][Hkv][128 + 144 r] unquantized
 *                summary (mu[128], V as [r][128], C as [16][r]) for testing
 *                (1280 floats at r=8).
 * Record layout (little-endian), offsets for rank r (r=8 in brackets):
 *   [0, 64r)          [0,512) basis codes, int4 two's complement in [-7,7]:
 *                     column k owns bytes [64k, 64k+64); 32-bit word w covers
 *                     dims [8w, 8w+8); byte m of the word holds dim 8w+m in its
 *                     low nibble and dim 8w+4+m in its high nibble.
 *   [64r, 80r)        [512,640) coefficient codes int8 [16 tokens][r columns].
 *   [80r, 80r+128)    [640,768) centroid codes int8 [128].
 *   [80r+128, 82r+128) [768,784) fp16 basis scales s_V[r];
 *   [82r+128, 84r+128) [784,800) fp16 coefficient scales s_c[r];
 *   [84r+128, +2)     [800,802) fp16 centroid scale; zero to the record end.
 *   Dequantized: mu = s_mu*mu_q, v_k = s_V[k]*V_q[:,k], c_ik = s_c[k]*C_q[i,k].
 * A record depends only on its page-head's keys: the same bytes whatever else
 * the call lists, in whatever order, and the same as locks_finalize_pages
 * writes for that page.  Block ids outside [0, num_blocks) are skipped;
 * a block listed twice gets the same record twice.
 */
locks_status locks_build_summaries(const locks_dims* dims, const void* k_cache,
                                   locks_kv_layout layout, const int32_t* block_ids,
                                   int32_t n_blocks, int32_t num_blocks, void* summaries,
                                   float* raw_debug, void* stream);

/* One layer of the decode step in one call: locks_score_select followed by
 * locks_sparse_attend (sec. 2 implementation: scoring, selection and sparse
 * attention run back to back inside the step's graph), with outputs
 * identical to those two calls when softmax_scale = 1/sqrt(d).  Pages are
 * scored at the logit scale they are attended with: the estimate's 1/sqrt(d)
 * (sec. 2 equation) is replaced by softmax_scale.  The last selection stage runs inside the
 * attention kernel when budget_pages <= 1024 and the chunk candidates number
 * at most 8192 (for one sequence, contexts up to 2M tokens at budget 2048
 * tokens; large batches use 4096-page chunks and fit twice that); otherwise
 * the stages run as in the two calls.
 *   summaries, k_cache, v_cache share the physical block numbering
 *   (num_blocks) and the block table.
 *   sel, sel_count : written as by locks_select_pages.
 *   out, out_lse   : as written by locks_sparse_attend.
 *   score_ws       : >= locks_score_workspace_bytes(dims, batch, max_pages,
 *                    budget_pages), 16-byte aligned.
 *   attend_ws      : >= locks_attend_workspace_bytes(dims, batch,
 *                    budget_pages + 1); or NULL, in which case score_ws holds
 *                    both parts and must be >= locks_workspace_bytes(dims,
 *                    batch, max_pages, budget_pages) (score_ws_bytes is
 *                    checked against the two parts). */
locks_status locks_decode_layer(const locks_dims* dims, const void* q, const void* summaries,
                                const void* k_cache, const void* v_cache, locks_kv_layout layout,
                                int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                float softmax_scale, int32_t* sel, int32_t* sel_count, void* out,
                                float* out_lse, void* score_ws, size_t score_ws_bytes,
                                void* attend_ws, size_t attend_ws_bytes, void* stream);

/* locks_decode_layer for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * kernels and outputs as locks_decode_layer (with one workspace), but the
 * workspace is the library's own device array of LOCKS_NOALLOC_SCRATCH_BYTES
 * (64 MiB), held by every GPU the library runs on until the process ends.
 * The call allocates and frees nothing.
 *   locks_decode_layer_noalloc_bytes : scratch bytes a call with these sizes
 *     uses (0 for unsupported dims or sizes); at most 64 MiB is accepted:
 *     about 10 MiB for one 1M-token sequence, 12 MiB for 8 x 128K tokens and
 *     38 MiB for 16 x 256K tokens (32 query heads, budget 128 pages).
 *   Larger requests return LOCKS_ERR_WORKSPACE before anything is launched;
 *   invalid shapes return what locks_decode_layer would.
 *   The first call on each device looks up that device's array address
 *   (hipGetSymbolAddress; make it outside graph capture).  Every call on one
 *   GPU shares that GPU's array and leaves its contents behind: calls that
 *   may overlap on one GPU (two streams, two threads) race on it and must be
 *   serialized by the caller.  Nothing in the array needs clearing between
 *   calls: every byte a call reads it has written first. */
#define LOCKS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t locks_decode_layer_noalloc_bytes(const locks_dims* dims, int32_t batch, int32_t max_pages,
                                        int32_t budget_pages);
locks_status locks_decode_layer_noalloc(const locks_dims* dims, const void* q,
                                        const void* summaries, const void* k_cache,
                                        const void* v_cache, locks_kv_layout layout,
                                        int32_t num_blocks, const int32_t* block_table,
                                        int32_t max_pages, const int32_t* seq_lens,
                                        int32_t batch, int32_t budget_pages, float softmax_scale,
                                        int32_t* sel, int32_t* sel_count, void* out,
                                        float* out_lse, void* stream);

/* Incremental finalization inside the decode step (sec. 2 implementation:
 * a page is summarized once, when it is finalized, off the critical path).
 * For every sequence b whose length seq_lens[b] is a positive multiple of 16
 * -- the newest token has just completed its page -- the summary of logical
 * page seq_lens[b]/16 - 1 is (re)built for every KV head, exactly as
 * locks_build_summaries would build it.  The decision is taken on the
 * device, so the call can sit in a captured graph and be replayed every
 * step; sequences whose tail page is partial are left untouched.  One call
 * serves n_layers layers at once (all their pages are built in parallel).
 * Called after the step, for every layer at once, when the step's calls run
 * with newest_page_pending = 1 (the page is selected from the next step on);
 * or per layer, after the layer's newest key is written and before it is
 * scored, when they run with 0 (the page is selected in the same step).
 *   k_cache     : bf16 key cache of layer 0, strides `layout`; layer l
 *                 starts k_layer_stride bf16 elements further on.
 *   block_table : [batch][max_pages]; a block id outside [0, num_blocks)
 *                 is skipped.
 *   summaries   : layer 0's records, [Hkv][num_blocks][locks_summary_bytes];
 *                 layer l starts summ_layer_stride bytes further on.
 *   n_layers    : >= 1 (the strides are ignored when it is 1). */
locks_status locks_finalize_pages(const locks_dims* dims, const void* k_cache,
                                  locks_kv_layout layout, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t batch, void* summaries,
                                  int32_t n_layers, int64_t k_layer_stride,
                                  int64_t summ_layer_stride, void* stream);

/* Score every summarized page of every sequence from its summary alone
 * (sec. 2 reconstruction and selection, the equation for s_hat_j(q)):
 *   s_hat[b][h][j] = LSE_i ( (q_h.mu_j + (V_j^T q_h).c_i) / sqrt(d) ),
 * natural log, for query head h and every summarized logical page j (j <
 * seq_lens[b] / 16, or (seq_lens[b] - 1) / 16 with the newest page pending).
 *   q           : bf16 [batch][Hq][d].
 *   summaries   : this layer's records, [Hkv][num_blocks][locks_summary_bytes].
 *   block_table : [batch][max_pages] physical block of each logical page.
 *   seq_lens    : [batch] tokens per sequence.
 *   page_lse    : fp32 [batch][Hq][max_pages]; entries for pages that are not
 *                 summarized (or whose block id is out of range) get -inf.
 *   workspace   : >= locks_score_workspace_bytes(dims, batch, max_pages, 0).
 * No candidate key or value is read. */
locks_status locks_score_pages(const locks_dims* dims, const void* q, const void* summaries,
                               int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                               const int32_t* seq_lens, int32_t batch, float* page_lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Select pages from scores (sec. 2 group-shared selection): for each
 * (sequence, KV head) the mass share of page j for query head h is
 * exp(s_hat_hj - LSE_j' s_hat_hj'); shares are averaged over the G query
 * heads of the group and the k = min(budget_pages, summarized pages) largest
 * are kept (ties to the lower page index).
 *   page_lse  : fp32 [batch][Hq][max_pages] as written by locks_score_pages.
 *   sel       : int32 [batch][Hkv][budget_pages] logical page ids in
 *               ascending order, padded with -1.
 *   sel_count : int32 [batch][Hkv] number of valid entries of sel. */
locks_status locks_select_pages(const locks_dims* dims, const float* page_lse, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                int32_t* sel, int32_t* sel_count, void* workspace,
                                size_t workspace_bytes, void* stream);

/* locks_score_pages followed by locks_select_pages in one call (the decode
 * step's selection half).  page_lse is nullable: when NULL the scores live
 * in the workspace. */
locks_status locks_score_select(const locks_dims* dims, const void* q, const void* summaries,
                                int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                int32_t* sel, int32_t* sel_count, float* page_lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Attention of each query head over the selected pages' tokens plus the
 * tail page (the tokens past the summarized pages: the partial last page, or
 * with the newest page pending the page that holds the newest token), an
 * ordinary softmax renormalized over those tokens (abstract: attend only the
 * top pages).
 *   k_cache, v_cache : bf16 caches of this layer, strides `layout`.
 *   sel, sel_count   : as written by locks_select_pages; sel == NULL means
 *                      every summarized page (dense attention).
 *   budget_pages     : row length of sel (ignored when sel is NULL).
 *   softmax_scale    : logit scale, normally 1/sqrt(d).
 *   out              : bf16 [batch][Hq][d].
 *   out_lse          : nullable fp32 [batch][Hq], natural-log LSE of the
 *                      scaled logits over the attended tokens.
 *   workspace        : >= locks_attend_workspace_bytes(dims, batch, n) with
 *                      n = budget_pages + 1 (or max_pages + 1 when dense). */
locks_status locks_sparse_attend(const locks_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, locks_kv_layout layout, int32_t num_blocks,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, int32_t batch, const int32_t* sel,
                                 const int32_t* sel_count, int32_t budget_pages,
                                 float softmax_scale, void* out, float* out_lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Selection-table scope.  The pages average the mass shares of the query
 * heads that share a selection table, so that they all attend the same pages
 * (sec. 2 group-shared selection); the calls above take that table to be one
 * per (sequence, KV head), over its G query heads.  The *_tables variants let
 * one table serve several KV heads: n_tables tables per sequence, table t
 * covering KV heads [t*Hkv/n_tables, (t+1)*Hkv/n_tables) and all their query
 * heads.  n_tables = Hkv gives the calls above exactly; n_tables = 1 gives one
 * table for the whole layer (the other reading of the shared table).
 *   n_tables      : >= 1 and a divisor of Hkv; otherwise LOCKS_ERR_SHAPE.
 *   sel           : int32 [batch][n_tables][budget_pages], ascending, -1 padded.
 *   sel_count     : int32 [batch][n_tables].
 * Every other argument, buffer size and workspace is as for the call without
 * the suffix (the workspaces sized for Hkv tables serve any n_tables). */
locks_status locks_select_pages_tables(const locks_dims* dims, const float* page_lse,
                                       int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                       int32_t budget_pages, int32_t n_tables, int32_t* sel,
                                       int32_t* sel_count, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Attention of every KV head's query heads over its table's selection
 * (table kvh / (Hkv / n_tables)); sel == NULL means dense attention, as for
 * locks_sparse_attend, whose rules apply otherwise too. */
locks_status locks_sparse_attend_tables(const locks_dims* dims, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        locks_kv_layout layout, int32_t num_blocks,
                                        const int32_t* block_table, int32_t max_pages,
                                        const int32_t* seq_lens, int32_t batch,
                                        const int32_t* sel, const int32_t* sel_count,
                                        int32_t budget_pages, int32_t n_tables,
                                        float softmax_scale, void* out, float* out_lse,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* locks_decode_layer with n_tables selection tables per sequence; outputs
 * identical to locks_score_pages, locks_select_pages_tables and
 * locks_sparse_attend_tables in a row. */
locks_status locks_decode_layer_tables(const locks_dims* dims, const void* q,
                                       const void* summaries, const void* k_cache,
                                       const void* v_cache, locks_kv_layout layout,
                                       int32_t num_blocks, const int32_t* block_table,
                                       int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                       int32_t budget_pages, int32_t n_tables,
                                       float softmax_scale, int32_t* sel, int32_t* sel_count,
                                       void* out, float* out_lse, void* score_ws,
                                       size_t score_ws_bytes, void* attend_ws,
                                       size_t attend_ws_bytes, void* stream);

/* The shared low-rank basis the pages contrast LOCKS with (sec. 1 and sec. 3,
 * Proposition 1: one query-independent rank-r projection for every page is
 * blind to in-page directions outside it).  For each KV head: the pooled
 * scatter S = sum_j X_j^T X_j of the listed pages' deviations from their own
 * centroids, and its top-r eigenvectors (r = dims->rank).
 *   block_ids : [n_blocks] physical blocks pooled (ids outside
 *               [0, num_blocks) add nothing); n_blocks >= 1.
 *   basis     : fp32 [Hkv][r][128], row k = the k-th eigenvector (descending
 *               eigenvalue, ties to the lower index), unit length, largest-
 *               |entry| component positive (lowest index on ties).
 *   eigvals   : nullable fp32 [Hkv][128], all eigenvalues of S, descending.
 *   workspace : >= locks_shared_basis_workspace_bytes(dims, n_blocks) bytes,
 *               16-byte aligned.
 * Eigenvectors of (near-)equal eigenvalues are any orthonormal basis of their
 * span.  Off the decode path; a few milliseconds per call. */
size_t locks_shared_basis_workspace_bytes(const locks_dims* dims, int32_t n_blocks);
locks_status locks_shared_basis(const locks_dims* dims, const void* k_cache,
                                locks_kv_layout layout, const int32_t* block_ids,
                                int32_t n_blocks, int32_t num_blocks, float* basis,
                                float* eigvals, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Summaries in a given basis instead of each page's own eigenbasis: the
 * shared-basis selector at the same state size.  Each record keeps its
 * page's centroid and coefficients c_i = V^T x_i in the given basis, stored
 * and quantized exactly as locks_build_summaries stores its own (the record
 * layout above), so locks_score_pages and the rest read them unchanged.
 *   basis : fp32 [Hkv][r][128] (rows = basis vectors), e.g. from
 *           locks_shared_basis.
 * Other arguments and errors as for locks_build_summaries. */
locks_status locks_build_summaries_basis(const locks_dims* dims, const void* k_cache,
                                         locks_kv_layout layout, const int32_t* block_ids,
                                         int32_t n_blocks, int32_t num_blocks,
                                         const float* basis, void* summaries, void* stream);

/* Exact page scores from the true keys, the "read every key" comparator the
 * pages measure LOCKS against (sec. 3 contributions: selection quality
 * against exact page attention mass):
 *   page_lse[b][h][j] = LSE_i ( q_h . k_ij * softmax_scale ),
 * natural log, over the 16 tokens of each summarized logical page j.  The
 * output has the layout of locks_score_pages', so locks_select_pages turns it
 * into the exact top-k page set.  Reads every key of every summarized page.
 *   k_cache       : bf16 key cache of this layer, strides `layout`.
 *   softmax_scale : logit scale, normally 1/sqrt(d).
 *   page_lse      : fp32 [batch][Hq][max_pages]; pages that are not summarized
 *                   (or whose block id is out of range) get -inf.
 * Needs no workspace. */
locks_status locks_exact_page_lse(const locks_dims* dims, const void* q, const void* k_cache,
                                  locks_kv_layout layout, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t batch, float softmax_scale,
                                  float* page_lse, void* stream);

/* Human-readable name of a status code (static string, host). */
const char* locks_status_str(locks_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOCKS_H */
