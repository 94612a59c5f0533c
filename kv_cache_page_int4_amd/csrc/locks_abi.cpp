// C ABI entry points: host-side validation, workspace carving, launches.
// Nothing here allocates, synchronizes or touches device memory from the host.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/locks.h"
#include "locks_internal.h"

using namespace locks;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Alignment the kernels' accesses need: 16 bytes for bf16 tensors read in
// 16-byte pieces, summaries and workspaces, 4 bytes for int32 / fp32 arrays
// and the bf16 output (written two values at a time).  NULL counts as
// aligned: presence is checked separately.
inline bool misaligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}

locks_status check_dims(const locks_dims* d) {
  if (!d) return LOCKS_ERR_NULL;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return LOCKS_ERR_SHAPE;
  if (d->head_dim != 128 || d->page_size != 16 || !rank_supported(d->rank))
    return LOCKS_ERR_UNSUPPORTED;
  // GQA: every KV head serves G = Hq / Hkv query heads, G in {1, 2, 4, 8}
  if (d->num_q_heads % d->num_kv_heads) return LOCKS_ERR_UNSUPPORTED;
  const int32_t g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return LOCKS_ERR_UNSUPPORTED;
  if (d->newest_page_pending != 0 && d->newest_page_pending != 1) return LOCKS_ERR_SHAPE;
  return LOCKS_OK;
}

// Logit scale the pages' estimate uses: 1 / sqrt(d).
constexpr float kDefaultScale = 0.08838834764831845f;

// The page grid is indexed with 32-bit integers on the device.
constexpr int64_t kMaxPages = (int64_t)1 << 26;

struct ScoreWs {
  size_t lse_off, part_off, key_off, idx_off, total;
  ScorePlan sp;
  SelectPlan sel;
};

ScoreWs score_ws_layout(const locks_dims* d, int32_t batch, int32_t max_pages, int32_t budget,
                        bool need_lse) {
  ScoreWs w{};
  w.sp = plan_score(batch, d->num_kv_heads, max_pages);
  w.sel = plan_select(max_pages, budget > 0 ? budget : 1, (int64_t)batch * d->num_kv_heads);
  size_t off = 0;
  w.lse_off = off;
  if (need_lse) off += align_up((size_t)batch * d->num_q_heads * max_pages * sizeof(float));
  w.part_off = off;
  // partials serve the scorer's chunking and the standalone-select chunking
  const int32_t n_part = w.sp.n_chunks > w.sel.n_chunks ? w.sp.n_chunks : w.sel.n_chunks;
  off += align_up((size_t)batch * d->num_q_heads * n_part * sizeof(float2));
  const size_t ncand = (size_t)batch * d->num_kv_heads * w.sel.n_chunks * w.sel.slots;
  w.key_off = off;
  off += align_up(ncand * sizeof(uint32_t));
  w.idx_off = off;
  off += align_up(ncand * sizeof(int32_t));
  w.total = off;
  return w;
}

struct AttendWs {
  size_t o_off, ml_off, total;
  AttendPlan ap;
};

AttendWs attend_ws_layout(const locks_dims* d, int32_t batch, int32_t max_attended) {
  AttendWs w{};
  w.ap = plan_attend(batch, d->num_kv_heads, max_attended);
  const size_t rows = (size_t)batch * d->num_q_heads * w.ap.n_splits;
  w.o_off = 0;
  w.ml_off = align_up(rows * 128 * sizeof(float));
  w.total = w.ml_off + align_up(rows * sizeof(float2));
  return w;
}

inline char* ws_at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

}  // namespace

extern "C" {

size_t locks_summary_bytes(const locks_dims* dims) {
  return check_dims(dims) == LOCKS_OK ? (size_t)rec_bytes(dims->rank) : 0;
}

size_t locks_score_workspace_bytes(const locks_dims* dims, int32_t batch, int32_t max_pages,
                                   int32_t budget_pages) {
  if (check_dims(dims) != LOCKS_OK || batch <= 0 || max_pages <= 0 || max_pages > kMaxPages)
    return 0;
  return score_ws_layout(dims, batch, max_pages, budget_pages, true).total;
}

size_t locks_attend_workspace_bytes(const locks_dims* dims, int32_t batch,
                                    int32_t max_attended_pages) {
  if (check_dims(dims) != LOCKS_OK || batch <= 0 || max_attended_pages <= 0) return 0;
  return attend_ws_layout(dims, batch, max_attended_pages).total;
}

size_t locks_workspace_bytes(const locks_dims* dims, int32_t batch, int32_t max_pages,
                             int32_t budget_pages) {
  if (check_dims(dims) != LOCKS_OK || batch <= 0 || max_pages <= 0 || max_pages > kMaxPages ||
      budget_pages <= 0)
    return 0;
  // the scoring / selection part first, then room for the attention
  // partials of a sparse or a dense pass
  const size_t score = align_up(score_ws_layout(dims, batch, max_pages, budget_pages, true).total);
  const int32_t att = (budget_pages > max_pages ? budget_pages : max_pages) + 1;
  return score + attend_ws_layout(dims, batch, att).total;
}

locks_status locks_build_summaries(const locks_dims* dims, const void* k_cache,
                                   locks_kv_layout layout, const int32_t* block_ids,
                                   int32_t n_blocks, int32_t num_blocks, void* summaries,
                                   float* raw_debug, void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (n_blocks < 0 || num_blocks <= 0) return LOCKS_ERR_SHAPE;
  if (n_blocks == 0) return LOCKS_OK;
  if (!k_cache || !block_ids || !summaries) return LOCKS_ERR_NULL;
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(k_cache, 16) || misaligned(summaries, 16) || misaligned(block_ids, 4) ||
      misaligned(raw_debug, 4))
    return LOCKS_ERR_SHAPE;
  hipError_t e = launch_build(dims->rank, static_cast<const uint16_t*>(k_cache), layout.block_stride,
                              layout.head_stride, layout.token_stride, block_ids, n_blocks,
                              num_blocks, dims->num_kv_heads, static_cast<uint8_t*>(summaries),
                              raw_debug, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

static locks_status score_checks(const locks_dims* dims, const void* q, const void* summaries,
                                 int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, int32_t batch) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (!q || !summaries || !block_table || !seq_lens) return LOCKS_ERR_NULL;
  if (batch <= 0 || max_pages <= 0 || max_pages > kMaxPages || num_blocks <= 0)
    return LOCKS_ERR_SHAPE;
  if (misaligned(q, 16) || misaligned(summaries, 16) || misaligned(block_table, 4) ||
      misaligned(seq_lens, 4))
    return LOCKS_ERR_SHAPE;
  if (batch > 65535 || dims->num_kv_heads > 65535) return LOCKS_ERR_SHAPE;
  return LOCKS_OK;
}

locks_status locks_score_pages(const locks_dims* dims, const void* q, const void* summaries,
                               int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                               const int32_t* seq_lens, int32_t batch, float* page_lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  locks_status st = score_checks(dims, q, summaries, num_blocks, block_table, max_pages, seq_lens, batch);
  if (st != LOCKS_OK) return st;
  if (!page_lse) return LOCKS_ERR_NULL;
  if (misaligned(page_lse, 4)) return LOCKS_ERR_SHAPE;
  const ScoreWs w = score_ws_layout(dims, batch, max_pages, 0, true);
  if (!workspace || workspace_bytes < w.total || misaligned(workspace, 16))
    return LOCKS_ERR_WORKSPACE;
  hipError_t e = launch_score(dims->rank, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(summaries),
                              num_blocks, block_table, max_pages, seq_lens, batch,
                              dims->num_q_heads, dims->num_kv_heads, dims->newest_page_pending,
                              kDefaultScale, page_lse,
                              reinterpret_cast<float2*>(ws_at(workspace, w.part_off)), w.sp,
                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

static locks_status select_pages_impl(const locks_dims* dims, const float* page_lse,
                                      int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                      int32_t budget_pages, int32_t n_tables, int32_t* sel,
                                      int32_t* sel_count, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (n_tables <= 0 || dims->num_kv_heads % n_tables) return LOCKS_ERR_SHAPE;
  if (!page_lse || !seq_lens || !sel || !sel_count) return LOCKS_ERR_NULL;
  if (batch <= 0 || max_pages <= 0 || max_pages > kMaxPages || budget_pages <= 0)
    return LOCKS_ERR_SHAPE;
  if (misaligned(page_lse, 4) || misaligned(seq_lens, 4) || misaligned(sel, 4) ||
      misaligned(sel_count, 4))
    return LOCKS_ERR_SHAPE;
  const ScoreWs w = score_ws_layout(dims, batch, max_pages, budget_pages, true);
  if (!workspace || workspace_bytes < w.total || misaligned(workspace, 16))
    return LOCKS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float2* part = reinterpret_cast<float2*>(ws_at(workspace, w.part_off));
  const int32_t pend = dims->newest_page_pending;
  hipError_t e = launch_lse_partials(page_lse, max_pages, seq_lens, batch, dims->num_q_heads, pend,
                                     part, w.sel.n_chunks, w.sel.chunk_pages, s);
  if (e == hipSuccess)
    e = launch_select(page_lse, max_pages, seq_lens, batch, dims->num_q_heads, n_tables, pend,
                      budget_pages, part, w.sel.n_chunks,
                      reinterpret_cast<uint32_t*>(ws_at(workspace, w.key_off)),
                      reinterpret_cast<int32_t*>(ws_at(workspace, w.idx_off)), w.sel, sel,
                      sel_count, s);
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

locks_status locks_select_pages(const locks_dims* dims, const float* page_lse, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                int32_t* sel, int32_t* sel_count, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return select_pages_impl(dims, page_lse, max_pages, seq_lens, batch, budget_pages,
                           dims ? dims->num_kv_heads : 0, sel, sel_count, workspace,
                           workspace_bytes, stream);
}

locks_status locks_select_pages_tables(const locks_dims* dims, const float* page_lse,
                                       int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                       int32_t budget_pages, int32_t n_tables, int32_t* sel,
                                       int32_t* sel_count, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return select_pages_impl(dims, page_lse, max_pages, seq_lens, batch, budget_pages, n_tables,
                           sel, sel_count, workspace, workspace_bytes, stream);
}

locks_status locks_score_select(const locks_dims* dims, const void* q, const void* summaries,
                                int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                int32_t* sel, int32_t* sel_count, float* page_lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  locks_status st = score_checks(dims, q, summaries, num_blocks, block_table, max_pages, seq_lens, batch);
  if (st != LOCKS_OK) return st;
  if (!sel || !sel_count) return LOCKS_ERR_NULL;
  if (budget_pages <= 0) return LOCKS_ERR_SHAPE;
  if (misaligned(sel, 4) || misaligned(sel_count, 4) || misaligned(page_lse, 4))
    return LOCKS_ERR_SHAPE;
  const ScoreWs w = score_ws_layout(dims, batch, max_pages, budget_pages, true);
  if (!workspace || workspace_bytes < w.total || misaligned(workspace, 16))
    return LOCKS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* lse = page_lse ? page_lse : reinterpret_cast<float*>(ws_at(workspace, w.lse_off));
  float2* part = reinterpret_cast<float2*>(ws_at(workspace, w.part_off));
  hipError_t e = launch_score(dims->rank, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(summaries),
                              num_blocks, block_table, max_pages, seq_lens, batch,
                              dims->num_q_heads, dims->num_kv_heads, dims->newest_page_pending,
                              kDefaultScale, lse, part, w.sp, s);
  if (e == hipSuccess)
    e = launch_select(lse, max_pages, seq_lens, batch, dims->num_q_heads, dims->num_kv_heads,
                      dims->newest_page_pending, budget_pages, part, w.sp.n_chunks,
                      reinterpret_cast<uint32_t*>(ws_at(workspace, w.key_off)),
                      reinterpret_cast<int32_t*>(ws_at(workspace, w.idx_off)), w.sel, sel,
                      sel_count, s);
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

static locks_status decode_layer_impl(const locks_dims* dims, const void* q,
                                      const void* summaries, const void* k_cache,
                                      const void* v_cache, locks_kv_layout layout,
                                      int32_t num_blocks, const int32_t* block_table,
                                      int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                      int32_t budget_pages, int32_t n_tables, float softmax_scale,
                                      int32_t* sel, int32_t* sel_count, void* out, float* out_lse,
                                      void* score_ws, size_t score_ws_bytes, void* attend_ws,
                                      size_t attend_ws_bytes, void* stream) {
  locks_status st = score_checks(dims, q, summaries, num_blocks, block_table, max_pages, seq_lens, batch);
  if (st != LOCKS_OK) return st;
  if (n_tables <= 0 || dims->num_kv_heads % n_tables) return LOCKS_ERR_SHAPE;
  if (!k_cache || !v_cache || !sel || !sel_count || !out) return LOCKS_ERR_NULL;
  if (budget_pages <= 0) return LOCKS_ERR_SHAPE;
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(sel, 4) ||
      misaligned(sel_count, 4) || misaligned(out, 4) || misaligned(out_lse, 4))
    return LOCKS_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale != softmax_scale) return LOCKS_ERR_SHAPE;
  const ScoreWs w = score_ws_layout(dims, batch, max_pages, budget_pages, true);
  const AttendWs a = attend_ws_layout(dims, batch, budget_pages + 1);
  if (!score_ws || misaligned(score_ws, 16) || misaligned(attend_ws, 16))
    return LOCKS_ERR_WORKSPACE;
  if (attend_ws) {
    if (score_ws_bytes < w.total || attend_ws_bytes < a.total) return LOCKS_ERR_WORKSPACE;
  } else {
    // one workspace: the attention part follows the scoring part
    if (score_ws_bytes < align_up(w.total) + a.total) return LOCKS_ERR_WORKSPACE;
    attend_ws = ws_at(score_ws, align_up(w.total));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* lse = reinterpret_cast<float*>(ws_at(score_ws, w.lse_off));
  float2* part = reinterpret_cast<float2*>(ws_at(score_ws, w.part_off));
  uint32_t* ck = reinterpret_cast<uint32_t*>(ws_at(score_ws, w.key_off));
  int32_t* ci = reinterpret_cast<int32_t*>(ws_at(score_ws, w.idx_off));
  float* po = reinterpret_cast<float*>(ws_at(attend_ws, a.o_off));
  float2* pml = reinterpret_cast<float2*>(ws_at(attend_ws, a.ml_off));
  const int hq = dims->num_q_heads, hkv = dims->num_kv_heads;
  const int32_t pend = dims->newest_page_pending;
  // pages are scored at the temperature they are attended with
  hipError_t e = launch_score(dims->rank, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(summaries),
                              num_blocks, block_table, max_pages, seq_lens, batch, hq, hkv, pend,
                              softmax_scale, lse, part, w.sp, s);
  if (e != hipSuccess) return LOCKS_ERR_LAUNCH;
  const int32_t n_cand = w.sel.n_chunks * w.sel.slots;
  if (fused_select_attend_fits(n_cand, budget_pages)) {
    e = launch_select_stage1(lse, max_pages, seq_lens, batch, hq, n_tables, pend, budget_pages,
                             part, w.sp.n_chunks, ck, ci, w.sel, s);
    if (e == hipSuccess)
      e = launch_select_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                               static_cast<const uint16_t*>(v_cache), layout.block_stride,
                               layout.head_stride, layout.token_stride, num_blocks, block_table,
                               max_pages, seq_lens, batch, hq, hkv, n_tables, pend, ck, ci, w.sel,
                               sel, sel_count, budget_pages, softmax_scale, po, pml, a.ap,
                               static_cast<uint16_t*>(out), out_lse, s);
  } else {
    e = launch_select(lse, max_pages, seq_lens, batch, hq, n_tables, pend, budget_pages, part,
                      w.sp.n_chunks, ck, ci, w.sel, sel, sel_count, s);
    if (e == hipSuccess)
      e = launch_attend(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                        static_cast<const uint16_t*>(v_cache), layout.block_stride,
                        layout.head_stride, layout.token_stride, num_blocks, block_table,
                        max_pages, seq_lens, batch, hq, hkv, n_tables, pend, sel, sel_count,
                        budget_pages, softmax_scale, po, pml, a.ap, static_cast<uint16_t*>(out),
                        out_lse, s);
  }
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

locks_status locks_decode_layer(const locks_dims* dims, const void* q, const void* summaries,
                                const void* k_cache, const void* v_cache, locks_kv_layout layout,
                                int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t budget_pages,
                                float softmax_scale, int32_t* sel, int32_t* sel_count, void* out,
                                float* out_lse, void* score_ws, size_t score_ws_bytes,
                                void* attend_ws, size_t attend_ws_bytes, void* stream) {
  return decode_layer_impl(dims, q, summaries, k_cache, v_cache, layout, num_blocks, block_table,
                           max_pages, seq_lens, batch, budget_pages, dims ? dims->num_kv_heads : 0,
                           softmax_scale, sel, sel_count, out, out_lse, score_ws, score_ws_bytes,
                           attend_ws, attend_ws_bytes, stream);
}

locks_status locks_decode_layer_tables(const locks_dims* dims, const void* q,
                                       const void* summaries, const void* k_cache,
                                       const void* v_cache, locks_kv_layout layout,
                                       int32_t num_blocks, const int32_t* block_table,
                                       int32_t max_pages, const int32_t* seq_lens, int32_t batch,
                                       int32_t budget_pages, int32_t n_tables,
                                       float softmax_scale, int32_t* sel, int32_t* sel_count,
                                       void* out, float* out_lse, void* score_ws,
                                       size_t score_ws_bytes, void* attend_ws,
                                       size_t attend_ws_bytes, void* stream) {
  return decode_layer_impl(dims, q, summaries, k_cache, v_cache, layout, num_blocks, block_table,
                           max_pages, seq_lens, batch, budget_pages, n_tables, softmax_scale, sel,
                           sel_count, out, out_lse, score_ws, score_ws_bytes, attend_ws,
                           attend_ws_bytes, stream);
}

// ---- the decode layer without workspaces ------------------------------------
// A file-scope device array stands in for the two workspaces.  Its name in
// host code is only a host-side stand-in, never a device address: the device
// address comes from hipGetSymbolAddress, once per device (each GPU holds its
// own copy of the array), and only that address reaches the kernels.
}  // extern "C"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // LOCKS_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == LOCKS_NOALLOC_SCRATCH_BYTES, "header and library agree");
__device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use).
locks_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOCKS_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return LOCKS_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LOCKS_OK;
}

}  // namespace

extern "C" {

size_t locks_decode_layer_noalloc_bytes(const locks_dims* dims, int32_t batch, int32_t max_pages,
                                        int32_t budget_pages) {
  if (check_dims(dims) != LOCKS_OK || batch <= 0 || max_pages <= 0 || max_pages > kMaxPages ||
      budget_pages <= 0)
    return 0;
  return align_up(score_ws_layout(dims, batch, max_pages, budget_pages, true).total) +
         attend_ws_layout(dims, batch, budget_pages + 1).total;
}

locks_status locks_decode_layer_noalloc(const locks_dims* dims, const void* q,
                                        const void* summaries, const void* k_cache,
                                        const void* v_cache, locks_kv_layout layout,
                                        int32_t num_blocks, const int32_t* block_table,
                                        int32_t max_pages, const int32_t* seq_lens,
                                        int32_t batch, int32_t budget_pages, float softmax_scale,
                                        int32_t* sel, int32_t* sel_count, void* out,
                                        float* out_lse, void* stream) {
  const size_t need = locks_decode_layer_noalloc_bytes(dims, batch, max_pages, budget_pages);
  if (need == 0) {
    // the shape itself is invalid: report why, as the workspace call would
    locks_status st = check_dims(dims);
    return st != LOCKS_OK ? st : LOCKS_ERR_SHAPE;
  }
  if (need > kScratchBytes) return LOCKS_ERR_WORKSPACE;
  void* ws = nullptr;
  locks_status st = scratch_address(&ws);
  if (st != LOCKS_OK) return st;
  return decode_layer_impl(dims, q, summaries, k_cache, v_cache, layout, num_blocks, block_table,
                           max_pages, seq_lens, batch, budget_pages, dims->num_kv_heads,
                           softmax_scale, sel, sel_count, out, out_lse, ws, kScratchBytes, nullptr,
                           0, stream);
}

locks_status locks_finalize_pages(const locks_dims* dims, const void* k_cache,
                                  locks_kv_layout layout, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t batch, void* summaries,
                                  int32_t n_layers, int64_t k_layer_stride,
                                  int64_t summ_layer_stride, void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (!k_cache || !block_table || !seq_lens || !summaries) return LOCKS_ERR_NULL;
  if (batch <= 0 || batch > 65535 || max_pages <= 0 || max_pages > kMaxPages || num_blocks <= 0)
    return LOCKS_ERR_SHAPE;
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(k_cache, 16) || misaligned(summaries, 16) || misaligned(block_table, 4) ||
      misaligned(seq_lens, 4))
    return LOCKS_ERR_SHAPE;
  if (n_layers <= 0 || n_layers > 65535 || (n_layers > 1 && (k_layer_stride <= 0 ||
      summ_layer_stride <= 0 || (k_layer_stride % 8) || (summ_layer_stride % 16))))
    return LOCKS_ERR_SHAPE;
  hipError_t e = launch_finalize(dims->rank, static_cast<const uint16_t*>(k_cache), layout.block_stride,
                                 layout.head_stride, layout.token_stride, block_table, max_pages,
                                 seq_lens, batch, num_blocks, dims->num_kv_heads,
                                 static_cast<uint8_t*>(summaries), n_layers, k_layer_stride,
                                 summ_layer_stride, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

locks_status locks_exact_page_lse(const locks_dims* dims, const void* q, const void* k_cache,
                                  locks_kv_layout layout, int32_t num_blocks,
                                  const int32_t* block_table, int32_t max_pages,
                                  const int32_t* seq_lens, int32_t batch, float softmax_scale,
                                  float* page_lse, void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (!q || !k_cache || !block_table || !seq_lens || !page_lse) return LOCKS_ERR_NULL;
  if (batch <= 0 || batch > 65535 || max_pages <= 0 || max_pages > kMaxPages || num_blocks <= 0)
    return LOCKS_ERR_SHAPE;
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(block_table, 4) ||
      misaligned(seq_lens, 4) || misaligned(page_lse, 4))
    return LOCKS_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale != softmax_scale) return LOCKS_ERR_SHAPE;
  hipError_t e = launch_exact_lse(static_cast<const uint16_t*>(q),
                                  static_cast<const uint16_t*>(k_cache), layout.block_stride,
                                  layout.head_stride, layout.token_stride, num_blocks, block_table,
                                  max_pages, seq_lens, batch, dims->num_q_heads,
                                  dims->num_kv_heads, dims->newest_page_pending, softmax_scale,
                                  page_lse,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

static locks_status sparse_attend_impl(const locks_dims* dims, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       locks_kv_layout layout, int32_t num_blocks,
                                       const int32_t* block_table, int32_t max_pages,
                                       const int32_t* seq_lens, int32_t batch, const int32_t* sel,
                                       const int32_t* sel_count, int32_t budget_pages,
                                       int32_t n_tables, float softmax_scale, void* out,
                                       float* out_lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (n_tables <= 0 || dims->num_kv_heads % n_tables) return LOCKS_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return LOCKS_ERR_NULL;
  if (sel && !sel_count) return LOCKS_ERR_NULL;
  if (batch <= 0 || batch > 65535 || max_pages <= 0 || max_pages > kMaxPages || num_blocks <= 0)
    return LOCKS_ERR_SHAPE;
  if (sel && budget_pages <= 0) return LOCKS_ERR_SHAPE;
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) ||
      misaligned(block_table, 4) || misaligned(seq_lens, 4) || misaligned(sel, 4) ||
      misaligned(sel_count, 4) || misaligned(out, 4) || misaligned(out_lse, 4))
    return LOCKS_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale != softmax_scale) return LOCKS_ERR_SHAPE;
  const int32_t max_att = (sel ? budget_pages : max_pages) + 1;
  const AttendWs w = attend_ws_layout(dims, batch, max_att);
  if (!workspace || workspace_bytes < w.total || misaligned(workspace, 16))
    return LOCKS_ERR_WORKSPACE;
  hipError_t e = launch_attend(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
      static_cast<const uint16_t*>(v_cache), layout.block_stride, layout.head_stride,
      layout.token_stride, num_blocks, block_table, max_pages, seq_lens, batch, dims->num_q_heads,
      dims->num_kv_heads, n_tables, dims->newest_page_pending, sel, sel_count, budget_pages,
      softmax_scale, reinterpret_cast<float*>(ws_at(workspace, w.o_off)),
      reinterpret_cast<float2*>(ws_at(workspace, w.ml_off)), w.ap, static_cast<uint16_t*>(out),
      out_lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

locks_status locks_sparse_attend(const locks_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, locks_kv_layout layout, int32_t num_blocks,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, int32_t batch, const int32_t* sel,
                                 const int32_t* sel_count, int32_t budget_pages,
                                 float softmax_scale, void* out, float* out_lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attend_impl(dims, q, k_cache, v_cache, layout, num_blocks, block_table, max_pages,
                            seq_lens, batch, sel, sel_count, budget_pages,
                            dims ? dims->num_kv_heads : 0, softmax_scale, out, out_lse, workspace,
                            workspace_bytes, stream);
}

locks_status locks_sparse_attend_tables(const locks_dims* dims, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        locks_kv_layout layout, int32_t num_blocks,
                                        const int32_t* block_table, int32_t max_pages,
                                        const int32_t* seq_lens, int32_t batch,
                                        const int32_t* sel, const int32_t* sel_count,
                                        int32_t budget_pages, int32_t n_tables,
                                        float softmax_scale, void* out, float* out_lse,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attend_impl(dims, q, k_cache, v_cache, layout, num_blocks, block_table, max_pages,
                            seq_lens, batch, sel, sel_count, budget_pages, n_tables,
                            softmax_scale, out, out_lse, workspace, workspace_bytes, stream);
}

size_t locks_shared_basis_workspace_bytes(const locks_dims* dims, int32_t n_blocks) {
  if (check_dims(dims) != LOCKS_OK || n_blocks <= 0) return 0;
  const SharedPlan pl = plan_shared(n_blocks);
  return align_up((size_t)dims->num_kv_heads * pl.n_chunks * 128 * 128 * sizeof(float));
}

static locks_status kv_layout_checks(const void* k_cache, locks_kv_layout layout) {
  if (layout.token_stride < 128 || layout.block_stride <= 0 || layout.head_stride <= 0 ||
      (layout.token_stride % 8) || (layout.head_stride % 8) || (layout.block_stride % 8))
    return LOCKS_ERR_SHAPE;
  if (misaligned(k_cache, 16)) return LOCKS_ERR_SHAPE;
  return LOCKS_OK;
}

locks_status locks_shared_basis(const locks_dims* dims, const void* k_cache,
                                locks_kv_layout layout, const int32_t* block_ids,
                                int32_t n_blocks, int32_t num_blocks, float* basis,
                                float* eigvals, void* workspace, size_t workspace_bytes,
                                void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (!k_cache || !block_ids || !basis) return LOCKS_ERR_NULL;
  if (n_blocks <= 0 || num_blocks <= 0 || dims->num_kv_heads > 65535) return LOCKS_ERR_SHAPE;
  st = kv_layout_checks(k_cache, layout);
  if (st != LOCKS_OK) return st;
  if (misaligned(basis, 4) || misaligned(eigvals, 4) || misaligned(block_ids, 4))
    return LOCKS_ERR_SHAPE;
  const SharedPlan pl = plan_shared(n_blocks);
  const size_t need = locks_shared_basis_workspace_bytes(dims, n_blocks);
  if (!workspace || workspace_bytes < need || misaligned(workspace, 16))
    return LOCKS_ERR_WORKSPACE;
  hipError_t e = launch_shared_basis(dims->rank, static_cast<const uint16_t*>(k_cache),
                                     layout.block_stride,
                                     layout.head_stride, layout.token_stride, block_ids, n_blocks,
                                     num_blocks, dims->num_kv_heads,
                                     static_cast<float*>(workspace), pl, basis, eigvals,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

locks_status locks_build_summaries_basis(const locks_dims* dims, const void* k_cache,
                                         locks_kv_layout layout, const int32_t* block_ids,
                                         int32_t n_blocks, int32_t num_blocks,
                                         const float* basis, void* summaries, void* stream) {
  locks_status st = check_dims(dims);
  if (st != LOCKS_OK) return st;
  if (n_blocks < 0 || num_blocks <= 0 || dims->num_kv_heads > 65535) return LOCKS_ERR_SHAPE;
  if (n_blocks == 0) return LOCKS_OK;
  if (!k_cache || !block_ids || !basis || !summaries) return LOCKS_ERR_NULL;
  st = kv_layout_checks(k_cache, layout);
  if (st != LOCKS_OK) return st;
  if (misaligned(summaries, 16) || misaligned(basis, 4) || misaligned(block_ids, 4))
    return LOCKS_ERR_SHAPE;
  hipError_t e = launch_build_basis(dims->rank, static_cast<const uint16_t*>(k_cache),
                                    layout.block_stride,
                                    layout.head_stride, layout.token_stride, block_ids, n_blocks,
                                    num_blocks, dims->num_kv_heads, basis,
                                    static_cast<uint8_t*>(summaries),
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOCKS_OK : LOCKS_ERR_LAUNCH;
}

const char* locks_status_str(locks_status status) {
  switch (status) {
    case LOCKS_OK: return "ok";
    case LOCKS_ERR_NULL: return "required pointer is NULL";
    case LOCKS_ERR_SHAPE: return "size, stride or alignment out of range";
    case LOCKS_ERR_UNSUPPORTED:
      return "unsupported dims (need head_dim 128, page 16, rank 4/8/16, Hq/Hkv in {1,2,4,8})";
    case LOCKS_ERR_WORKSPACE: return "workspace missing or too small";
    case LOCKS_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
