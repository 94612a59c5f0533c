// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace locks {

// ---- summary records ----------------------------------------------------------
// A rank-r record holds 84r + 130 bytes of fields (basis codes, coefficient
// codes, centroid codes, fp16 scales), padded to a multiple of 64 bytes.
constexpr int rec_bytes(int r) { return (84 * r + 130 + 63) / 64 * 64; }
constexpr bool rank_supported(int r) { return r == 4 || r == 8 || r == 16; }
// raw_debug floats per page-head: mu [128], V [r][128], C [16][r]
constexpr int raw_floats(int r) { return 128 + 144 * r; }

// ---- scoring ---------------------------------------------------------------
constexpr int32_t kScoreSteps = 4;     // 4-page steps per scoring wave
struct ScorePlan {
  int32_t n_chunks;          // workgroups per (sequence, KV head); one partial each
};
ScorePlan plan_score(int32_t batch, int32_t hkv, int32_t max_pages);

hipError_t launch_score(int32_t rank, const uint16_t* q, const uint8_t* summ, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
                        int32_t batch, int32_t hq, int32_t hkv, int32_t pending, float scale,
                        float* page_lse, float2* partials, const ScorePlan& plan,
                        hipStream_t stream);

// ---- selection -------------------------------------------------------------
constexpr int32_t kSelChunk = 2048;   // pages per first-stage select workgroup (at least)
struct SelectPlan {
  int32_t chunk_pages;  // kSelChunk, or twice it when the grid is large
  int32_t n_chunks;     // first-stage chunks per (sequence, table)
  int32_t slots;        // candidates kept per chunk = min(budget, chunk_pages)
};
// groups: the most (sequence, table) pairs a call may select for (batch * Hkv)
SelectPlan plan_select(int32_t max_pages, int32_t budget_pages, int64_t groups);

// Per-head (max, sum) base-2 partials straight from page scores.
hipError_t launch_lse_partials(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                               int32_t batch, int32_t hq, int32_t pending, float2* partials,
                               int32_t n_chunks, int32_t pages_per_chunk, hipStream_t stream);

// Selection runs per (sequence, table): `ntab` tables per sequence, each over
// hq / ntab query heads (ntab = hkv: one table per KV head).  `pending` = 1:
// the page holding each sequence's newest token is not summarized (every
// kernel of the path reads the page count the same way).
//
// Stage 1 only: every chunk's candidates (page order); each chunk workgroup
// merges the per-head (max, sum) partials into the normalizers it needs.
hipError_t launch_select_stage1(const float* page_lse, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t ntab,
                                int32_t pending, int32_t budget_pages, const float2* partials,
                                int32_t n_partials, uint32_t* cand_key,
                                int32_t* cand_idx, const SelectPlan& plan, hipStream_t stream);

hipError_t launch_select(const float* page_lse, int32_t max_pages, const int32_t* seq_lens,
                         int32_t batch, int32_t hq, int32_t ntab, int32_t pending,
                         int32_t budget_pages, const float2* partials, int32_t n_partials,
                         uint32_t* cand_key, int32_t* cand_idx, const SelectPlan& plan,
                         int32_t* sel, int32_t* sel_count, hipStream_t stream);

// ---- sparse attention ---------------------------------------------------------
struct AttendPlan {
  int32_t pages_per_split;  // 8 .. 8192; a split is one workgroup of 4 waves
  int32_t n_splits;         // splits per (sequence, KV head)
};
AttendPlan plan_attend(int32_t batch, int32_t hkv, int32_t max_attended);

hipError_t launch_attend(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         int64_t block_stride, int64_t head_stride, int64_t token_stride,
                         int32_t num_blocks, const int32_t* block_table, int32_t max_pages,
                         const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                         int32_t ntab, int32_t pending, const int32_t* sel,
                         const int32_t* sel_count, int32_t budget_pages, float scale,
                         float* part_o, float2* part_ml, const AttendPlan& plan, uint16_t* out,
                         float* out_lse, hipStream_t stream);

// Final selection stage fused with the attention (candidates from stage 1).
constexpr int32_t kFusedMaxBudget = 1024;
bool fused_select_attend_fits(int32_t n_cand, int32_t budget_pages);
hipError_t launch_select_attend(const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, int64_t block_stride,
                                int64_t head_stride, int64_t token_stride, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_pages,
                                const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                                int32_t ntab, int32_t pending, const uint32_t* cand_key,
                                const int32_t* cand_idx, const SelectPlan& sp, int32_t* sel,
                                int32_t* sel_count, int32_t budget_pages, float scale,
                                float* part_o, float2* part_ml, const AttendPlan& plan,
                                uint16_t* out, float* out_lse, hipStream_t stream);

// ---- shared basis (the rejected baseline, for comparison) ------------------------
constexpr int32_t kSharedMaxChunks = 64;   // partial 128x128 sums per KV head
struct SharedPlan {
  int32_t n_chunks;    // partial sums per KV head
  int32_t per_chunk;   // pages per partial
};
SharedPlan plan_shared(int32_t n_blocks);
// partials: float [hkv][n_chunks][128][128]; basis: float [hkv][8][128];
// eigvals: nullable float [hkv][128], descending.
// basis: float [hkv][rank][128] (the top-rank eigenvectors).
hipError_t launch_shared_basis(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                               int64_t head_stride, int64_t token_stride,
                               const int32_t* block_ids, int32_t n_blocks, int32_t num_blocks,
                               int32_t hkv, float* partials, const SharedPlan& plan,
                               float* basis, float* eigvals, hipStream_t stream);
// Summaries in a given basis (float [hkv][rank][128], rows = basis vectors).
hipError_t launch_build_basis(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                              int64_t head_stride, int64_t token_stride,
                              const int32_t* block_ids, int32_t n_blocks, int32_t num_blocks,
                              int32_t hkv, const float* basis, uint8_t* summaries,
                              hipStream_t stream);

// ---- exact page LSE (read-every-key comparator) ---------------------------------
hipError_t launch_exact_lse(const uint16_t* q, const uint16_t* k_cache, int64_t block_stride,
                            int64_t head_stride, int64_t token_stride, int32_t num_blocks,
                            const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, int32_t batch, int32_t hq, int32_t hkv,
                            int32_t pending, float scale, float* page_lse, hipStream_t stream);

// ---- summary build -----------------------------------------------------------
hipError_t launch_build(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                        int64_t head_stride, int64_t token_stride, const int32_t* block_ids,
                        int32_t n_blocks, int32_t num_blocks, int32_t hkv, uint8_t* summaries,
                        float* raw_debug, hipStream_t stream);

// Incremental finalization: summarize, for every sequence whose length is a
// positive multiple of the page size, its last full page (decided on the device).
hipError_t launch_finalize(int32_t rank, const uint16_t* k_cache, int64_t block_stride,
                           int64_t head_stride, int64_t token_stride, const int32_t* block_table,
                           int32_t max_pages,
                           const int32_t* seq_lens, int32_t batch, int32_t num_blocks,
                           int32_t hkv, uint8_t* summaries, int32_t n_layers,
                           int64_t k_layer_stride, int64_t summ_layer_stride,
                           hipStream_t stream);

}  // namespace locks
