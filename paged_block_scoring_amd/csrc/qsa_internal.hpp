// qsa_internal.hpp -- host-side interface between the C-ABI layer and the
// kernel launchers.  Not installed; the public contract is include/qsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

// Everything a kernel needs to locate the keys and rows of one call.
struct PagedArgs {
    const _Float16* q;          // [rows][4][128]
    const _Float16* kcache;     // [num_pages][kpp][128]
    const int32_t* page_table;  // [num_reqs][pt_stride]
    int64_t pt_stride;
    int32_t num_pages;
    int32_t num_reqs;
    const int32_t* row_req;     // [rows] or null (all request 0)
    const int32_t* pos;         // [rows]
    int32_t rows;
    int32_t kpp;                // keys per page = page_size / compress_ratio
    int32_t cr;
    int32_t max_visible;
    bool relu;
};

// Head sums of the query rows (default form) in the MFMA fragment order of
// the row-tiled scorer: qsum[((tile*4 + wave)*16 + t)*64 + lane] holds 8
// fp16 values, t = 2*slice + (0: hi, 1: lo); zero for rows past the end.
// After the fragments: one int32 per tile of 128 rows, the largest visible-key
// count of its rows (qsum_tile_visible); then one float per row slot of every
// tile, the row's head-sum factor f (qsa_device.hpp head_sum_factor; 1 for
// slots past the last row): a chain over the fragments gives score / f.
// The relu form computes no head sums: launch_qsum_prep then writes only, for
// calls with several requests, the largest visible-key count of each 64-row
// relu tile at the start of the buffer (and nothing for one request).
size_t qsum_bytes(int32_t rows);
const int32_t* qsum_tile_visible(const _Float16* qsum, int32_t rows);
const float* qsum_row_factor(const _Float16* qsum, int32_t rows);
hipError_t launch_qsum_prep(const PagedArgs& a, _Float16* qsum, hipStream_t stream);

// Candidate counters of the fused arm: row r's count is cand_count[r *
// kCountStride], one counter per 128-byte line, so that the atomics of
// different rows do not queue on one line.
constexpr int32_t kCountStride = 32;

// Which materialising scorer runs: chosen from the rows per request, or forced.
enum class ScorerChoice { Auto, Tiles, Groups };

// Scorer: writes scores[r*ld + j] for j < V_r.  qsum (default form) may be
// null, in which case the scorer forms the head sums itself.  `cus` is the
// device's compute-unit count.
hipError_t launch_score_paged(const PagedArgs& a, const _Float16* qsum, float* scores, int64_t ld, int32_t cus,
                              ScorerChoice choice, hipStream_t stream);

// Rows per window of the few-rows-per-request scorer: the rows per request
// rounded up to a power of two, at most 32 (8 in the relu form).
int32_t group_rows_for(int32_t rows, int32_t num_reqs, bool relu);

// Few-rows-per-request scorer (score_group.hip): same scores as the tiled one.
hipError_t launch_score_group(const PagedArgs& a, float* out, int64_t ld, int32_t cus, hipStream_t stream);

// Streaming arm (stream_select.hip): chunks of each row are scored and cut
// to their exact top-kb on chip (workspace: stream_bytes), then one
// workgroup per row merges them; out as qsa_select_paged_tokens.  `mark` is
// called between the two kernels.
size_t stream_bytes(int32_t rows, int32_t max_visible, int32_t kb);
hipError_t launch_stream_select(const PagedArgs& a, int32_t kb, int32_t expand, int32_t out_len, int32_t* out,
                                void* workspace, hipStream_t stream, hipError_t (*mark)(hipStream_t));

// Scorer over logical keys i (key stride*i): out[r*ld + i] for i < ceil(V_r/stride).
// With true_scores false the default form stores chain results (score / f of
// the row's head-sum factor f), the unit the filtering pass compares in.
hipError_t launch_score_store(const PagedArgs& a, const _Float16* qsum, int32_t stride, bool true_scores, float* out,
                              int64_t ld, int32_t cus, hipStream_t stream);

// Scorer that appends every composite >= thresh[r] to row r's candidate list
// (default form: composites of chain results, the sampling pass's unit).
hipError_t launch_score_filter(const PagedArgs& a, const _Float16* qsum, const uint64_t* thresh, uint64_t* cand,
                               int32_t* cand_count, int32_t cand_cap, int32_t cus, hipStream_t stream);

// Where a selector takes each row's candidate count from.
struct VisibleSource {
    const int32_t* visible;  // explicit counts, or
    const int32_t* pos;      // counts derived from positions (with row_req / cr), or neither: max_visible
    const int32_t* row_req;
    int32_t num_reqs;
    int32_t cr;
    int32_t max_visible;
};

// Exact top-kk per row over materialised scores; writes rank-ordered indices
// (expanded by `expand` consecutive tokens each when expand > 1) into
// out[r*out_len ...], padding with -1.
hipError_t launch_topk_rows(const float* scores, int64_t ld, const VisibleSource& vis, int32_t rows,
                            int32_t kk, int32_t expand, int32_t out_len, int32_t* out,
                            hipStream_t stream);

// Sizes of the fused arm for one call.
struct FusedPlan {
    int32_t stride;    // sampling stride
    int32_t m;         // rank of the sample composite used as threshold
    int32_t capl;      // LDS candidate capacity of the final kernel
    int32_t cand_cap;  // candidate list capacity per row
    int64_t ld_s;      // row stride of the sample scores
};
FusedPlan plan_fused(int32_t max_visible, int32_t kb);

// The fused arm's redo list (rows the final select's candidate pass leaves
// to its full pass): kRedoHead int32 (the count, alone on a 256-byte
// stretch), then one int32 per row.  The threshold kernel clears the count.
constexpr int32_t kRedoHead = 64;
inline size_t redo_bytes(int32_t rows) { return (size_t)(kRedoHead + rows) * sizeof(int32_t); }

hipError_t launch_sample_threshold(const float* samp, int64_t ld_s, const VisibleSource& vis, const FusedPlan& f,
                                   bool force_fallback, uint64_t* thresh, int32_t* cand_count, int32_t* redo,
                                   int32_t rows,
                                   hipStream_t stream);

hipError_t launch_fused_final(const PagedArgs& a, const VisibleSource& vis, const FusedPlan& f, const uint64_t* thresh,
                              const uint64_t* cand, const int32_t* cand_count, int32_t* redo, bool force_redo,
                              int32_t kb, int32_t expand,
                              int32_t out_len, int32_t* out, hipStream_t stream);

// Sparse attention over selected tokens (attend.hip): head_dim 256, at most
// 16 query heads per KV head; out fp32 [rows][q_heads][256].  With few rows
// each row's list is split over several workgroups whose partial results
// (attend_workspace_bytes of workspace) a second kernel merges.
size_t attend_workspace_bytes(int32_t rows, int32_t kv_heads, int32_t k);
hipError_t launch_attend(const _Float16* q, const _Float16* kc, const _Float16* vc, const int32_t* page_table,
                         int64_t pt_stride, int32_t num_pages, int32_t num_reqs, const int32_t* row_req,
                         const int32_t* tokens, int32_t k, int32_t rows, int32_t q_heads, int32_t kv_heads,
                         int32_t page_size, float scale, float* out, void* workspace, hipStream_t stream);

// Compressed-key producer (compress.hip): finishes the blocks that close in
// this call and stages the keys of blocks left open; `mark` is called on the
// stream before the first kernel and after each one.
hipError_t launch_compress(const _Float16* k_tok, const int32_t* tok_req, const int32_t* tok_pos, int32_t T,
                           const float* norm_w, float eps, int32_t rope_dim, double rope_base, bool interleaved,
                           _Float16* state, _Float16* kcache, const int32_t* page_table, int64_t pt_stride,
                           int32_t num_pages, int32_t num_reqs, int32_t page_size, int32_t cr, int32_t cus,
                           hipStream_t stream, hipError_t (*mark)(hipStream_t));

}  // namespace qsa
