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

// Scorer: writes scores[r*ld + j] for j < V_r.
hipError_t launch_score_paged(const PagedArgs& a, float* scores, int64_t ld, hipStream_t stream);

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

}  // namespace qsa
