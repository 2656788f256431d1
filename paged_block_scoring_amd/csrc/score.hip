// score.hip -- launchers of the tiled scoring kernel (score_core.hpp): the
// materialising scorer behind qsa_score_paged and the two-pass arm, the
// strided sampling pass and the filtering pass of the fused arm.
#include <stdlib.h>
#include <string.h>

#include "qsa_internal.hpp"
#include "score_core.hpp"

namespace qsa {
namespace {

// Even shares of each XCD's (tile, key) positions, in whole stages: about
// the form's resident workgroups per compute unit, but no share below
// `min_seg` positions.
template <bool RELU, Epi EPI>
hipError_t launch_form(ScoreKernelArgs A, int32_t cus, int64_t min_seg, hipStream_t stream) {
    constexpr int64_t g = Stage<RELU>::STEP;
    A.tiles = (A.a.rows + Form<RELU>::TILE - 1) / Form<RELU>::TILE;
    const int64_t stripe = ((int64_t)(A.lmax + kXcds - 1) / kXcds + g - 1) / g * g;
    A.xcd_keys = (int32_t)stripe;
    const int64_t positions = (int64_t)A.tiles * stripe;
    int64_t per_xcd = (int64_t)(cus / kXcds > 0 ? cus / kXcds : 1) * Form<RELU>::WG_PER_CU;
    int64_t seg = ((positions + per_xcd - 1) / per_xcd + g - 1) / g * g;
    if (seg < min_seg) seg = (min_seg + g - 1) / g * g;
    per_xcd = (positions + seg - 1) / seg;
    A.seg_len = seg;
    score_tiles_kernel<RELU, EPI><<<dim3((unsigned)(kXcds * per_xcd)), ScoreShape::NT, 0, stream>>>(A);
    return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_epi(const ScoreKernelArgs& A, int32_t cus, hipStream_t stream) {
    if (A.a.relu) return launch_form<true, EPI>(A, cus, 64, stream);
    return launch_form<false, EPI>(A, cus, 64, stream);
}

}  // namespace

hipError_t launch_score_store(const PagedArgs& a, int32_t stride, float* out, int64_t ld, int32_t cus,
                              hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    ScoreKernelArgs A = {};
    A.a = a;
    A.stride = stride;
    A.lmax = (a.max_visible + stride - 1) / stride;
    A.out = out;
    A.ld = ld;
    A.vec_store = (ld % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
    return launch_epi<Epi::Store>(A, cus, stream);
}

// The tiled scorer shares each staged key among a tile's rows; with fewer than
// 32 rows per request on average those rows mostly belong to different
// requests, and the windowed scorer, which streams every key once per window,
// takes over.
static bool use_group_scorer(const PagedArgs& a) {
    const char* f = getenv("QSA_FORCE_SCORER");
    if (f && strcmp(f, "tiles") == 0) return false;
    if (f && strcmp(f, "groups") == 0) return true;
    const int32_t reqs = a.num_reqs > 0 ? a.num_reqs : 1;
    return a.rows / reqs < 32;
}

hipError_t launch_score_paged(const PagedArgs& a, float* scores, int64_t ld, hipStream_t stream) {
    if (use_group_scorer(a)) return launch_score_group(a, scores, ld, stream);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return launch_score_store(a, 1, scores, ld, cus, stream);
}

hipError_t launch_score_filter(const PagedArgs& a, const uint64_t* thresh, uint64_t* cand, int32_t* cand_count,
                               int32_t cand_cap, int32_t cus, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    ScoreKernelArgs A = {};
    A.a = a;
    A.stride = 1;
    A.lmax = a.max_visible;
    A.thresh = thresh;
    A.cand = cand;
    A.cand_count = cand_count;
    A.cand_cap = cand_cap;
    return launch_epi<Epi::Filter>(A, cus, stream);
}

}  // namespace qsa
