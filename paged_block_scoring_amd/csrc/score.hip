// score.hip -- launchers of the tiled scorers (score_rows.hpp for the default
// form, score_core.hpp for the relu form): the materialising scorer behind
// qsa_score_paged and the two-pass arm, the strided sampling pass and the
// filtering pass of the fused arm.
#include <stdlib.h>
#include <string.h>

#include "qsa_internal.hpp"
#include "score_core.hpp"

namespace qsa {
namespace {

// Relu form: the tiled scorer of score_core.hpp.  Even shares of each XCD's
// (tile, key) positions, in whole stages: about the form's resident
// workgroups per compute unit, but no share below `min_seg` positions.
template <Epi EPI>
hipError_t launch_relu(ScoreKernelArgs A, int32_t cus, int64_t min_seg, hipStream_t stream) {
    constexpr int64_t g = ReluForm::STEP;
    A.tiles = (A.a.rows + ReluForm::TILE - 1) / ReluForm::TILE;
    const int64_t stripe = ((int64_t)(A.lmax + kXcds - 1) / kXcds + g - 1) / g * g;
    A.xcd_keys = (int32_t)stripe;
    const int64_t positions = (int64_t)A.tiles * stripe;
    int64_t per_xcd = (int64_t)(cus / kXcds > 0 ? cus / kXcds : 1) * ReluForm::WG_PER_CU;
    int64_t seg = ((positions + per_xcd - 1) / per_xcd + g - 1) / g * g;
    if (seg < min_seg) seg = (min_seg + g - 1) / g * g;
    per_xcd = (positions + seg - 1) / seg;
    A.seg_len = seg;
    score_tiles_kernel<EPI><<<dim3((unsigned)(kXcds * per_xcd)), ScoreShape::NT, 0, stream>>>(A);
    return hipGetLastError();
}

// Default form: the row-tiled scorer of score_rows.hpp, same share rule.
template <Epi EPI>
hipError_t launch_rows(const ScoreKernelArgs& K, int32_t cus, int64_t min_seg, hipStream_t stream) {
    constexpr int64_t g = RowsShape::STEP;
    RowsArgs A = {};
    A.a = K.a;
    A.qsum = K.qsum;
    A.stride = K.stride;
    A.lmax = K.lmax;
    A.out = K.out;
    A.ld = K.ld;
    A.vec_store = K.vec_store;
    A.thresh = K.thresh;
    A.cand = K.cand;
    A.cand_count = K.cand_count;
    A.cand_cap = K.cand_cap;
    A.tiles = (A.a.rows + RowsShape::TILE - 1) / RowsShape::TILE;
    A.tile_v = qsum_tile_visible(K.qsum, A.a.rows);
    A.kpp_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == A.a.kpp) A.kpp_shift = sh;
    const int64_t stripe = ((int64_t)(A.lmax + kXcds - 1) / kXcds + g - 1) / g * g;
    A.xcd_keys = (int32_t)stripe;
    const int64_t positions = (int64_t)A.tiles * stripe;
    // The balanced mapping pays a scan of the tile counts in every workgroup;
    // one request's tiles (a prefill chunk) see about the same keys, so there
    // the plain split is as even.  It counts positions in 32 bits.
    if (A.a.num_reqs <= 1 || positions + (int64_t)A.tiles * g >= (1ll << 31)) A.tile_v = nullptr;
    int64_t per_xcd = (int64_t)(cus / kXcds > 0 ? cus / kXcds : 1) * 2;
    int64_t seg = ((positions + per_xcd - 1) / per_xcd + g - 1) / g * g;
    if (seg < min_seg) seg = (min_seg + g - 1) / g * g;
    per_xcd = (positions + seg - 1) / seg;
    A.seg_len = seg;
    score_rows_kernel<EPI><<<dim3((unsigned)(kXcds * per_xcd)), RowsShape::NT, 0, stream>>>(A);
    return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_epi(const ScoreKernelArgs& A, int32_t cus, hipStream_t stream) {
    if (A.a.relu) return launch_relu<EPI>(A, cus, 64, stream);
    return launch_rows<EPI>(A, cus, 64, stream);
}

}  // namespace

hipError_t launch_score_store(const PagedArgs& a, const _Float16* qsum, int32_t stride, float* out, int64_t ld,
                              int32_t cus, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    ScoreKernelArgs A = {};
    A.a = a;
    A.qsum = qsum;
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

hipError_t launch_score_paged(const PagedArgs& a, const _Float16* qsum, float* scores, int64_t ld,
                              hipStream_t stream) {
    if (use_group_scorer(a)) return launch_score_group(a, scores, ld, stream);
    if (qsum && !a.relu) {
        const hipError_t e = launch_qsum_prep(a, const_cast<_Float16*>(qsum), stream);
        if (e != hipSuccess) return e;
    }
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return launch_score_store(a, qsum, 1, scores, ld, cus, stream);
}

hipError_t launch_score_filter(const PagedArgs& a, const _Float16* qsum, const uint64_t* thresh, uint64_t* cand,
                               int32_t* cand_count, int32_t cand_cap, int32_t cus, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    ScoreKernelArgs A = {};
    A.a = a;
    A.qsum = qsum;
    A.stride = 1;
    A.lmax = a.max_visible;
    A.thresh = thresh;
    A.cand = cand;
    A.cand_count = cand_count;
    A.cand_cap = cand_cap;
    return launch_epi<Epi::Filter>(A, cus, stream);
}

// One thread per (tile, wave, slice, lane): the fp32 head sum of the 8 query
// dims that lane supplies for that slice, as its fp16 hi/lo pair
// (head_sum_split, the same arithmetic as the scorers' own), stored at steps
// t = 2*slice and 2*slice + 1 of the fragment order.  The last `tiles`
// workgroups instead write each tile's visible-key count (the largest over
// its rows; 0 for rows past the end or of an unknown request), which the
// tiled scorer uses to share out only the keys a tile can see.
__global__ __launch_bounds__(256) void qsum_prep_kernel(PagedArgs a, _Float16* __restrict__ qsum, int32_t n,
                                                        int32_t frag_blocks, int32_t* __restrict__ tile_v) {
    if ((int)blockIdx.x >= frag_blocks) {
        __shared__ int32_t s_w[4];
        const int t = blockIdx.x - frag_blocks;
        const int row = t * RowsShape::TILE + threadIdx.x;
        int v = 0;
        if (threadIdx.x < RowsShape::TILE && row < a.rows) {
            const int req = a.row_req ? a.row_req[row] : 0;
            if (req >= 0 && req < a.num_reqs) v = visible_keys(a.pos[row], a.cr, a.max_visible);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
        if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
        __syncthreads();
        if (threadIdx.x == 0) tile_v[t] = max(max(s_w[0], s_w[1]), max(s_w[2], s_w[3]));
        return;
    }
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int lane = i & 63, s = (i >> 6) & 7, wave = (i >> 9) & 3, tile = i >> 11;
    const int row = tile * RowsShape::TILE + wave * RowsShape::RPW + (lane & 31);
    half8 hi = {}, lo = {};
    if (row < a.rows) {
        const _Float16* qr = a.q + (int64_t)row * kHeads * kHeadDim + 16 * s + 8 * (lane >> 5);
        head_sum_split(*reinterpret_cast<const half8*>(qr), *reinterpret_cast<const half8*>(qr + kHeadDim),
                       *reinterpret_cast<const half8*>(qr + 2 * kHeadDim),
                       *reinterpret_cast<const half8*>(qr + 3 * kHeadDim), hi, lo);
    }
    half8* out = reinterpret_cast<half8*>(qsum) + ((int64_t)tile * RowsShape::WAVES + wave) * 16 * 64 + lane;
    out[64 * (2 * s)] = hi;
    out[64 * (2 * s + 1)] = lo;
}

// fragments of every tile, then one visible-key count per tile
static size_t qsum_frag_bytes(int32_t rows) {
    const int64_t tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    return (size_t)tiles * RowsShape::WAVES * 16 * 64 * sizeof(half8);
}

size_t qsum_bytes(int32_t rows) {
    const int64_t tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    return qsum_frag_bytes(rows) + (size_t)((tiles * sizeof(int32_t) + 255) / 256 * 256);
}

const int32_t* qsum_tile_visible(const _Float16* qsum, int32_t rows) {
    return qsum ? reinterpret_cast<const int32_t*>(reinterpret_cast<const unsigned char*>(qsum) + qsum_frag_bytes(rows))
                : nullptr;
}

hipError_t launch_qsum_prep(const PagedArgs& a, _Float16* qsum, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t tiles = (a.rows + RowsShape::TILE - 1) / RowsShape::TILE;
    const int32_t n = (int32_t)(tiles * RowsShape::WAVES * kSlices * 64);
    const int32_t frag_blocks = (n + 255) / 256;
    int32_t* tile_v = const_cast<int32_t*>(qsum_tile_visible(qsum, a.rows));
    qsum_prep_kernel<<<dim3((unsigned)(frag_blocks + tiles)), 256, 0, stream>>>(a, qsum, n, frag_blocks, tile_v);
    return hipGetLastError();
}

}  // namespace qsa
