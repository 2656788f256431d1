// score.hip -- launchers of the tiled scorers (score_rows.hpp for the default
// form, score_core.hpp for the relu form): the materialising scorer behind
// qsa_score_paged and the two-pass arm, the strided sampling pass and the
// filtering pass of the fused arm.
#include "qsa_internal.hpp"
#include "score_core.hpp"

namespace qsa {
namespace {

// The relu form scores q itself and leaves the head-sum buffer unused; with
// several requests its first bytes hold the visible-key count of each relu
// tile's longest row (relu_tile_visible_kernel).
int32_t* relu_tile_visible(const _Float16* qsum) { return reinterpret_cast<int32_t*>(const_cast<_Float16*>(qsum)); }

// Relu form: the tiled scorer of score_core.hpp.  Even shares of each XCD's
// (tile, key) positions, in whole stages: about the form's resident
// workgroups per compute unit, but no share below `min_seg` positions.  With
// several requests and the tile counts in the head-sum buffer, the kernel
// shares only the keys each tile can see (the grid stays the same).
template <Epi EPI>
hipError_t launch_relu(ScoreKernelArgs A, int32_t cus, int64_t min_seg, hipStream_t stream) {
    constexpr int64_t g = ReluForm::STEP;
    A.tiles = (A.a.rows + ReluForm::TILE - 1) / ReluForm::TILE;
    const int64_t stripe = ((int64_t)(A.lmax + kXcds - 1) / kXcds + g - 1) / g * g;
    A.xcd_keys = (int32_t)stripe;
    const int64_t positions = (int64_t)A.tiles * stripe;
    // (positions are counted in 32 bits, as in the default form's kernel)
    A.tile_v = A.qsum && A.a.num_reqs > 1 && positions + (int64_t)A.tiles * g < (1ll << 31)
                   ? relu_tile_visible(A.qsum)
                   : nullptr;
    int64_t per_xcd = (int64_t)(cus / kXcds > 0 ? cus / kXcds : 1) * ReluForm::WG_PER_CU;
    int64_t seg = ((positions + per_xcd - 1) / per_xcd + g - 1) / g * g;
    if (seg < min_seg) seg = (min_seg + g - 1) / g * g;
    per_xcd = (positions + seg - 1) / seg;
    A.seg_len = seg;
    score_tiles_kernel<EPI><<<dim3((unsigned)(kXcds * per_xcd)), ScoreShape::NT, 0, stream>>>(A);
    return hipGetLastError();
}

// The row-tiled scorer's grid: even whole-stage shares of each XCD's
// (tile, key) positions, two workgroups per compute unit, no share below
// min_seg positions.
struct RowsSplit {
    int32_t tiles;
    int64_t stripe, positions, seg, per_xcd;
};

RowsSplit rows_split(int32_t rows, int32_t lmax, int32_t cus, int64_t min_seg) {
    constexpr int64_t g = RowsShape::STEP;
    RowsSplit r;
    r.tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    r.stripe = ((int64_t)(lmax + kXcds - 1) / kXcds + g - 1) / g * g;
    r.positions = (int64_t)r.tiles * r.stripe;
    const int64_t per = (int64_t)(cus / kXcds > 0 ? cus / kXcds : 1) * 2;
    r.seg = ((r.positions + per - 1) / per + g - 1) / g * g;
    if (r.seg < min_seg) r.seg = (min_seg + g - 1) / g * g;
    r.per_xcd = (r.positions + r.seg - 1) / r.seg;
    return r;
}

// Default form: the row-tiled scorer of score_rows.hpp, same share rule.
template <Epi EPI>
hipError_t launch_rows(const ScoreKernelArgs& K, int32_t cus, int64_t min_seg, hipStream_t stream) {
    constexpr int64_t g = RowsShape::STEP;
    RowsArgs A = {};
    A.a = K.a;
    A.qsum = K.qsum;
    A.qfac = qsum_row_factor(K.qsum, K.a.rows);
    A.true_scores = K.true_scores;
    A.stride = K.stride;
    A.lmax = K.lmax;
    A.out = K.out;
    A.ld = K.ld;
    A.vec_store = K.vec_store;
    A.thresh = K.thresh;
    A.cand = K.cand;
    A.cand_count = K.cand_count;
    A.cand_cap = K.cand_cap;
    const RowsSplit sp = rows_split(A.a.rows, A.lmax, cus, min_seg);
    A.tiles = sp.tiles;
    A.tile_v = qsum_tile_visible(K.qsum, A.a.rows);
    A.kpp_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == A.a.kpp) A.kpp_shift = sh;
    A.xcd_keys = (int32_t)sp.stripe;
    // The balanced mapping pays a scan of the tile counts in every workgroup;
    // one request's tiles (a prefill chunk) see about the same keys, so there
    // the plain split is as even.  It counts positions in 32 bits.
    if (A.a.num_reqs <= 1 || sp.positions + (int64_t)A.tiles * g >= (1ll << 31)) A.tile_v = nullptr;
    A.seg_len = sp.seg;
    score_rows_kernel<EPI><<<dim3((unsigned)(kXcds * sp.per_xcd)), RowsShape::NT, 0, stream>>>(A);
    return hipGetLastError();
}

template <Epi EPI>
hipError_t launch_epi(const ScoreKernelArgs& A, int32_t cus, hipStream_t stream) {
    if (A.a.relu) return launch_relu<EPI>(A, cus, 64, stream);
    return launch_rows<EPI>(A, cus, 64, stream);
}

}  // namespace

hipError_t launch_score_store(const PagedArgs& a, const _Float16* qsum, int32_t stride, bool true_scores, float* out,
                              int64_t ld, int32_t cus, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    ScoreKernelArgs A = {};
    A.a = a;
    A.qsum = qsum;
    A.stride = stride;
    A.lmax = (a.max_visible + stride - 1) / stride;
    A.out = out;
    A.ld = ld;
    A.vec_store = (ld % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
    A.true_scores = true_scores ? 1 : 0;
    return launch_epi<Epi::Store>(A, cus, stream);
}

// The tiled scorer shares each staged key among a tile's rows; with fewer than
// 32 rows per request on average those rows mostly belong to different
// requests, and the windowed scorer, which streams every key once per window,
// takes over.
static bool use_group_scorer(const PagedArgs& a, ScorerChoice choice) {
    if (choice != ScorerChoice::Auto) return choice == ScorerChoice::Groups;
    const int32_t reqs = a.num_reqs > 0 ? a.num_reqs : 1;
    return a.rows / reqs < 32;
}

hipError_t launch_score_paged(const PagedArgs& a, const _Float16* qsum, float* scores, int64_t ld, int32_t cus,
                              ScorerChoice choice, hipStream_t stream) {
    if (use_group_scorer(a, choice)) return launch_score_group(a, scores, ld, cus, stream);
    // Default form: the head sums are prepared once per call, unless the
    // scorer's grid holds at most 8 workgroups per tile; those then fold their
    // tile's head sums themselves (the same arithmetic) for less than the
    // preparation's launch (64 rows x 256 keys: 17.6 -> 15.9 us per call; with
    // 128 workgroups per tile the folds cost more, 36.0 -> 38.5 us).
    if (qsum && !a.relu) {
        const RowsSplit sp = rows_split(a.rows, a.max_visible, cus, 64);
        if (sp.per_xcd * kXcds <= 8 * (int64_t)sp.tiles) qsum = nullptr;
    }
    if (qsum) {
        const hipError_t e = launch_qsum_prep(a, const_cast<_Float16*>(qsum), stream);
        if (e != hipSuccess) return e;
    }
    return launch_score_store(a, qsum, 1, true, scores, ld, cus, stream);
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

// One workgroup per (tile, wave) of the fragment order, i.e. 32 query rows,
// with one wave per slice s: lane l handles dims 16s + 8g .. 16s + 8g + 7 (g =
// l/32) of row l%32 and stores their fp32 head sums as fp16 hi/lo pairs
// (head_sum_split, the same arithmetic as the scorers' own) at steps t = 2s
// and 2s + 1.  The row's head-sum factor comes from the largest |u| over its
// 16 (slice, half) parts, met in LDS; the slice-0 wave also stores it.  The
// last `tiles` workgroups instead write each tile's visible-key count (the
// largest over its rows; 0 for rows past the end or of an unknown request),
// which the tiled scorer uses to share out only the keys a tile can see.
constexpr int kPrepNT = 64 * kSlices;

__global__ __launch_bounds__(kPrepNT) void qsum_prep_kernel(PagedArgs a, _Float16* __restrict__ qsum,
                                                            int32_t frag_blocks, int32_t* __restrict__ tile_v,
                                                            float* __restrict__ row_f) {
    const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
    if ((int)blockIdx.x >= frag_blocks) {
        __shared__ int32_t s_w[kSlices];
        const int t = blockIdx.x - frag_blocks;
        const int row = t * RowsShape::TILE + threadIdx.x;
        int v = 0;
        if (threadIdx.x < RowsShape::TILE && row < a.rows) {
            const int req = a.row_req ? a.row_req[row] : 0;
            if (req >= 0 && req < a.num_reqs) v = visible_keys(a.pos[row], a.cr, a.max_visible);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
        if (lane == 0) s_w[s] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            int m = 0;
#pragma unroll
            for (int i = 0; i < kSlices; ++i) m = max(m, s_w[i]);
            tile_v[t] = m;
        }
        return;
    }
    __shared__ float s_um[kSlices][64];
    const int tw = blockIdx.x;  // tile * 4 + wave of the fragment order
    const int row = tw * RowsShape::RPW + (lane & 31);
    const bool live = row < a.rows;
    const _Float16* qr = a.q + (int64_t)(live ? row : 0) * kHeads * kHeadDim + 16 * s + 8 * (lane >> 5);
    half8 h[kHeads];
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh) {
        const half8 v = *reinterpret_cast<const half8*>(qr + hh * kHeadDim);
        h[hh] = live ? v : half8{};
    }
    s_um[s][lane] = head_sum_absmax(h[0], h[1], h[2], h[3]);
    __syncthreads();
    float um = 0.0f;
#pragma unroll
    for (int i = 0; i < kSlices; ++i) um = fmaxf(um, fmaxf(s_um[i][lane & 31], s_um[i][(lane & 31) + 32]));
    const float f = head_sum_factor(um);
    half8 hi, lo;
    head_sum_split(h[0], h[1], h[2], h[3], 1.0f / f, hi, lo);
    half8* out = reinterpret_cast<half8*>(qsum) + (int64_t)tw * 16 * 64 + lane;
    out[64 * (2 * s)] = hi;
    out[64 * (2 * s + 1)] = lo;
    if (s == 0 && lane < 32) row_f[tw * RowsShape::RPW + lane] = f;
}

// fragments of every tile, then one visible-key count per tile, then one
// head-sum factor per row slot of every tile
static size_t qsum_frag_bytes(int32_t rows) {
    const int64_t tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    return (size_t)tiles * RowsShape::WAVES * 16 * 64 * sizeof(half8);
}

static size_t qsum_tile_v_bytes(int32_t rows) {
    const int64_t tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    return (size_t)((tiles * sizeof(int32_t) + 255) / 256 * 256);
}

size_t qsum_bytes(int32_t rows) {
    const int64_t tiles = (rows + RowsShape::TILE - 1) / RowsShape::TILE;
    return qsum_frag_bytes(rows) + qsum_tile_v_bytes(rows) +
           (size_t)((tiles * RowsShape::TILE * sizeof(float) + 255) / 256 * 256);
}

const int32_t* qsum_tile_visible(const _Float16* qsum, int32_t rows) {
    return qsum ? reinterpret_cast<const int32_t*>(reinterpret_cast<const unsigned char*>(qsum) + qsum_frag_bytes(rows))
                : nullptr;
}

const float* qsum_row_factor(const _Float16* qsum, int32_t rows) {
    return qsum ? reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(qsum) +
                                                 qsum_frag_bytes(rows) + qsum_tile_v_bytes(rows))
                : nullptr;
}

// Relu form, several requests: the visible-key count of each relu tile's
// longest row (0 for rows past the end or of an unknown request), one wave
// per tile.
__global__ __launch_bounds__(64) void relu_tile_visible_kernel(PagedArgs a, int32_t* __restrict__ tile_v) {
    static_assert(ReluForm::TILE == 64, "one row per lane");
    const int row = blockIdx.x * ReluForm::TILE + threadIdx.x;
    int v = 0;
    if (row < a.rows) {
        const int req = a.row_req ? a.row_req[row] : 0;
        if (req >= 0 && req < a.num_reqs) v = visible_keys(a.pos[row], a.cr, a.max_visible);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    if (threadIdx.x == 0) tile_v[blockIdx.x] = v;
}

hipError_t launch_qsum_prep(const PagedArgs& a, _Float16* qsum, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    if (a.relu) {
        if (a.num_reqs <= 1) return hipSuccess;
        const int64_t tiles = (a.rows + ReluForm::TILE - 1) / ReluForm::TILE;
        relu_tile_visible_kernel<<<dim3((unsigned)tiles), 64, 0, stream>>>(a, relu_tile_visible(qsum));
        return hipGetLastError();
    }
    const int64_t tiles = (a.rows + RowsShape::TILE - 1) / RowsShape::TILE;
    int32_t* tile_v = const_cast<int32_t*>(qsum_tile_visible(qsum, a.rows));
    float* row_f = const_cast<float*>(qsum_row_factor(qsum, a.rows));
    const int32_t frag_blocks = (int32_t)(tiles * RowsShape::WAVES);
    qsum_prep_kernel<<<dim3((unsigned)(frag_blocks + tiles)), kPrepNT, 0, stream>>>(a, qsum, frag_blocks, tile_v,
                                                                                    row_f);
    return hipGetLastError();
}

}  // namespace qsa
