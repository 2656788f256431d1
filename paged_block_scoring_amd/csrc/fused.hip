// fused.hip -- the fused arm of qsa_select_paged_tokens: exact lexicographic
// top-k without materialising the score matrix.
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", section "Purpose" (exact selector, deterministic ties) and "Test
// Plan" (top-k 2,048 tokens); "qwen4_exp QSA cooperative_topk cannot launch on
// NVIDIA Thor (sm_110): cluster misconfiguration", section "What happens" (the
// two-stage score-then-top-k structure this arm replaces).
//
// Every (row, key) has a distinct composite c = (order key of the score,
// inverted key index); the selected blocks are the row's kb largest
// composites.  The arm runs in four steps:
//  1. sampling pass: the scorer materialises the scores of every stride-th
//     key (logical sample i is key stride*i);
//  2. threshold: per row, fT = the score of the m-th largest sample
//     composite, with m sized so that comfortably more than kb keys of the
//     whole row are expected to score >= fT; a row with fewer than m samples
//     gets a threshold no score reaches;
//  3. filtering pass: the scorer keeps every key with score >= fT in the
//     row's candidate list (staged in LDS, one global atomic per row and
//     piece);
//  4. final select: if the row has at least min(kb, V) and at most cap
//     candidates they contain its exact top-kb (kb scores >= fT force the
//     kb-th largest score to be >= fT, so every member of the top-kb passed
//     the filter), which a radix select over composites and a bitonic sort in
//     LDS turn into rank order.  Otherwise the workgroup recomputes the row's
//     scores itself with the same MFMA sequence and keeps an exact running
//     top-kb in LDS.  Either way the result is exact; the sample only decides
//     how fast.
#include <algorithm>
#include <cmath>

#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_select.hpp"

namespace qsa {
namespace {

__device__ __forceinline__ int row_visible_count(const VisibleSource& v, int r) {
    if (v.visible) return min(max(v.visible[r], 0), v.max_visible);
    if (v.pos) {
        const int req = v.row_req ? v.row_req[r] : 0;
        if (req < 0 || req >= v.num_reqs) return 0;
        return visible_keys(v.pos[r], v.cr, v.max_visible);
    }
    return v.max_visible;
}

constexpr int kThrNT = 256;
constexpr int kMaxSamples = 4096;

// Threshold of one row: the samples are binned linearly by value between
// their minimum and maximum (the bin index is monotone in the value); T is
// the smallest sample of the bin holding the m-th largest, so at least m
// samples are >= T.  Stored as a composite whose high word is T's order key.
__global__ __launch_bounds__(kThrNT) void sample_threshold_kernel(const float* __restrict__ samp, int64_t ld_s,
                                                                  VisibleSource vis, int32_t stride, int32_t m,
                                                                  int32_t force_fallback,
                                                                  uint64_t* __restrict__ thresh,
                                                                  int32_t* __restrict__ cand_count,
                                                                  int32_t* __restrict__ redo_count) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && redo_count) *redo_count = 0;  // (for the split select)
    constexpr int EPT = kMaxSamples / kThrNT;
    __shared__ HistScratch hs;
    __shared__ float s_f[2 * (kThrNT / 64)];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int V = row_visible_count(vis, row);
    const int ns = (V + stride - 1) / stride;
    uint64_t T = ~0ull;  // decodes to a NaN threshold score: nothing passes
    if (ns >= m && !force_fallback) {
        const float* srow = samp + (int64_t)row * ld_s;
        float x[EPT];
        float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
        // every load is issued before any is used: indices past the row's
        // samples are clamped into its stride (ld_s >= ns) and masked after
#pragma unroll
        for (int e = 0; e < EPT; ++e) x[e] = srow[min(e * kThrNT + (int)threadIdx.x, (int)ld_s - 1)];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = e * kThrNT + (int)threadIdx.x < ns;
            lo = in ? fminf(lo, x[e]) : lo;
            hi = in ? fmaxf(hi, x[e]) : hi;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, o, 64));
            hi = fmaxf(hi, __shfl_xor(hi, o, 64));
        }
        if (lane == 0) {
            s_f[wave] = lo;
            s_f[kThrNT / 64 + wave] = hi;
        }
        for (int i = threadIdx.x; i < kSelBins; i += kThrNT) hs.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kThrNT / 64; ++w) {
            lo = fminf(lo, s_f[w]);
            hi = fmaxf(hi, s_f[kThrNT / 64 + w]);
        }
        float t = lo;
        const float scale = (float)kSelBins / (hi - lo);
        if (hi > lo && scale < __builtin_huge_valf()) {  // (block-uniform)
            auto bin = [&](float v) { return min((int)((v - lo) * scale), kSelBins - 1); };
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (e * kThrNT < ns && e * kThrNT + (int)threadIdx.x < ns) atomicAdd(&hs.hist[bin(x[e])], 1u);
            __syncthreads();
            // thread u owns bins kSelBins-1-BPT*u .. (high to low); find the bin of the m-th largest
            constexpr int BPT = kSelBins / kThrNT;
            uint32_t c[BPT];
            int local = 0;
#pragma unroll
            for (int j = 0; j < BPT; ++j) {
                c[j] = hs.hist[kSelBins - 1 - BPT * (int)threadIdx.x - j];
                local += (int)c[j];
            }
            int tot;
            int run = block_inclusive_scan<kThrNT>(local, hs.wsum, &tot) - local;
#pragma unroll
            for (int j = 0; j < BPT; ++j) {
                if (run < m && run + (int)c[j] >= m) hs.bin = kSelBins - 1 - BPT * (int)threadIdx.x - j;
                run += (int)c[j];
            }
            __syncthreads();
            const int b = hs.bin;
            float tm = __builtin_huge_valf();
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (e * kThrNT < ns && e * kThrNT + (int)threadIdx.x < ns && bin(x[e]) == b) tm = fminf(tm, x[e]);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) tm = fminf(tm, __shfl_xor(tm, o, 64));
            if (lane == 0) s_f[wave] = tm;
            __syncthreads();
            t = s_f[0];
#pragma unroll
            for (int w = 1; w < kThrNT / 64; ++w) t = fminf(t, s_f[w]);
        }
        T = (uint64_t)order_key(t) << 32;
    }
    if (threadIdx.x == 0) {
        thresh[row] = T;
        cand_count[(int64_t)row * kCountStride] = 0;
    }
}

struct FinalArgs {
    PagedArgs a;
    VisibleSource vis;
    const uint64_t* cand;
    const int32_t* cand_count;
    const uint64_t* thresh;  // [rows] the filter's threshold composites (high word: order key of the score)
    int32_t cand_cap;
    int32_t kb;
    int32_t expand;
    int32_t out_len;
    int32_t* out;
    int32_t* redo_count;  // split select: rows the candidate pass left to the full pass (count, then rows)
    int32_t* redo_rows;
    int32_t force_redo;   // the candidate pass leaves every row to the full pass (debug override)
};

constexpr int kFinNT = 256;
constexpr int kRedoGrid = 256;  // workgroups of the split select's second pass
constexpr int kFinWaves = kFinNT / 64;

// Exact top-kb of one row by recomputation: each wave scores 32 keys at a
// time straight from the cache with the same MFMA sequences as the tiled
// scorer, with zero query fragments outside the row (default form: keys as
// MFMA rows, the row's head sum as column 0; relu form: the row's four heads
// as MFMA rows 0..3, keys as columns).  Composites above the running cutoff are appended in
// LDS, and the buffer is cut back to its kb largest whenever it exceeds kb.
// Leaves the selected composites (unsorted) in a[0 .. return value).
template <int CAPL>
__device__ int recompute_row_topk(const FinalArgs& A, int row, int V, uint64_t* a, KthScratch* ks, int* s_pend,
                                  float* s_rs) {
    const PagedArgs& p = A.a;
    const int kb = A.kb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ch = (CAPL - kb) / (32 * kFinWaves) * (32 * kFinWaves);
    const int req = p.row_req ? p.row_req[row] : 0;
    const int32_t* ptrow = p.page_table + (int64_t)req * p.pt_stride;
    const _Float16* qrow = p.q + (int64_t)row * kHeads * kHeadDim;
    const int m = lane & 31, g = lane >> 5;
    // default form: the row's head-sum factor f; the row is ranked on chain
    // results (score / f), as the filtering pass ranks it
    float inv_f = 1.0f;
    if (!p.relu) {
        float um = 0.0f;
#pragma unroll
        for (int s = 0; s < kSlices; ++s) {
            const _Float16* qs = qrow + 16 * s + 8 * g;
            um = fmaxf(um, head_sum_absmax(*reinterpret_cast<const half8*>(qs),
                                           *reinterpret_cast<const half8*>(qs + kHeadDim),
                                           *reinterpret_cast<const half8*>(qs + 2 * kHeadDim),
                                           *reinterpret_cast<const half8*>(qs + 3 * kHeadDim)));
        }
        um = fmaxf(um, __shfl_xor(um, 32, 64));
        inv_f = 1.0f / head_sum_factor(um);
    }
    int na = 0;
    uint64_t cut = 0ull;  // composites must exceed this to matter once na == kb
    for (int c0 = 0; c0 < V; c0 += ch) {
        if (threadIdx.x == 0) *s_pend = 0;
        __syncthreads();
        const int cend = min(c0 + ch, V);
        for (int j0 = c0 + 32 * wave; j0 < cend; j0 += 32 * kFinWaves) {
            const int j = j0 + m;
            const int jc = min(j, V - 1);
            const int lp = jc / p.kpp;
            const int slot = jc - lp * p.kpp;
            const int pg = min(max(ptrow[lp], 0), p.num_pages - 1);
            const _Float16* key = p.kcache + ((size_t)pg * p.kpp + slot) * kHeadDim;
            half8 kb8[kSlices];
#pragma unroll
            for (int s = 0; s < kSlices; ++s) kb8[s] = *reinterpret_cast<const half8*>(key + 16 * s + 8 * g);
            float16v acc = {};
            float sc;
            if (p.relu) {
#pragma unroll
                for (int s = 0; s < kSlices; ++s) {
                    half8 qv = {};
                    if (m < 4) qv = *reinterpret_cast<const half8*>(qrow + m * kHeadDim + 16 * s + 8 * g);
                    acc = mfma32(qv, kb8[s], acc);
                }
                sc = combine_relu_heads(acc[0], acc[1], acc[2], acc[3]);
            } else {
                // keys as MFMA rows, the row's head sum (hi, lo) as column 0
#pragma unroll
                for (int s = 0; s < kSlices; ++s) {
                    half8 hi = {}, lo = {};
                    if (m == 0) {
                        half8 h[kHeads];
#pragma unroll
                        for (int hh = 0; hh < kHeads; ++hh)
                            h[hh] = *reinterpret_cast<const half8*>(qrow + hh * kHeadDim + 16 * s + 8 * g);
                        head_sum_split(h[0], h[1], h[2], h[3], inv_f, hi, lo);
                    }
                    acc = mfma32(kb8[s], hi, acc);
                    acc = mfma32(kb8[s], lo, acc);
                }
                // lanes 0 and 32 hold the 32 scores (element v: key 8*(v/4) + 4*g + v%4);
                // hand key m's score to lane m through LDS
                float* rs = s_rs + 32 * wave;
                if (m == 0) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) rs[8 * (v >> 2) + 4 * g + (v & 3)] = acc[v];
                }
                __builtin_amdgcn_wave_barrier();
                sc = rs[m];
                __builtin_amdgcn_wave_barrier();
            }
            // lanes 0..31 now hold the row's score of key j0 + lane
            if (g == 0 && j < cend) {
                const uint64_t comp = compose(order_key(sc), (uint32_t)j);
                if (comp > cut) a[na + atomicAdd(s_pend, 1)] = comp;
            }
        }
        __syncthreads();
        const int tot = na + *s_pend;
        __syncthreads();
        if (tot > kb) {
            cut = lds_kth_largest<kFinNT>(a, tot, kb, ks);
            lds_compact_ge<kFinNT, CAPL / kFinNT>(a, tot, cut, ks->wsum);
            na = kb;
        } else {
            na = tot;
        }
    }
    return na;
}

constexpr int kRecChunk = 512;  // keys scored per round by the recompute path

// LDS of the select kernel: the candidate path and the recompute path use
// the same memory (a row takes one of them).
template <int KBMAX>
union SelectLds {
    BoundSelectLds<KBMAX> f;
    struct {
        uint64_t a[KBMAX + kRecChunk];
        KthScratch ks;
        int pend;
        float rs[32 * kFinWaves];
    } r;
};

// The select of one row, by a whole workgroup.  The row's visible count,
// candidate count, threshold and first 2,048 candidate slots are loaded at
// once (slots past the count are clamped into the list and masked).
// Candidate path: the candidates are held in registers as (order key,
// index) and binned by order key between the threshold's key (no candidate
// is below it) and their largest (kSelBins ordered bins); with start[bin] =
// entries in higher bins, every entry of a bin at or above the bin b holding
// the kb-th largest is scattered into LDS at start[bin] + (its arrival in the
// bin) and ranks itself inside its bin by counting larger members: ranks
// below min(kb, V) are the selection, already in rank order.  A bin at or
// above b with more than kMaxBucket entries (heavy clustering or ties)
// switches the row to an exact histogram descent (ties at the cut broken by
// a second descent over inverted indices) and a bitonic sort of the
// selected set.
// Rows whose candidate list is unusable (too short: the threshold was too
// high; too long: it was too low or its score has many ties; or the
// sampling pass left the row out) take the recompute path: exact top-kb by
// recomputation (recompute_row_topk), then a sort in LDS.
// LEAN: the candidate path only, for lists of at most CAPC entries; any
// other row is appended to the redo list for the full version (which then
// writes the whole row), so that the common case runs without the recompute
// path's registers.
template <int KBMAX>
__device__ __forceinline__ BoundSelectLds<KBMAX>& bound_lds(SelectLds<KBMAX>& L) { return L.f; }
template <int KBMAX>
__device__ __forceinline__ BoundSelectLds<KBMAX>& bound_lds(BoundSelectLds<KBMAX>& L) { return L; }

template <int KBMAX, int CAPC, bool LEAN, class LdsT>
__device__ __forceinline__ void select_row(const FinalArgs& A, const int row, LdsT& L) {
    constexpr int EPT = CAPC / kFinNT;
    static_assert(EPT % 4 == 0 && EPT >= 8, "slot groups of 4, two issued up front");
    const int tid = threadIdx.x;
    const int kb = A.kb;
    int32_t* orow = A.out + (int64_t)row * A.out_len;
    const bool vec4 = A.expand == 4 && (A.out_len & 3) == 0 && (reinterpret_cast<uintptr_t>(A.out) & 15) == 0;

    // everything the row needs first, in one round of loads
    const uint64_t* c = A.cand + (int64_t)row * A.cand_cap;
    // (the candidate pass loads 1,280 slots with the count, which covers
    // about 85% of the rows at kb = 512, and the rest only where it is needed)
    constexpr int U0 = LEAN ? 5 : 8;
    uint64_t en[8];
#pragma unroll
    for (int e = 0; e < U0; ++e) en[e] = c[min(e * kFinNT + tid, A.cand_cap - 1)];  // (score bits, key)
    const int n = A.cand_count[(int64_t)row * kCountStride];
    const uint32_t tkey = (uint32_t)(A.thresh[row] >> 32);
    const int V = row_visible_count(A.vis, row);
    const int nsel = min(kb, V);

    if constexpr (LEAN) {
        if (n < nsel || n > A.cand_cap || n > CAPC || A.force_redo) {
            if (tid == 0) A.redo_rows[atomicAdd(A.redo_count, 1)] = row;
            return;
        }
#pragma unroll
        for (int e = U0; e < 8; ++e) en[e] = e * kFinNT < n ? c[min(e * kFinNT + tid, A.cand_cap - 1)] : 0ull;
    } else {
        if (n < nsel || n > A.cand_cap) {
            const int have = recompute_row_topk<KBMAX + kRecChunk>(A, row, V, L.r.a, &L.r.ks, &L.r.pend, L.r.rs);
            lds_sort_desc<kFinNT>(L.r.a, have);
            for (int i = tid; i < A.out_len; i += kFinNT) {
                const int rank = i / A.expand, t = i - rank * A.expand;
                int v = -1;
                if (rank < nsel) v = (int)composite_index(L.r.a[rank]) * A.expand + t;
                orow[i] = v;
            }
            return;
        }
    }
    if (nsel > 0) {
        uint32_t k[EPT], idx[EPT];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool in = e * kFinNT + tid < n;
            k[e] = in ? order_key(__uint_as_float((uint32_t)(en[e] >> 32))) : 0u;
            idx[e] = in ? (uint32_t)en[e] : 0u;
        }
        // the rest of a long list, 4 slots per group
#pragma unroll
        for (int g = 8; g < EPT; g += 4) {
#pragma unroll
            for (int e = g; e < g + 4; ++e) {
                k[e] = 0u;
                idx[e] = 0u;
            }
            if (g * kFinNT < n) {
                uint64_t ex[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ex[e] = c[min((g + e) * kFinNT + tid, A.cand_cap - 1)];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if ((g + e) * kFinNT + tid < n) {
                        k[g + e] = order_key(__uint_as_float((uint32_t)(ex[e] >> 32)));
                        idx[g + e] = (uint32_t)ex[e];
                    }
                }
            }
        }
        // every candidate's key is >= the threshold's
        select_from_bound<kFinNT, EPT, KBMAX>(
            k, [&](int e) { return idx[e]; }, n, nsel, tkey, bound_lds(L),
            [&](int r, uint64_t c) { write_rank(orow, r, composite_index(c), A.expand, vec4); });
    }
    for (int i = nsel * A.expand + tid; i < A.out_len; i += kFinNT) orow[i] = -1;
}

// One row per workgroup (both paths).
template <int KBMAX, int CAPC>
__global__ __launch_bounds__(kFinNT) void fused_select_kernel(FinalArgs A) {
    __shared__ SelectLds<KBMAX> L;
    select_row<KBMAX, CAPC, false>(A, blockIdx.x, L);
}

// Split select, first pass: one row per workgroup, candidate path only.
template <int KBMAX, int CAPC>
__global__ __launch_bounds__(kFinNT) void fused_select_lean_kernel(FinalArgs A) {
    __shared__ BoundSelectLds<KBMAX> L;
    select_row<KBMAX, CAPC, true>(A, blockIdx.x, L);
}

// Split select, second pass: the rows the first pass left, spread over the
// grid (every workgroup reads the same count, so the loop is uniform).
template <int KBMAX, int CAPC>
__global__ __launch_bounds__(kFinNT) void fused_select_redo_kernel(FinalArgs A) {
    __shared__ SelectLds<KBMAX> L;
    const int cnt = min(*A.redo_count, A.a.rows);
    for (int i = blockIdx.x; i < cnt; i += gridDim.x) {
        select_row<KBMAX, CAPC, false>(A, A.redo_rows[i], L);
        __syncthreads();  // before the next row reuses the LDS
    }
}

}  // namespace

FusedPlan plan_fused(int32_t max_visible, int32_t kb) {
    FusedPlan f;
    int stride = 16;
    while ((max_visible + stride - 1) / stride > kMaxSamples) stride *= 2;
    f.stride = stride;
    const double e = (double)kb / stride;
    f.m = (int32_t)(e + 4.0 * std::sqrt(e) + 16.0 + 0.999);
    f.capl = kb <= 1024 ? 4096 : 8192;
    f.cand_cap = f.capl;
    f.ld_s = ((max_visible + stride - 1) / stride + 63) / 64 * 64;
    if (f.ld_s < 64) f.ld_s = 64;
    return f;
}

hipError_t launch_sample_threshold(const float* samp, int64_t ld_s, const VisibleSource& vis, const FusedPlan& f,
                                   bool force_fallback, uint64_t* thresh, int32_t* cand_count, int32_t* redo,
                                   int32_t rows, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    sample_threshold_kernel<<<dim3((unsigned)rows), kThrNT, 0, stream>>>(
        samp, ld_s, vis, f.stride, f.m, force_fallback ? 1 : 0, thresh, cand_count, redo);
    return hipGetLastError();
}

hipError_t launch_fused_final(const PagedArgs& a, const VisibleSource& vis, const FusedPlan& f, const uint64_t* thresh,
                              const uint64_t* cand, const int32_t* cand_count, int32_t* redo, bool force_redo,
                              int32_t kb, int32_t expand, int32_t out_len, int32_t* out, hipStream_t stream) {
    if (a.rows <= 0) return hipSuccess;
    FinalArgs A;
    A.a = a;
    A.vis = vis;
    A.cand = cand;
    A.cand_count = cand_count;
    A.thresh = thresh;
    A.cand_cap = f.cand_cap;
    A.kb = kb;
    A.expand = expand;
    A.out_len = out_len;
    A.out = out;
    A.redo_count = redo;
    A.redo_rows = redo + kRedoHead;
    A.force_redo = force_redo ? 1 : 0;
    const dim3 grid((unsigned)a.rows);
    if (f.capl == 4096) {
        // split: the candidate path for lists of up to 2,048 entries (the
        // common case: about 16m, 1,100 at kb = 512), then every other row
        fused_select_lean_kernel<1024, 2048><<<grid, kFinNT, 0, stream>>>(A);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        fused_select_redo_kernel<1024, 4096><<<dim3((unsigned)std::min(a.rows, kRedoGrid)), kFinNT, 0, stream>>>(A);
    } else {
        fused_select_kernel<QSA_MAX_SELECT, 8192><<<grid, kFinNT, 0, stream>>>(A);
    }
    return hipGetLastError();
}

}  // namespace qsa
