// topk.hip -- exact lexicographic top-k per row over materialised fp32 scores.
//
// Sources: "qwen4_exp QSA cooperative_topk cannot launch on NVIDIA Thor
// (sm_110): cluster misconfiguration", section "What happens" (the top-k op
// takes the score matrix, each row's visible count, k and the column count,
// plus a caller workspace); "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and
// exact top-k on Turing", section "Purpose" (an exact selector: higher score
// first, lower index on ties, so the selected set is unique even when scores
// tie at the cutoff) and "Test Result" (the invariant that no selected value
// is below an unselected one).
//
// Method: one workgroup per row.  Scores map to order-preserving 32-bit keys;
// a (key, inverted index) 64-bit composite is a total order whose descending
// order is exactly the selection order.
//  * Rows with at most kCap candidates are sorted whole in LDS.
//  * Longer rows run an MSB radix select with 11/11/10-bit digits and an LDS
//    histogram per level.  After each level the count of keys whose resolved
//    high bits are >= the cutoff prefix is known; as soon as it fits in kCap
//    those candidates (a superset of the top k) are gathered into LDS and
//    sorted.  If 32 bits are resolved and the cutoff key still has more
//    copies than fit, the keys above the cutoff are gathered and the
//    lowest-index copies of the cutoff key are taken by an index-ordered
//    block prefix scan.
//  * A bitonic sort of the 64-bit composites in LDS yields rank order; block
//    j is written as `expand` consecutive entries j*expand .. j*expand+expand-1
//    (tokens) or as j (keys), and missing ranks as -1.
#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_select.hpp"

namespace qsa {
namespace {

constexpr int kNT = 512;
constexpr int kCap = 4096;
constexpr int kBins = 2048;
static_assert(kBins == 4 * kNT, "bin scan assumes 4 bins per thread");

struct TopkArgs {
    const float* scores;
    int64_t ld;
    VisibleSource vis;
    int32_t kk;
    int32_t expand;
    int32_t out_len;
    int32_t* out;
};

__device__ __forceinline__ int row_visible(const VisibleSource& v, int r) {
    if (v.visible) return min(max(v.visible[r], 0), v.max_visible);
    if (v.pos) {
        const int req = v.row_req ? v.row_req[r] : 0;
        if (req < 0 || req >= v.num_reqs) return 0;
        return visible_keys(v.pos[r], v.cr, v.max_visible);
    }
    return v.max_visible;
}

// Descending bitonic sort of n (a power of two, <= kCap) composites in LDS.
__device__ void bitonic_sort_desc(uint64_t* a, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += kNT) {
                const int p = i ^ j;
                if (p > i) {
                    const uint64_t x = a[i], y = a[p];
                    const bool desc = (i & k) == 0;
                    if (desc ? (x < y) : (x > y)) {
                        a[i] = y;
                        a[p] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(kNT) void topk_rows_kernel(TopkArgs A) {
    __shared__ uint64_t s_cand[kCap];
    __shared__ uint32_t s_hist[kBins];
    __shared__ int s_wsum[kNT / 64];
    __shared__ int s_count, s_bin, s_above;

    const int row = blockIdx.x, tid = threadIdx.x;
    const int V = row_visible(A.vis, row);
    const float* srow = A.scores + (int64_t)row * A.ld;
    const int kk = A.kk;
    const int nsel = min(kk, V);
    int ncand;

    if (V <= kCap) {
        for (int j = tid; j < V; j += kNT) s_cand[j] = compose(order_key(srow[j]), (uint32_t)j);
        ncand = V;
    } else {
        uint32_t prefix = 0;
        int shift = 32, above_total = 0, need = kk;
        bool done = false;
        ncand = 0;
        for (int level = 0; level < 3 && !done; ++level) {
            const int bits = level < 2 ? 11 : 10;
            const int nshift = shift - bits;
            const uint32_t mask = (1u << bits) - 1u;
            for (int i = tid; i < kBins; i += kNT) s_hist[i] = 0u;
            __syncthreads();
            for (int j = tid; j < V; j += kNT) {
                const uint32_t u = order_key(srow[j]);
                if (level == 0 || (u >> shift) == prefix) atomicAdd(&s_hist[(u >> nshift) & mask], 1u);
            }
            __syncthreads();
            // Thread t owns bins 2047-4t .. 2044-4t (descending); a block scan
            // gives the number of keys in higher bins.
            int local[4], lsum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                local[i] = (int)s_hist[kBins - 1 - (4 * tid + i)];
                lsum += local[i];
            }
            int total;
            int run = block_inclusive_scan<kNT>(lsum, s_wsum, &total) - lsum;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (run < need && run + local[i] >= need) {
                    s_bin = kBins - 1 - (4 * tid + i);
                    s_above = run;
                }
                run += local[i];
            }
            __syncthreads();
            const int b = s_bin, above = s_above;
            need -= above;
            above_total += above;
            prefix = (level == 0) ? (uint32_t)b : ((prefix << bits) | (uint32_t)b);
            shift = nshift;
            const int cnt_ge = above_total + (int)s_hist[b];
            __syncthreads();
            if (cnt_ge <= kCap) {
                if (tid == 0) s_count = 0;
                __syncthreads();
                for (int j = tid; j < V; j += kNT) {
                    const uint32_t u = order_key(srow[j]);
                    if ((u >> shift) >= prefix) s_cand[atomicAdd(&s_count, 1)] = compose(u, (uint32_t)j);
                }
                __syncthreads();
                ncand = s_count;
                done = true;
            }
        }
        if (!done) {
            // prefix is the exact cutoff key; above_total keys exceed it and
            // `need` of its copies are taken, lowest indices first.
            const uint32_t tau = prefix;
            if (tid == 0) s_count = 0;
            __syncthreads();
            for (int j = tid; j < V; j += kNT) {
                const uint32_t u = order_key(srow[j]);
                if (u > tau) s_cand[atomicAdd(&s_count, 1)] = compose(u, (uint32_t)j);
            }
            int base = 0;
            for (int j0 = 0; j0 < V && base < need; j0 += kNT) {
                const int j = j0 + tid;
                const int f = (j < V && order_key(srow[j]) == tau) ? 1 : 0;
                int total;
                const int incl = block_inclusive_scan<kNT>(f, s_wsum, &total);
                const int rank = base + incl - f;
                if (f && rank < need) s_cand[above_total + rank] = compose(tau, (uint32_t)j);
                base += total;
            }
            __syncthreads();
            ncand = above_total + min(need, base);
        }
    }

    int npow = 1;
    while (npow < ncand) npow <<= 1;
    for (int i = ncand + tid; i < npow; i += kNT) s_cand[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc(s_cand, npow);

    int32_t* orow = A.out + (int64_t)row * A.out_len;
    for (int i = tid; i < A.out_len; i += kNT) {
        const int rank = i / A.expand, t = i - rank * A.expand;
        int v = -1;
        if (rank < nsel) v = (int)composite_index(s_cand[rank]) * A.expand + t;
        orow[i] = v;
    }
}

// Rows whose visible keys fit in registers (V <= NT * EPT, with NT threads
// per workgroup).  Every score is loaded once, all loads issued before any
// use, and kept as its order key (element e of thread t is key e*NT + t).  One
// histogram level (kSelBins bins of a power-of-two width between the smallest
// and largest key) finds the bin holding the kk-th largest -- for long rows
// first over every 8th slot only, the bound then checked by an exact count --
// and the keys from that bin's lower edge up (usually a few more than kk) are
// compacted into LDS, where select_from_bound (qsa_select.hpp) ranks them
// exactly, usually with no sort at all.  If more than kCompact keys survive
// (heavy ties or clustering at the cut), the row is selected by
// select_exact_sorted instead, with keys re-read from the score row at each
// level.
constexpr int kRegNT = 512;  // threads per workgroup for rows of 8,193 .. 49,152 keys

// x, with the compiler unable to reuse an earlier expression built from it:
// element indices e*NT + tid are then formed where used instead of being
// held in EPT registers across the kernel.
__device__ __forceinline__ int fresh(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
constexpr int kCompact = 4096;

template <int KBMAX>
struct TopkRegsLds {
    BoundSelectLds<KBMAX> s;
    uint64_t c[kCompact];
    int nc;
};

// The rare path of topk_regs_kernel, kept out of line so that its register
// needs do not constrain the common path.
template <int NT, int EPT, int KBMAX>
__device__ __noinline__ void topk_row_exact_sorted(const uint32_t* srow, int V, int nsel, BoundSelectLds<KBMAX>* L,
                                                   int32_t* orow, int expand, bool vec4) {
    const int tid = threadIdx.x;
    select_exact_sorted<NT, EPT, KBMAX>(
        [&](int e) {
            const int j = e * NT + tid;
            return j < V ? order_key(__uint_as_float(srow[j])) : 0u;
        },
        [&](int e) { return (uint32_t)(e * NT + tid); }, V, nsel, *L,
        [&](int r, uint64_t c) { write_rank(orow, r, composite_index(c), expand, vec4); });
}

template <int NT, int EPT, int KBMAX>
__global__ __launch_bounds__(NT) void topk_regs_kernel(TopkArgs A) {
    __shared__ TopkRegsLds<KBMAX> L;
    const int row = blockIdx.x, tid = threadIdx.x;
    const int V = row_visible(A.vis, row);
    const int nsel = min(A.kk, V);
    int32_t* orow = A.out + (int64_t)row * A.out_len;
    const bool vec4 = A.expand == 4 && (A.out_len & 3) == 0 && (reinterpret_cast<uintptr_t>(A.out) & 15) == 0;
    const auto emit = [&](int r, uint64_t c) { write_rank(orow, r, composite_index(c), A.expand, vec4); };
    if (nsel > 0) {
        const uint32_t* srow = reinterpret_cast<const uint32_t*>(A.scores + (int64_t)row * A.ld);
        uint32_t k[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) k[e] = srow[min(e * NT + tid, V - 1)];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {  // keys past V become 0 (a per-lane test only in the slot V falls in)
            const uint32_t ke = order_key(__uint_as_float(k[e]));
            if ((e + 1) * NT <= V)
                k[e] = ke;
            else
                k[e] = e * NT + tid < V ? ke : 0u;
        }
        const auto key = [&](int e) { return k[e]; };
        // A cheap bound first: the range and histogram of every 8th slot give
        // the bin of its m-th largest key (m covers nsel/8 with a margin); the
        // keys at or above that bin's lower edge are then counted exactly, and
        // the count's prefix sum gives every thread its survivors' places.
        // With nsel .. kCompact of them they hold the row's top nsel; with too
        // few or too many the range and histogram of every key decide instead.
        uint32_t lo = 0u;
        int surv = -1, myoff = 0;
        if constexpr (EPT >= 64) {
            constexpr int S = EPT / 8;
            int sampled = 0;  // nonzero keys in slots 0, 8, 16, ...
#pragma unroll
            for (int j = 0; j < S; ++j) sampled += min(max(V - 8 * j * NT, 0), NT);
            const float q = (float)nsel / 8.0f;
            const int m = (int)(q + 3.0f * sqrtf(q) + 8.0f);
            if (m <= sampled) {
                const auto skey = [&](int j) { return k[8 * j]; };
                uint32_t smn, smx;
                block_minmax_u32<NT, S>(skey, (V + 7) / 8, &smn, &smx, &L.s.hs);
                const int sshift = max(0, bit_length32(smx - smn) - kSelBits);
                int sa, sc;
                const uint32_t bs = hist_level32<NT, S>(skey, (V + 7) / 8, smn, sshift, 32, 0u, m, &L.s.hs,
                                                            nullptr, &sa, &sc);
                lo = smn + (bs << sshift);
                int c = 0;
#pragma unroll
                for (int e = 0; e < EPT; ++e) c += k[e] >= lo ? 1 : 0;
                int total;
                myoff = block_inclusive_scan<NT>(c, L.s.hs.wsum, &total) - c;
                surv = total;
            }
        }
        const bool placed = surv >= nsel && surv <= kCompact;
        if (!placed) {
            uint32_t mn, mx;
            block_minmax_u32<NT, EPT>(key, V, &mn, &mx, &L.s.hs);  // (slots wholly past V skipped)
            const int shift1 = max(0, bit_length32(mx - mn) - kSelBits);
            int above, cnt;
            const uint32_t b = hist_level32<NT, EPT>(key, V, mn, shift1, 32, 0u, nsel, &L.s.hs, nullptr, &above, &cnt);
            lo = mn + (b << shift1);
            surv = above + cnt;  // keys >= lo (lo >= the smallest key > 0)
        }
        if (surv <= kCompact) {
            const int lane = tid & 63;
            if (placed) {
                // every thread stores its survivors from its own place on (no
                // atomics); a key's store has its compare's ballot as exec
                uint32_t ad =
                    (uint32_t)reinterpret_cast<uintptr_t>(static_cast<void*>(&L.c[0])) + 8u * (uint32_t)myoff;
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const bool p = k[e] >= lo;
                    const uint64_t mk = __builtin_amdgcn_ballot_w64(p);
                    const uint64_t cv = compose(k[e], (uint32_t)(e * NT + fresh(tid)));
                    asm volatile(
                        "s_mov_b64 exec, %[m]\n\t"
                        "ds_write_b64 %[ad], %[d]\n\t"
                        "s_mov_b64 exec, -1"
                        :
                        : [m] "s"(mk), [ad] "v"(ad), [d] "v"(cv)
                        : "memory");
                    ad += p ? 8u : 0u;
                }
                // (the compiler's wait counting does not see these stores: they
                // must land before the barrier lets other waves read them)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            } else {
                if (tid == 0) L.nc = 0;
                __syncthreads();
                // the survivors, eight slots at a time: one LDS atomic per wave
                // and batch reserves the batch's places, ballots order the lanes
                const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
                for (int g = 0; g < EPT; g += 8) {
                    uint64_t mk[8];
                    int tot = 0;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        mk[u] = __ballot(g + u < EPT && k[g + u] >= lo);
                        tot += __popcll(mk[u]);
                    }
                    if (tot) {  // (wave-uniform)
                        int at = 0;
                        if (lane == 0) at = atomicAdd(&L.nc, tot);
                        at = __builtin_amdgcn_readfirstlane(at);
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            if (g + u < EPT && ((mk[u] >> lane) & 1ull))
                                L.c[at + __popcll(mk[u] & below)] =
                                    compose(k[g + u], (uint32_t)((g + u) * NT + fresh(tid)));
                            at += __popcll(mk[u]);
                        }
                    }
                }
            }
            __syncthreads();
            constexpr int E2 = kCompact / NT;
            uint32_t k2[E2], i2[E2];
#pragma unroll
            for (int e = 0; e < E2; ++e) {
                const int p = e * NT + tid;
                const uint64_t ce = p < surv ? L.c[p] : 0ull;
                k2[e] = (uint32_t)(ce >> 32);
                i2[e] = composite_index(ce);
            }
            select_from_bound<NT, E2, KBMAX>(k2, [&](int e) { return i2[e]; }, surv, nsel, lo, L.s, emit);
        } else {
            topk_row_exact_sorted<NT, EPT, KBMAX>(srow, V, nsel, &L.s, orow, A.expand, vec4);
        }
    }
    for (int i = nsel * A.expand + tid; i < A.out_len; i += NT) orow[i] = -1;
}

template <int NT, int EPT>
void launch_regs(const TopkArgs& A, int32_t rows, hipStream_t stream) {
    if (A.kk <= 1024)
        topk_regs_kernel<NT, EPT, 1024><<<dim3((unsigned)rows), NT, 0, stream>>>(A);
    else
        topk_regs_kernel<NT, EPT, QSA_MAX_SELECT><<<dim3((unsigned)rows), NT, 0, stream>>>(A);
}

}  // namespace

hipError_t launch_topk_rows(const float* scores, int64_t ld, const VisibleSource& vis, int32_t rows,
                            int32_t kk, int32_t expand, int32_t out_len, int32_t* out,
                            hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    TopkArgs A;
    A.scores = scores;
    A.ld = ld;
    A.vis = vis;
    A.kk = kk;
    A.expand = expand;
    A.out_len = out_len;
    A.out = out;
    // rows of up to 8,192 keys: 256-thread workgroups (two resident per compute
    // unit) when the rows outnumber the compute units, else 512 threads per row
    // (lower latency); longer rows: 512 threads
    if (vis.max_visible <= kRegNT * 16 && rows < 256)
        launch_regs<kRegNT, 16>(A, rows, stream);
    else if (vis.max_visible <= 256 * 32)
        launch_regs<256, 32>(A, rows, stream);
    else if (vis.max_visible <= kRegNT * 96)
        launch_regs<kRegNT, 96>(A, rows, stream);
    else
        topk_rows_kernel<<<dim3((unsigned)rows), kNT, 0, stream>>>(A);
    return hipGetLastError();
}

}  // namespace qsa
