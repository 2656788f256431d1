// qsa_select.hpp -- workgroup-level exact selection primitives on 64-bit
// composites (order key of the score in the high word, inverted index in the
// low word) held in LDS.  Composites of one row are pairwise distinct, so
// "the k-th largest" is unique and "the elements >= it" are exactly k.
//
// The selection rule is the pages' exact lexicographic top-k ("[Perf][Qwen4Exp]
// Admit the cuBLAS QSA indexer and exact top-k on Turing", section "Purpose":
// higher score first, lower index on ties, one unique set).
#pragma once

#include "qsa_device.hpp"

namespace qsa {

// Descending bitonic sort of n composites (n a power of two) in LDS.
template <int NT>
__device__ void lds_bitonic_sort_desc(uint64_t* a, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += NT) {
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

// Pads a[n .. next_pow2(n)) with 0 (below every real composite), sorts
// descending and returns the padded size.  Contains barriers.
template <int NT>
__device__ int lds_sort_desc(uint64_t* a, int n) {
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = n + (int)threadIdx.x; i < np; i += NT) a[i] = 0ull;
    __syncthreads();
    lds_bitonic_sort_desc<NT>(a, np);
    return np;
}

// Scratch for lds_kth_largest: a 256-bin histogram plus a few words.
struct KthScratch {
    uint32_t hist[256];
    int wsum[16];
    int bin, above;
    uint64_t found;
};

// k-th largest (1 <= k <= n) of the distinct composites a[0..n) in LDS: an
// MSB-first radix select with 8-bit digits.  Each level histograms the
// elements that share the resolved prefix; once a single element remains in
// the cutoff bin it is the answer.  All NT threads must call it.
template <int NT>
__device__ uint64_t lds_kth_largest(const uint64_t* a, int n, int k, KthScratch* s) {
    static_assert(NT >= 256, "one histogram bin per thread");
    uint64_t prefix = 0;
    int need = k;
    for (int level = 0; level < 8; ++level) {
        const int shift = 56 - 8 * level;
        for (int i = threadIdx.x; i < 256; i += NT) s->hist[i] = 0u;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += NT) {
            const uint64_t v = a[i];
            if (level == 0 || (v >> (shift + 8)) == prefix) atomicAdd(&s->hist[(v >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread t < 256 owns bin 255 - t; a block scan orders bins high to low
        const int t = threadIdx.x;
        const int cnt = t < 256 ? (int)s->hist[255 - t] : 0;
        int total;
        const int incl = block_inclusive_scan<NT>(cnt, s->wsum, &total);
        if (t < 256 && incl - cnt < need && incl >= need) {
            s->bin = 255 - t;
            s->above = incl - cnt;
        }
        __syncthreads();
        const int b = s->bin;
        need -= s->above;
        prefix = (prefix << 8) | (uint64_t)b;
        const uint32_t in_bin = s->hist[b];
        __syncthreads();
        if (in_bin == 1u || level == 7) {
            // the unique element whose top (64 - shift) bits equal prefix
            for (int i = threadIdx.x; i < n; i += NT) {
                const uint64_t v = a[i];
                if ((v >> shift) == prefix) s->found = v;
            }
            __syncthreads();
            const uint64_t r = s->found;
            __syncthreads();
            return r;
        }
    }
    return 0ull;  // not reached
}

// Keeps, in order of appearance, the elements of a[0..n) that are >= t,
// compacting them to the front of a; returns their number.  EPT elements per
// thread are staged in registers (n <= EPT * NT).  Contains barriers.
template <int NT, int EPT>
__device__ int lds_compact_ge(uint64_t* a, int n, uint64_t t, int* wsum) {
    uint64_t v[EPT];
    int keep = 0;
    const int base = threadIdx.x * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = base + e;
        v[e] = (i < n) ? a[i] : 0ull;
        keep += (i < n && v[e] >= t) ? 1 : 0;
    }
    int total;
    int dst = block_inclusive_scan<NT>(keep, wsum, &total) - keep;
    // block_inclusive_scan ends with a barrier, so every read above is done
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = base + e;
        if (i < n && v[e] >= t) a[dst++] = v[e];
    }
    __syncthreads();
    return total;
}

// ---------------------------------------------------------------------------
// Register-resident histogram selection on 32-bit keys.  Each of the NT
// threads holds EPT keys in registers, key e being element e*NT + threadIdx.x;
// 0 marks an empty slot (order keys of finite scores are never 0, nor are
// inverted indices).  Keys are binned relative to `base` (the smallest key)
// with kSelBins bins per level: the top level spans the whole key range, each
// further level splits one bin of the level above, until the bin holding the
// wanted rank is exactly filled or one key wide.

constexpr int kSelBits = 10;
constexpr int kSelBins = 1 << kSelBits;

struct HistScratch {
    uint32_t hist[kSelBins + 1];  // the last bin takes empty slots' counts and is never read
    uint32_t wmin[16], wmax[16];
    int wsum[16];
    int bin, above, cnt;
    int flag;
};

__device__ __forceinline__ int bit_length32(uint32_t x) { return x ? 32 - __clz((int)x) : 0; }

// The helpers below read key e of the calling thread as key(e) (a functor,
// so that derived keys need no register array of their own).

// Block-wide smallest and largest nonzero key (both 0 if there is none).
// Slots e with e*NT >= nmax are skipped.  Contains barriers.
template <int NT, int EPT, class KeyF>
__device__ __forceinline__ void block_minmax_u32(KeyF key, int nmax, uint32_t* mn, uint32_t* mx, HistScratch* s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // a = min(key - 1) over all slots (kept in that form until the end): an
    // empty slot (0) wraps to the largest value, so it never wins unless
    // every slot is empty; max ignores empty slots too
    uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        if (e * NT >= nmax) continue;
        const uint32_t ke = key(e);
        a = min(a, ke - 1u);
        b = max(b, ke);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a = min(a, (uint32_t)__shfl_xor((int)a, o, 64));
        b = max(b, (uint32_t)__shfl_xor((int)b, o, 64));
    }
    if (lane == 0) {
        s->wmin[wave] = a;
        s->wmax[wave] = b;
    }
    __syncthreads();
    a = 0xFFFFFFFFu;
    b = 0u;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        a = min(a, s->wmin[w]);
        b = max(b, s->wmax[w]);
    }
    __syncthreads();
    *mn = b ? a + 1u : 0u;
    *mx = b;
}

// One histogram level.  Participants are the nonzero keys whose offset d =
// k - base satisfies d >> pshift == prefix (every key when pshift is 32);
// their digit is (d >> shift) mod 2^(pshift - shift) (< kSelBins).  Finds the
// bin holding the need-th largest participant (1 <= need <= participants) and
// returns it, with *above = participants in higher bins and *cnt =
// participants in that bin.  If `start` is given, start[bin] receives the
// number of participants in bins above `bin`, for every bin.  Contains
// barriers.
template <int NT, int EPT, class KeyF>
__device__ __forceinline__ uint32_t hist_level32(KeyF key, int nmax, uint32_t base, int shift, int pshift,
                                 uint32_t prefix, int need, HistScratch* s, uint32_t* start, int* above, int* cnt) {
    constexpr int BPT = kSelBins / NT;
    static_assert(BPT * NT == kSelBins, "bins per thread");
    const int t = threadIdx.x;
    for (int i = t; i < kSelBins; i += NT) s->hist[i] = 0u;
    __syncthreads();
    const uint32_t dmask = pshift - shift >= 32 ? 0xFFFFFFFFu : ((1u << (pshift - shift)) - 1u);
    if (pshift >= 32) {
        // every key takes part (no branch): an empty slot lands in the guard bin
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (e * NT >= nmax) continue;
            const uint32_t ke = key(e);
            atomicAdd(&s->hist[ke ? (ke - base) >> shift : (uint32_t)kSelBins], 1u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (e * NT >= nmax) continue;
            const uint32_t ke = key(e);
            if (!ke) continue;
            const uint32_t d = ke - base;
            if ((d >> pshift) != prefix) continue;
            atomicAdd(&s->hist[(d >> shift) & dmask], 1u);
        }
    }
    __syncthreads();
    // thread t owns bins kSelBins-1-BPT*t .. kSelBins-BPT*(t+1), high to low
    uint32_t c[BPT];
    int local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        c[j] = s->hist[kSelBins - 1 - BPT * t - j];
        local += (int)c[j];
    }
    int total;
    int run = block_inclusive_scan<NT>(local, s->wsum, &total) - local;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int bin = kSelBins - 1 - BPT * t - j;
        if (start) start[bin] = (uint32_t)run;
        if (run < need && run + (int)c[j] >= need) {
            s->bin = bin;
            s->above = run;
            s->cnt = (int)c[j];
        }
        run += (int)c[j];
    }
    __syncthreads();
    const uint32_t b = (uint32_t)s->bin;
    *above = s->above;
    *cnt = s->cnt;
    __syncthreads();
    return b;
}

// Result of a histogram descent for the need-th largest key.
struct Descent {
    uint32_t pivot;  // keys >= pivot: `need` of them if exact, else more (ties at pivot)
    bool exact;
    int above;       // keys > pivot when !exact (all of them selected)
    uint32_t base;   // smallest key and top-level shift: top-level bin = (k - base) >> shift1
    int shift1;
};

// Descends to the need-th largest of the nonzero keys (1 <= need <= their
// number).  Either some bin is exactly filled -- then exactly `need` keys are
// >= pivot -- or the descent reaches a single key value with more copies than
// needed: pivot is that value, `above` keys are larger.  start1 (optional)
// receives the top level's "keys in higher bins" counts.  Contains barriers.
template <int NT, int EPT, class KeyF>
__device__ __forceinline__ Descent hist_descent32(KeyF key, int nmax, int need, HistScratch* s, uint32_t* start1) {
    Descent r;
    uint32_t mn, mx;
    block_minmax_u32<NT, EPT>(key, nmax, &mn, &mx, s);
    const int shift1 = max(0, bit_length32(mx - mn) - kSelBits);
    r.base = mn;
    r.shift1 = shift1;
    int above, cnt;
    uint32_t prefix = hist_level32<NT, EPT>(key, nmax, mn, shift1, 32, 0u, need, s, start1, &above, &cnt);
    int total_above = above;
    int nd = need - above;
    int cur = shift1;
    while (cnt != nd && cur > 0) {
        const int ns = cur > kSelBits ? cur - kSelBits : 0;
        const uint32_t b = hist_level32<NT, EPT>(key, nmax, mn, ns, cur, prefix, nd, s, nullptr, &above, &cnt);
        prefix = (prefix << (cur - ns)) | b;
        cur = ns;
        nd -= above;
        total_above += above;
    }
    r.pivot = mn + (prefix << cur);
    r.exact = cnt == nd;
    r.above = total_above;
    return r;
}

// ---------------------------------------------------------------------------
// Selection of a row's top-nsel from keys held by the workgroup's threads.

constexpr int kMaxBucket = 256;

template <int KBMAX>
struct BoundSelectLds {
    uint64_t a[KBMAX + kMaxBucket];
    uint32_t start[kSelBins];
    HistScratch hs;
};

// Exact top-nsel of the nonzero keys key(e) (indices idx(e)), sorted: the
// cut is found by a histogram descent over the keys, ties at the cut by a
// second descent over the inverted indices of the keys equal to it; the
// selected set is gathered into LDS and sorted (bitonic).  emit(r, c) is
// called once for each rank r < nsel with that rank's composite c.  Contains
// barriers.
template <int NT, int EPT, int KBMAX, class KeyF, class IdxF, class EmitF>
__device__ __forceinline__ void select_exact_sorted(KeyF key, IdxF idx, int nmax, int nsel, BoundSelectLds<KBMAX>& L,
                                                    EmitF emit) {
    HistScratch& hs = L.hs;
    const int tid = threadIdx.x;
    const Descent d = hist_descent32<NT, EPT>(key, nmax, nsel, &hs, nullptr);
    uint32_t jpiv = 0u;
    if (!d.exact)
        jpiv = hist_descent32<NT, EPT>(
                   [&](int e) {
                       const uint32_t ke = key(e);
                       return ke && ke == d.pivot ? ~idx(e) : 0u;
                   },
                   nmax, nsel - d.above, &hs, nullptr)
                   .pivot;
    if (tid == 0) hs.cnt = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        if (e * NT >= nmax) continue;
        const uint32_t ke = key(e);
        const bool sel = ke && (ke > d.pivot || (ke == d.pivot && (d.exact || ~idx(e) >= jpiv)));
        if (sel) L.a[atomicAdd(&hs.cnt, 1)] = compose(ke, idx(e));
    }
    __syncthreads();
    lds_sort_desc<NT>(L.a, nsel);
    for (int r = tid; r < nsel; r += NT) emit(r, L.a[r]);
}

// Exact top-nsel of register-resident keys with a known lower bound.
//
// Each of the NT threads holds EPT keys k[e] (element e*NT + threadIdx.x,
// index idx(e)); 0 marks an empty slot, slots e with e*NT >= nmax are
// skipped, and every nonempty key is >= lo.  nsel (>= 1) must not exceed the
// number of nonempty keys, nor KBMAX.  emit(r, c) is called exactly once for
// each rank r < nsel, with that rank's composite c.
//
// Method: the keys are binned between lo and their maximum (kSelBins bins of
// a power-of-two width); with start[bin] = keys in higher bins, every key of a
// bin at or above the bin b holding the nsel-th largest is scattered into LDS
// at start[bin] + (its arrival in the bin) and ranks itself inside its bin by
// counting the larger (key, ~index) composites there: its rank is start[bin]
// plus that count.  The result comes out in rank order with no sort.  If a
// bin at or above b holds more than kMaxBucket keys (clustering or ties), the
// workgroup takes select_exact_sorted instead.
template <int NT, int EPT, int KBMAX, class IdxF, class EmitF>
__device__ __forceinline__ void select_from_bound(const uint32_t (&k)[EPT], IdxF idx, int nmax, int nsel, uint32_t lo,
                                  BoundSelectLds<KBMAX>& L, EmitF emit) {
    static_assert(KBMAX >= 1 && (KBMAX & (KBMAX - 1)) == 0, "the sort pads nsel to a power of two <= KBMAX");
    constexpr int BPT = kSelBins / NT;
    static_assert(BPT * NT == kSelBins, "bins per thread");
    HistScratch& hs = L.hs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t mx = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (e * NT < nmax) mx = max(mx, k[e]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
    if (lane == 0) hs.wmax[wave] = mx;
    for (int i = tid; i < kSelBins; i += NT) hs.hist[i] = 0u;
    if (tid == 0) {  // (kept only if fewer than nsel keys were given: then nothing is emitted)
        hs.bin = kSelBins - 1;
        hs.above = 0;
        hs.cnt = 0;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) mx = max(mx, hs.wmax[w]);
    const uint32_t mn = min(lo, mx);
    const int shift1 = max(0, bit_length32(mx - mn) - kSelBits);
    // a key's bin; an empty slot, and (outside the contract) a key below the
    // bound, land in the guard bin kSelBins
    auto bin_of = [&](uint32_t key) {
        return key >= mn ? min((key - mn) >> shift1, (uint32_t)kSelBins) : (uint32_t)kSelBins;
    };
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (e * NT < nmax) atomicAdd(&hs.hist[k[e] ? bin_of(k[e]) : (uint32_t)kSelBins], 1u);
    __syncthreads();
    // thread t owns bins kSelBins-1-BPT*t .. (high to low)
    uint32_t cb[BPT];
    int local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        cb[j] = hs.hist[kSelBins - 1 - BPT * tid - j];
        local += (int)cb[j];
    }
    int total;
    int run = block_inclusive_scan<NT>(local, hs.wsum, &total) - local;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        const int bin = kSelBins - 1 - BPT * tid - j;
        L.start[bin] = (uint32_t)run;
        if (run < nsel && run + (int)cb[j] >= nsel) {
            hs.bin = bin;
            hs.above = run;
            hs.cnt = (int)cb[j];
        }
        run += (int)cb[j];
    }
    __syncthreads();
    const int b = hs.bin, above = hs.above, cnt = hs.cnt;
    bool slow = cnt > kMaxBucket;
    if (!slow) {
        __syncthreads();
        for (int i = tid; i < kSelBins; i += NT) hs.hist[i] = 0u;
        if (tid == 0) hs.flag = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (e * NT < nmax && k[e]) {
                const uint32_t bn = bin_of(k[e]);
                if (bn < (uint32_t)kSelBins && (int)bn >= b) L.a[L.start[bn] + atomicAdd(&hs.hist[bn], 1u)] = compose(k[e], idx(e));
            }
        }
        __syncthreads();
        for (int p = tid; p < above + cnt; p += NT) {
            const uint64_t me = L.a[p];
            const uint32_t bn = min(bin_of((uint32_t)(me >> 32)), (uint32_t)kSelBins - 1u);
            const int st = (int)L.start[bn], cn = (int)hs.hist[bn];
            if (cn > kMaxBucket) {
                hs.flag = 1;  // a crowded bin above b: the sort below takes over
                continue;
            }
            int r = 0;
            for (int i = st; i < st + cn; ++i) r += L.a[i] > me ? 1 : 0;
            // (unsigned: a rank is never negative, whatever the list held)
            if ((unsigned)(st + r) < (unsigned)nsel) emit(st + r, me);
        }
        __syncthreads();
        slow = hs.flag != 0;
    }
    if (slow) select_exact_sorted<NT, EPT, KBMAX>([&](int e) { return k[e]; }, idx, nmax, nsel, L, emit);
}

// Writes rank r's block, expanded to `expand` consecutive tokens, into an
// output row (one 16-byte store for 4-token blocks when the row is 16-byte
// aligned and its length a multiple of 4).
__device__ __forceinline__ void write_rank(int32_t* orow, int r, uint32_t idx, int expand, bool vec4) {
    const int base = (int)idx * expand;
    if (vec4) {
        typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<i32x4*>(orow + 4 * r) = i32x4{base, base + 1, base + 2, base + 3};
        return;
    }
    for (int t = 0; t < expand; ++t) orow[r * expand + t] = base + t;
}

}  // namespace qsa
