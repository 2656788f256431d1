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

}  // namespace qsa
