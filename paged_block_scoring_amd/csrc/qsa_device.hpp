// qsa_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// The score of (row r, key j) is computed in exactly one way by every kernel
// of this library, so that the scorer, the fused selectors and the fallback
// paths all produce the same bits.  All of them use v_mfma_f32_32x32x16_f16
// (the full-rate fp16 MFMA shape of gfx950) with the key as the column; lane
// half g = lane/32 supplies dims 16s+8g .. 16s+8g+7 of head-dim slice s of
// both operands, and the 32x32 output puts rows 8*(v/4) + 4*(l/32) + (v%4) of
// column l%32 in accumulator element v of lane l.  Accumulation is fp32 from
// +0 in the order given.
//   default form (head sum in K): the score is linear in the query heads,
//     sum_h q_h.k = (sum_h q_h).k, so each query row is first reduced to the
//     fp32 head sum u = ((q_0 + q_1) + q_2) + q_3 (exact fp16 -> fp32 adds),
//     carried as the fp16 pair hi = fp16(u/f), lo = fp16(u/f - hi), which
//     represents u/f to a relative 2^-22 (exactly for small integers); f is
//     1, or 2 or 4 for a row whose head sums leave the fp16 range
//     (head_sum_factor), and the chain's result times f is the score.  The
//     keys are the MFMA rows and the query rows its columns; a chain of 16
//     MFMAs, step t = (slice t/2, part t%2), with A = slice t/2 of the key and
//     B = slice t/2 of hi (t even) or lo (t odd), accumulates the score in one
//     sum.  Element v of lane l is the score of query column l%32 and key row
//     8*(v/4) + 4*(l/32) + v%4.
//   relu form (per head): MFMA row m = 4*row + head (8 query rows x 4 heads);
//     a chain of 8 MFMAs over the slices gives every head's dot, elements
//     4o'..4o'+3 are the four heads of one (row, key), and the score is
//     ((relu h0 + relu h1) + relu h2) + relu h3 times the fp32 value nearest
//     1/sqrt(128).
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", section "Purpose" (FP16 inputs, FP32 accumulation) and "Test Plan"
// (4 index heads, head dim 128); "spec(MODEL-MM-QWEN4-EXP): Qwen3.8-Flash-Next
// is a new architecture ...", section "The component deep-dives, and two
// corrections to the above" (one key head shared by the index heads, scores
// summed over heads, relu and 1/sqrt(head_dim) in its form).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 4;
constexpr int kHeadDim = 128;
constexpr int kKeyBytes = kHeadDim * 2;        // 256 B per compressed key
constexpr int kChunksPerKey = kKeyBytes / 16;  // 16-byte chunks per key
constexpr int kSlices = kHeadDim / 16;         // K-slices of one head per 32x32x16 MFMA chain

// fp32 nearest 1/sqrt(128) = 2^-3.5 (bit pattern 0x3DB504F3).
constexpr float kRsqrtHeadDim = 0x1.6a09e6p-4f;

// Visible keys of a row at position `pos`: key j covers tokens cr*j..cr*j+cr-1
// and exists once token cr*j+cr-1 does, so j < (pos+1)/cr.  Clamped to the
// caller's bound so that no kernel ever reads beyond it.
__device__ __forceinline__ int32_t visible_keys(int32_t pos, int32_t cr, int32_t max_visible) {
    if (pos < 0) return 0;
    int64_t v = ((int64_t)pos + 1) / cr;
    return v > (int64_t)max_visible ? max_visible : (int32_t)v;
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger
// key); -0 is mapped with +0 so that the two tie, as IEEE compares them.
// Adding +0 turns -0 into +0 and leaves every other finite value unchanged
// (fp32 denormals are kept); then a negative value's bits are inverted and a
// non-negative value's sign bit is set -- four VALU operations, no branch.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inverse of order_key (for keys produced by it).
__device__ __forceinline__ float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// 64-bit selection key: score key in the high word, inverted index in the low
// word, so that a larger composite means "higher score, then lower index".
__device__ __forceinline__ uint64_t compose(uint32_t key, uint32_t j) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - j);
}
__device__ __forceinline__ uint32_t composite_index(uint64_t c) {
    return 0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFull);
}

__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Largest magnitude the hi part of a head sum may take: fp16's largest
// finite value.
constexpr float kHalfMax = 65504.0f;

// max |u_i| over the 8 query dims of one fragment, u = ((q0 + q1) + q2) + q3
// in fp32 (default form).
__device__ __forceinline__ float head_sum_absmax(const half8& q0, const half8& q1, const half8& q2,
                                                 const half8& q3) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = fmaxf(m, fabsf((((float)q0[i] + (float)q1[i]) + (float)q2[i]) + (float)q3[i]));
    return m;
}

// The power of two f by which a row's head sum is divided before it is split
// into fp16 parts, from the largest |u| over the row's 128 dims: 1 while every
// u fits fp16 (the common case, where nothing changes), else 2 or 4 -- four
// finite fp16 values sum to at most 4 * 65504, so u / 4 always fits.  The
// split then carries u / f, and the chain's fp32 result times f (an exact
// scale) is the score.  Every score of a row carries the same f, so a row may
// be ranked on chain results directly.
__device__ __forceinline__ float head_sum_factor(float umax) {
    return umax <= kHalfMax ? 1.0f : (umax <= 2.0f * kHalfMax ? 2.0f : 4.0f);
}

// hi/lo fp16 pair of the fp32 head sum of 8 query dims times inv_f (the
// reciprocal of the row's head_sum_factor: 1, 1/2 or 1/4, an exact scale).
__device__ __forceinline__ void head_sum_split(const half8& q0, const half8& q1, const half8& q2, const half8& q3,
                                               float inv_f, half8& hi, half8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float u = ((((float)q0[i] + (float)q1[i]) + (float)q2[i]) + (float)q3[i]) * inv_f;
        const _Float16 h = (_Float16)u;
        hi[i] = h;
        lo[i] = (_Float16)(u - (float)h);
    }
}

// relu of a finite fp32 as one integer max: a value with the sign bit set
// (negative, or -0) is a negative int32 and becomes +0; any other value keeps
// its bits.  (fmaxf would also quiet signalling NaNs first, one more VALU
// operation per head; inputs are finite.)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The four head dots of one (row, key) -> score (relu form).
__device__ __forceinline__ float combine_relu_heads(float h0, float h1, float h2, float h3) {
    const float s = ((relu_bits(h0) + relu_bits(h1)) + relu_bits(h2)) + relu_bits(h3);
    return s * kRsqrtHeadDim;
}

// Byte offset of 16-byte chunk c of key n inside an LDS key tile (256 B per
// key).  The chunk index is XOR-swizzled with the key's low 4 bits so that 16
// consecutive lanes, which read the same chunk of 16 consecutive keys, hit 16
// different bank groups.
__device__ __forceinline__ int lds_key_chunk(int n, int c) {
    return n * kKeyBytes + ((c ^ (n & 15)) << 4);
}

// Block-wide inclusive prefix sum of one int per thread (NT threads, NT a
// multiple of 64).  `wsum` is LDS scratch of NT/64 ints.  Returns the
// inclusive prefix; *total receives the block total.  Contains barriers.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        int x = wsum[w];
        before += (w < wave) ? x : 0;
        all += x;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

}  // namespace qsa
