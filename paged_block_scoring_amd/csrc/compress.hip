// compress.hip -- the compressed-key producer: builds the indexer's paged side
// cache, one key per block of `cr` tokens, from the raw per-token index keys.
//
// Source: "spec(MODEL-MM-QWEN4-EXP): Qwen3.8-Flash-Next is a new architecture
// ...", section "The component deep-dives, and two corrections to the above":
// one stored state per ratio tokens, written when a token's (position + 1) is a
// multiple of the ratio, holding a pooled key with RMSNorm applied to it and
// RoPE applied at the block-start position.  The pages name no pooling for
// this model (the DeepSeek-V4 learned pool does not apply); readings taken
// here: the arithmetic mean of the block's token keys, RMSNorm
// w_i x_i / sqrt(mean x^2 + eps), RoPE over the leading rope_dim values at
// angles p0 * base^(-2i/rope_dim) with p0 = cr * block, pairs (i, i + rope_dim/2)
// or, with the interleaved flag, (2i, 2i + 1).
//
// A call sees each request's new tokens as one run of consecutive positions
// in consecutive token slots (a prefill chunk, or one decode token).  A block
// whose last token is in the call is finished here; its earlier tokens are
// either earlier in the same run or, when an earlier call saw them, in the
// request's staging state [cr][128].  Two launches, in this order:
//   compress_blocks_kernel -- a workgroup takes 256 token slots at a time:
//     their (request, position) pairs, with the cr-1 slots before them, go to
//     LDS; the slots whose token closes a block are compacted into a list and
//     dealt round-robin to the workgroup's sixteen 16-lane groups.  A group
//     gathers its block's cr keys (16 bytes per lane per key, one 256-byte key
//     per group), takes the mean in fp32, RMSNorm (sum of squares over the
//     group by lane exchange) and RoPE (partner values by lane exchange),
//     rounds to fp16 and writes the key's slot of its page.  Each rotation
//     angle p0 * f_i (f_i / 2 pi from a host table) loses its whole turns in
//     fp64, so positions near 2^31 keep full fp32 accuracy, then cos and sin
//     are Taylor polynomials in fp32; the two lanes of a rotate-half pair
//     share one set of angles;
//   stage_open_kernel      -- one thread per token: copies the keys of tokens
//     whose block stays open at the end of the call into the staging state.
// The second launch may overwrite staging slots the first one reads (a run
// that finishes one block and leaves a later one open), hence two launches on
// one stream rather than one.
#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

#include <cmath>

namespace qsa {
namespace {

constexpr int kD = 128;           // key length
constexpr int kNT = 256;          // threads per workgroup; token slots per window
constexpr int kGroups = kNT / 16; // 16-lane groups per workgroup: one key each
constexpr int kMaxCr = 64;
constexpr int kMaxPairs = kD / 2;

typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

struct CompressArgs {
    const _Float16* k_tok;     // [T][128]
    const int32_t* tok_req;    // [T] or null (request 0)
    const int32_t* tok_pos;    // [T]
    int32_t T;
    const float* norm_w;       // [128] or null (weight 1)
    float eps;
    int32_t rope_dim;          // multiple of 16, <= 128
    bool interleaved;
    _Float16* state;           // [num_reqs][cr][128]
    _Float16* kcache;          // [num_pages][kpp][128]
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t num_pages;
    int32_t num_reqs;
    int32_t cr;
    int32_t kpp;
    int32_t cr_shift;          // log2(cr) and log2(kpp) when both are powers of two
    int32_t kpp_shift;
    double turns[kMaxPairs];   // rope_base^(-2i/rope_dim) / (2 pi), i < rope_dim/2
};

__device__ __forceinline__ void unpack8(const u32x4a v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = v[j];
        f[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
        f[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
}

__device__ __forceinline__ u32x4a pack8(const float* f) {
    u32x4a v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint16_t lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * j]);
        const uint16_t hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * j + 1]);
        v[j] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return v;
}

// cos and sin of the angle p0 * f_i, with g = f_i / (2 pi) in fp64: the angle
// in quarter turns, 4 (p0 g - round(p0 g)), splits exactly in fp64 into an
// integer q and w in [-1/2, 1/2] (so positions near 2^31 keep full fp32
// accuracy); r = w pi/2 in fp32, the Taylor series of sin and cos at 0
// through r^9 and r^10 (truncation below 2e-9 on |r| <= pi/4), and q mod 4
// picks signs and swaps.
__device__ __forceinline__ void turn(double p0, double g, float* c, float* s) {
    const double u = p0 * g;
    const double t4 = 4.0 * (u - rint(u));
    const double qd = rint(t4);
    const float r = (float)(t4 - qd) * 1.57079632679489662f;
    const float r2 = r * r;
    const float sr = r * (1.0f + r2 * (-1.0f / 6 + r2 * (1.0f / 120 + r2 * (-1.0f / 5040 + r2 * (1.0f / 362880)))));
    const float cr = 1.0f + r2 * (-0.5f + r2 * (1.0f / 24 + r2 * (-1.0f / 720 + r2 * (1.0f / 40320 +
                                                                                      r2 * (-1.0f / 3628800)))));
    const int quad = (int)qd & 3;                  // q in -2 .. 2
    const float sa = (quad & 1) ? cr : sr;
    const float ca = (quad & 1) ? sr : cr;
    *s = (quad & 2) ? -sa : sa;
    *c = (quad == 1 || quad == 2) ? -ca : ca;
}

// a / d and a % d for a >= 0; with POW2, d = 1 << sh.
template <bool POW2>
__device__ __forceinline__ int32_t qdiv(int32_t a, int32_t d, int sh) { return POW2 ? a >> sh : a / d; }
template <bool POW2>
__device__ __forceinline__ int32_t qmod(int32_t a, int32_t d, int sh) { return POW2 ? a & (d - 1) : a % d; }

// (request, position) of a token slot as one word; slots outside the call
// hold a request of -1
__device__ __forceinline__ uint64_t slot_key(int32_t q, int32_t p) {
    return ((uint64_t)(uint32_t)q << 32) | (uint32_t)p;
}

struct CompressLds {
    uint64_t rp[kNT + kMaxCr];   // window slots base-(cr-1) .. base+255
    int32_t list[kNT];           // window offsets of the closing tokens
    int32_t wcount[kNT / 64];
};

template <bool POW2>
__global__ __launch_bounds__(kNT) void compress_blocks_kernel(CompressArgs A) {
    __shared__ CompressLds L;
    const int tid = threadIdx.x;
    const int lane16 = tid & 15;
    const int group = tid >> 4;
    const int wave = tid >> 6;
    const int d0 = lane16 * 8;                      // this lane's 8 values
    const int half = A.rope_dim / 2;
    const bool in_rope = d0 < A.rope_dim;
    const bool first_half = d0 < half;
    // rotate-half partner lane (values d0 .. d0+7 pair with d0 +- half; half is
    // a multiple of 8, so the partner holds the same element positions and
    // the same frequencies: each of the two turns four of them and they swap)
    const int partner = !in_rope || A.interleaved ? lane16 : (first_half ? lane16 + half / 8 : lane16 - half / 8);
    // this lane's four frequencies, in turns per position
    double g[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = A.interleaved ? (d0 >> 1) + m : (first_half ? d0 + m : d0 - half + 4 + m);
        g[m] = in_rope ? A.turns[i] : 0.0;
    }
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = A.norm_w ? A.norm_w[d0 + e] : 1.0f;
    const float inv_cr = 1.0f / (float)A.cr;
    const int halo = A.cr - 1;
    const int crs = A.cr_shift, kps = A.kpp_shift;

    for (int64_t base = (int64_t)blockIdx.x * kNT; base < A.T; base += (int64_t)gridDim.x * kNT) {
        bool closer = false;
        int cx = 0;                                      // window index of this thread's closing token
        for (int i = tid; i < kNT + halo; i += kNT) {
            const int64_t s = base - halo + i;
            const bool in = s >= 0 && s < A.T;
            const int32_t p = in ? A.tok_pos[s] : -1;
            const int32_t q = in ? (A.tok_req ? A.tok_req[s] : 0) : -1;
            L.rp[i] = slot_key(q, p);
            // indices halo .. halo+255 are the window's own slots, one per thread
            if (i >= halo && p >= 0 && q >= 0 && q < A.num_reqs && qmod<POW2>(p, A.cr, crs) == A.cr - 1 &&
                qdiv<POW2>(qdiv<POW2>(p, A.cr, crs), A.kpp, kps) < A.pt_stride) {
                closer = true;
                cx = i;
            }
        }
        const uint64_t mask = __ballot(closer);
        if ((tid & 63) == 0) L.wcount[wave] = __popcll(mask);
        __syncthreads();
        int off = 0, n = 0;
#pragma unroll
        for (int v = 0; v < kNT / 64; ++v) {
            off += v < wave ? L.wcount[v] : 0;
            n += L.wcount[v];
        }
        if (closer) L.list[off + __popcll(mask & __lanemask_lt())] = cx;
        __syncthreads();

        for (int k = group; k < n; k += kGroups) {
            const int x = L.list[k];                     // window index of the closing token
            const int64_t t = base - halo + x;
            const uint64_t key = L.rp[x];
            const int32_t p = (int32_t)(uint32_t)key;
            const int32_t q = (int32_t)(key >> 32);
            const int32_t c = qdiv<POW2>(p, A.cr, crs);           // block index
            int32_t page = A.page_table[(int64_t)q * A.pt_stride + qdiv<POW2>(c, A.kpp, kps)];
            page = min(max(page, 0), A.num_pages - 1);
            const int32_t p0 = c * A.cr;

            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int j0 = 0; j0 < A.cr; j0 += 4) {
                // position p0 + j sits cr-1-j slots before the closing token when
                // this call holds it, else in the request's staging state
                uint64_t have[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) have[u] = j0 + u < A.cr ? L.rp[x - (A.cr - 1 - j0 - u)] : 0;
                u32x4a raw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = j0 + u;
                    if (j < A.cr) {
                        const _Float16* src = have[u] == slot_key(q, p0 + j)
                                                  ? A.k_tok + (t - (A.cr - 1 - j)) * kD
                                                  : A.state + ((int64_t)q * A.cr + j) * kD;
                        raw[u] = *reinterpret_cast<const u32x4a*>(src + d0);
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (j0 + u < A.cr) {
                        float f[8];
                        unpack8(raw[u], f);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] += f[e];
                    }
                }
            }
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc[e] *= inv_cr;
                ss += acc[e] * acc[e];
            }
            ss += __shfl_xor(ss, 1, 16);
            ss += __shfl_xor(ss, 2, 16);
            ss += __shfl_xor(ss, 4, 16);
            ss += __shfl_xor(ss, 8, 16);
            const float r = 1.0f / sqrtf(ss * (1.0f / kD) + A.eps);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = acc[e] * r * w[e];

            float cs[4], sn[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                cs[m] = 1.0f;
                sn[m] = 0.0f;
            }
            if (in_rope) {
#pragma unroll
                for (int m = 0; m < 4; ++m) turn((double)p0, g[m], &cs[m], &sn[m]);
            }
            float o[8];
            if (A.interleaved) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    o[2 * m] = y[2 * m] * cs[m] - y[2 * m + 1] * sn[m];
                    o[2 * m + 1] = y[2 * m + 1] * cs[m] + y[2 * m] * sn[m];
                }
            } else {
                float pc[4], ps[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    pc[m] = __shfl(cs[m], partner, 16);
                    ps[m] = __shfl(sn[m], partner, 16);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = __shfl(y[e], partner, 16);
                    // values e < 4 use the first-half lane's angles, e >= 4 the other's
                    const float ce = (e < 4) == first_half ? cs[e & 3] : pc[e & 3];
                    const float se = (e < 4) == first_half ? sn[e & 3] : ps[e & 3];
                    o[e] = first_half ? y[e] * ce - pv * se : y[e] * ce + pv * se;
                }
            }
            *reinterpret_cast<u32x4a*>(A.kcache + ((int64_t)page * A.kpp + qmod<POW2>(c, A.kpp, kps)) * kD + d0) =
                pack8(o);
        }
        __syncthreads();   // the window is rewritten next
    }
}

// One thread per token: a token whose block has no closing token in this call
// goes to the staging state (16 pieces of 16 bytes).
__global__ __launch_bounds__(kNT) void stage_open_kernel(CompressArgs A) {
    const int64_t t = (int64_t)blockIdx.x * kNT + threadIdx.x;
    if (t >= A.T) return;
    const int32_t p = A.tok_pos[t];
    const int32_t q = A.tok_req ? A.tok_req[t] : 0;
    if (p < 0 || q < 0 || q >= A.num_reqs) return;
    const int32_t slot = p % A.cr;
    const int64_t d = A.cr - 1 - slot;           // slots to the block's last token
    if (t + d < A.T && (A.tok_req ? A.tok_req[t + d] : 0) == q && (int64_t)A.tok_pos[t + d] == (int64_t)p + d)
        return;                                  // finished in this call
    const u32x4a* src = reinterpret_cast<const u32x4a*>(A.k_tok + t * kD);
    u32x4a* dst = reinterpret_cast<u32x4a*>(A.state + ((int64_t)q * A.cr + slot) * kD);
#pragma unroll
    for (int u = 0; u < kD / 8; ++u) dst[u] = src[u];
}

}  // namespace

hipError_t launch_compress(const _Float16* k_tok, const int32_t* tok_req, const int32_t* tok_pos, int32_t T,
                           const float* norm_w, float eps, int32_t rope_dim, double rope_base, bool interleaved,
                           _Float16* state, _Float16* kcache, const int32_t* page_table, int64_t pt_stride,
                           int32_t num_pages, int32_t num_reqs, int32_t page_size, int32_t cr, int32_t cus,
                           hipStream_t stream, hipError_t (*mark)(hipStream_t)) {
    if (T <= 0) return hipSuccess;
    if (cr < 1 || cr > kMaxCr || rope_dim < 0 || rope_dim > kD || rope_dim % 16 != 0) return hipErrorInvalidValue;
    CompressArgs A;
    A.k_tok = k_tok;
    A.tok_req = tok_req;
    A.tok_pos = tok_pos;
    A.T = T;
    A.norm_w = norm_w;
    A.eps = eps;
    A.rope_dim = rope_dim;
    A.interleaved = interleaved;
    A.state = state;
    A.kcache = kcache;
    A.page_table = page_table;
    A.pt_stride = pt_stride;
    A.num_pages = num_pages;
    A.num_reqs = num_reqs;
    A.cr = cr;
    A.kpp = page_size / cr;
    for (int i = 0; i < kMaxPairs; ++i)
        A.turns[i] = i < rope_dim / 2 ? std::pow(rope_base, -2.0 * i / rope_dim) / (2.0 * M_PI) : 0.0;
    auto log2_exact = [](int v) {
        int s = 0;
        while ((1 << s) < v) ++s;
        return (1 << s) == v ? s : -1;
    };
    A.cr_shift = log2_exact(cr);
    A.kpp_shift = log2_exact(A.kpp);
    const bool pow2 = A.cr_shift >= 0 && A.kpp_shift >= 0;
    const int64_t windows = ((int64_t)T + kNT - 1) / kNT;
    const int64_t grid = windows < (int64_t)cus * 8 ? windows : (int64_t)cus * 8;
    hipError_t e = mark(stream);
    if (e != hipSuccess) return e;
    if (pow2) compress_blocks_kernel<true><<<dim3((unsigned)grid), kNT, 0, stream>>>(A);
    else compress_blocks_kernel<false><<<dim3((unsigned)grid), kNT, 0, stream>>>(A);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(stream)) != hipSuccess || cr == 1) return e;
    stage_open_kernel<<<dim3((unsigned)windows), kNT, 0, stream>>>(A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(stream);
}

}  // namespace qsa
