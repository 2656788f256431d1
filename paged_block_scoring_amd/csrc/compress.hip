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
//   compress_blocks_kernel -- one 16-lane group per closing token: gathers the
//     block's cr keys (16 bytes per lane per key, one 256-byte key per group),
//     mean in fp32, RMSNorm (sum of squares over the group by lane exchange),
//     RoPE (partner values by lane exchange; each angle reduced modulo 2 pi in
//     fp64 so that positions near 2^31 keep full fp32 accuracy), rounds to
//     fp16 and writes the key's slot of its page;
//   stage_open_kernel      -- copies the keys of tokens whose block stays open
//     at the end of the call into the staging state.
// The second launch may overwrite staging slots the first one reads (a run
// that finishes one block and leaves a later one open), hence two launches on
// one stream rather than one.
#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

#include <math.h>

namespace qsa {
namespace {

constexpr int kD = 128;           // key length
constexpr int kNT = 256;          // threads per workgroup
constexpr int kGroups = kNT / 16; // 16-lane groups per workgroup: one key each

typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

struct CompressArgs {
    const _Float16* k_tok;     // [T][128]
    const int32_t* tok_req;    // [T] or null (request 0)
    const int32_t* tok_pos;    // [T]
    int32_t T;
    const float* norm_w;       // [128] or null (weight 1)
    float eps;
    int32_t rope_dim;          // multiple of 16, <= 128
    double rope_base;
    bool interleaved;
    _Float16* state;           // [num_reqs][cr][128]
    _Float16* kcache;          // [num_pages][kpp][128]
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t num_pages;
    int32_t num_reqs;
    int32_t cr;
    int32_t kpp;
};

__device__ __forceinline__ int32_t req_of(const CompressArgs& A, int32_t t) {
    return A.tok_req ? A.tok_req[t] : 0;
}

// True when token slot s of this call holds (request q, position p).
__device__ __forceinline__ bool holds(const CompressArgs& A, int64_t s, int32_t q, int64_t p) {
    return s >= 0 && s < A.T && req_of(A, (int32_t)s) == q && (int64_t)A.tok_pos[s] == p;
}

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

// cos and sin of p0 * invf: the product and its reduction modulo 2 pi in fp64
// (2 pi split in two parts, Cody and Waite's method), the small remainder's
// cos and sin in fp32.
__device__ __forceinline__ void angle(double p0, double invf, float* c, float* s) {
    constexpr double kInv2Pi = 0.15915494309189535;
    constexpr double k2PiHi = 6.283185307179586;
    constexpr double k2PiLo = 2.4492935982947064e-16;
    const double a = p0 * invf;
    const double k = rint(a * kInv2Pi);
    double r = fma(-k, k2PiHi, a);
    r = fma(-k, k2PiLo, r);
    sincosf((float)r, s, c);
}

__global__ __launch_bounds__(kNT) void compress_blocks_kernel(CompressArgs A) {
    const int lane16 = threadIdx.x & 15;
    const int d0 = lane16 * 8;                      // this lane's 8 values
    const int half = A.rope_dim / 2;
    const bool in_rope = d0 < A.rope_dim;
    const bool first_half = d0 < half;
    // rotate-half partner lane (values d0 .. d0+7 pair with d0 +- half; half is
    // a multiple of 8, so the partner holds the same element positions)
    const int partner = !in_rope || A.interleaved ? lane16 : (first_half ? lane16 + half / 8 : lane16 - half / 8);

    // per-lane inverse frequencies, fixed for the launch
    double invf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int i;
        if (A.interleaved) i = (d0 + e) >> 1;
        else i = first_half ? d0 + e : d0 + e - half;
        invf[e] = in_rope ? pow(A.rope_base, -2.0 * (double)i / (double)A.rope_dim) : 0.0;
    }
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = A.norm_w ? A.norm_w[d0 + e] : 1.0f;
    const float inv_cr = 1.0f / (float)A.cr;

    const int64_t step = (int64_t)gridDim.x * kGroups;
    for (int64_t t = (int64_t)blockIdx.x * kGroups + (threadIdx.x >> 4); t < A.T; t += step) {
        const int32_t p = A.tok_pos[t];
        const int32_t q = req_of(A, (int32_t)t);
        if (p < 0 || q < 0 || q >= A.num_reqs || ((int64_t)p + 1) % A.cr != 0) continue;
        const int32_t c = p / A.cr;                  // block index
        const int64_t lp = c / A.kpp;                // logical page
        if (lp >= A.pt_stride) continue;
        int32_t page = A.page_table[(int64_t)q * A.pt_stride + lp];
        page = min(max(page, 0), A.num_pages - 1);
        const int32_t p0 = c * A.cr;

        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        for (int i = 0; i < A.cr; ++i) {
            const int64_t s = t - (A.cr - 1 - i);
            const _Float16* src = holds(A, s, q, p0 + i) ? A.k_tok + s * kD
                                                         : A.state + ((int64_t)q * A.cr + i) * kD;
            float f[8];
            unpack8(*reinterpret_cast<const u32x4a*>(src + d0), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += f[e];
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

        float o[8];
        if (A.interleaved) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                float cs, sn;
                angle((double)p0, invf[e], &cs, &sn);
                if (!in_rope) { cs = 1.0f; sn = 0.0f; }
                o[e] = y[e] * cs - y[e + 1] * sn;
                o[e + 1] = y[e + 1] * cs + y[e] * sn;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = __shfl(y[e], partner, 16);
                float cs, sn;
                angle((double)p0, invf[e], &cs, &sn);
                if (!in_rope) { cs = 1.0f; sn = 0.0f; }
                o[e] = first_half ? y[e] * cs - pv * sn : y[e] * cs + pv * sn;
            }
        }
        *reinterpret_cast<u32x4a*>(A.kcache + ((int64_t)page * A.kpp + c % A.kpp) * kD + d0) = pack8(o);
    }
}

// One thread per 16-byte piece of a token key: tokens whose block has no
// closing token in this call go to the staging state.
__global__ __launch_bounds__(kNT) void stage_open_kernel(CompressArgs A) {
    const int64_t g = (int64_t)blockIdx.x * kNT + threadIdx.x;
    const int64_t t = g >> 4;
    if (t >= A.T) return;
    const int32_t p = A.tok_pos[t];
    const int32_t q = req_of(A, (int32_t)t);
    if (p < 0 || q < 0 || q >= A.num_reqs) return;
    const int32_t slot = p % A.cr;
    const int64_t end = (int64_t)p + (A.cr - 1 - slot);
    if (holds(A, t + (A.cr - 1 - slot), q, end)) return;   // finished in this call
    const int d0 = (int)(g & 15) * 8;
    *reinterpret_cast<u32x4a*>(A.state + ((int64_t)q * A.cr + slot) * kD + d0) =
        *reinterpret_cast<const u32x4a*>(A.k_tok + t * kD + d0);
}

}  // namespace

hipError_t launch_compress(const _Float16* k_tok, const int32_t* tok_req, const int32_t* tok_pos, int32_t T,
                           const float* norm_w, float eps, int32_t rope_dim, double rope_base, bool interleaved,
                           _Float16* state, _Float16* kcache, const int32_t* page_table, int64_t pt_stride,
                           int32_t num_pages, int32_t num_reqs, int32_t page_size, int32_t cr, int32_t cus,
                           hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    CompressArgs A;
    A.k_tok = k_tok;
    A.tok_req = tok_req;
    A.tok_pos = tok_pos;
    A.T = T;
    A.norm_w = norm_w;
    A.eps = eps;
    A.rope_dim = rope_dim;
    A.rope_base = rope_base;
    A.interleaved = interleaved;
    A.state = state;
    A.kcache = kcache;
    A.page_table = page_table;
    A.pt_stride = pt_stride;
    A.num_pages = num_pages;
    A.num_reqs = num_reqs;
    A.cr = cr;
    A.kpp = page_size / cr;
    const int64_t items = ((int64_t)T + kGroups - 1) / kGroups;
    const int64_t grid = items < (int64_t)cus * 16 ? items : (int64_t)cus * 16;
    compress_blocks_kernel<<<dim3((unsigned)grid), kNT, 0, stream>>>(A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || cr == 1) return e;
    const int64_t pieces = (int64_t)T * 16;
    stage_open_kernel<<<dim3((unsigned)((pieces + kNT - 1) / kNT)), kNT, 0, stream>>>(A);
    return hipGetLastError();
}

}  // namespace qsa
