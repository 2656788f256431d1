// attend.hip -- the sparse-attention consumer of the indexer's selection:
// softmax attention of every query head over the raw tokens the indexer
// selected, gathered from the paged main KV cache.
//
// Sources: "spec(MODEL-MM-QWEN4-EXP): Qwen3.8-Flash-Next is a new architecture
// ...": the model's attention is plain GQA, 24 query heads over 2 KV heads,
// head_dim 256 (the op-survey paragraph on QSA's twin), and its consumer
// attends to the raw tokens selected at ratio-4 granularity (section "The
// component deep-dives, and two corrections to the above").  Readings where
// the pages are silent: scale 1/sqrt(head_dim) (the caller passes it), exactly
// the listed tokens (entries < 0 are padding; a row with none yields zeros),
// query head h reads KV head h / (q_heads / kv_heads), and the main cache is
// paged like the index cache: token t of a request at slot t % page_size of
// page page_table[req][t / page_size], K and V each [page][slot][kv_head][256].
//
// One workgroup per (row, KV head): the group's query heads (at most 16) are
// the 16 columns of 16x16 MFMA tiles.  The token list is walked in chunks of
// 64; K and V rows of a chunk are gathered through the page table into LDS
// (the next chunk's loads are in flight while the current one is used), and
// wave w takes tokens 16w .. 16w+15 of each chunk:
//   S^T = K . Q^T   -- v_mfma_f32_16x16x32_f16, keys as rows, heads as
//                      columns; lane l then holds 4 tokens of head l%16;
//   online softmax  -- per head (lane-local, plus two lane exchanges), in fp32;
//   O^T += V^T . P^T -- v_mfma_f32_16x16x16_f16: P^T's operand layout is
//                      exactly S^T's result layout, so P never leaves the
//                      lanes; V^T's fragments are read from the chunk's rows.
// Each wave thus keeps its own running max, sum and output for its tokens;
// the four are merged at the end (the same rescaling as between chunks).
// With fewer than 512 (row, KV head) pairs, each pair's list is cut into up
// to 16 spans of at least 128 entries, one workgroup each; a span leaves its
// merged state (max, sum, unnormalised output) in the caller's workspace and
// attend_merge_kernel combines the spans with the same rescaling.
#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

#include <algorithm>

namespace qsa {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));

constexpr int kD = 256;          // head_dim
constexpr int kNT = 256;         // 4 waves
constexpr int kCh = 64;          // tokens per chunk (16 per wave)
constexpr int kWin = 2048;       // list entries whose rows are staged at once
constexpr int kRow = kD + 8;     // LDS row of a K or V vector, in halves (padded against bank conflicts)
constexpr int kPieces = kCh * kD / 8 / kNT;  // 16-byte pieces per thread per chunk, K or V
constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr int kMaxSplits = 16;   // workgroups per (row, KV head) at most

struct AttendArgs {
    const _Float16* q;      // [rows][q_heads][256]
    const _Float16* kc;     // [num_pages][page_size][kv_heads][256]
    const _Float16* vc;
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t num_pages, num_reqs;
    const int32_t* row_req;
    const int32_t* tokens;  // [rows][k]
    int32_t k, rows, q_heads, kv_heads, group, page_size;
    float scale;
    float* out;             // [rows][q_heads][256]
    int32_t splits;         // workgroups per (row, KV head), each over `span` list entries
    int32_t span;
    float* part;            // splits > 1: [rows * kv_heads * splits] partial records
};

// Partial result of one split of a (row, KV head): per head of the group its
// running max m (-inf when the split saw no token), its sum l of e^(s - m) and
// its unnormalised output sum_t e^(s_t - m) V_t.
struct AttendPart {
    float m[16];
    float l[16];
    float o[16 * kD];
};

struct AttendLds {
    union {
        struct {
            _Float16 k[kCh * kRow];
            _Float16 v[kCh * kRow];
        } kv;
        float o[4][16 * kD];  // the waves' outputs, merged at the end
    } u;
    uint32_t row[kWin];       // K/V row index of each staged list entry, or kNone
    float m[4][16], l[4][16];
    float mh[16], lh[16];  // merged max and sum per head
    int last;
};

__device__ __forceinline__ float4v mfma16x32(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma16x16(half4 a, half4 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kNT, 2) void attend_kernel(AttendArgs A) {
    __shared__ AttendLds L;
    const int split = blockIdx.x % A.splits, rk = blockIdx.x / A.splits;
    const int row = rk / A.kv_heads, kvh = rk - row * A.kv_heads;
    const int e_begin = split * A.span, e_end = min(A.k, e_begin + A.span);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, quad = lane >> 4;  // MFMA column (head) and lane group
    const int req = A.row_req ? A.row_req[row] : 0;
    const bool req_ok = req >= 0 && req < A.num_reqs;

    // query fragments (B operand of S^T = K . Q^T): head n of the group, dims
    // 32s + 8*quad .. +7; columns past the group are zero
    half8 qb[kD / 32];
    {
        const int h = kvh * A.group + n;
        const _Float16* qr = A.q + ((int64_t)row * A.q_heads + (n < A.group ? h : 0)) * kD + 8 * quad;
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) {
            const half8 v = *reinterpret_cast<const half8*>(qr + 32 * s);
            qb[s] = n < A.group ? v : half8{};
        }
    }
    float mrun = -__builtin_huge_valf(), lrun = 0.0f;  // of head n, over this wave's tokens
    float4v o[kD / 16];                                 // O^T tiles: dims 16t + 4*quad + i, head n
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) o[t] = float4v{};

    const int32_t* list = A.tokens + (int64_t)row * A.k;
    const int32_t* ptrow = A.page_table + (int64_t)(req_ok ? req : 0) * A.pt_stride;
    for (int w0 = e_begin; w0 < e_end; w0 += kWin) {
        const int wl = min(kWin, e_end - w0);
        // rows of this window's entries, and the last valid one
        if (tid == 0) L.last = -1;
        __syncthreads();
        int my_last = -1;
        for (int i = tid; i < wl; i += kNT) {
            const int t = list[w0 + i];
            uint32_t r = kNone;
            if (t >= 0 && req_ok) {
                const int64_t lp = min((int64_t)(t / A.page_size), A.pt_stride - 1);
                const int pg = min(max(ptrow[lp], 0), A.num_pages - 1);
                r = ((uint32_t)pg * (uint32_t)A.page_size + (uint32_t)(t % A.page_size)) * (uint32_t)A.kv_heads +
                    (uint32_t)kvh;
                my_last = i;
            }
            L.row[i] = r;
        }
        if (my_last >= 0) atomicMax(&L.last, my_last);
        __syncthreads();
        const int nch = (L.last + kCh) / kCh;  // chunks up to the last valid entry

        // this thread's pieces of a chunk: token p >> 5, 16-byte piece p & 31
        u32x4a pk[kPieces], pv[kPieces];
        auto issue = [&](int c) {
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                const int p = j * kNT + tid, i = c * kCh + (p >> 5);
                const uint32_t r = i < wl ? L.row[i] : kNone;
                const int64_t off = (int64_t)(r == kNone ? 0u : r) * kD + 8 * (p & 31);
                pk[j] = *reinterpret_cast<const u32x4a*>(A.kc + off);
                pv[j] = *reinterpret_cast<const u32x4a*>(A.vc + off);
            }
        };
        auto stage = [&]() {
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                const int p = j * kNT + tid;
                const int at = (p >> 5) * kRow + 8 * (p & 31);
                *reinterpret_cast<u32x4a*>(&L.u.kv.k[at]) = pk[j];
                *reinterpret_cast<u32x4a*>(&L.u.kv.v[at]) = pv[j];
            }
        };
        if (nch > 0) {
            issue(0);
            stage();
        }
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) issue(c + 1);
            // S^T for this wave's 16 tokens: lane holds tokens 4*quad + i of head n
            const int tb = 16 * wave;
            float4v s = {};
            const _Float16* kr = &L.u.kv.k[(tb + n) * kRow + 8 * quad];
#pragma unroll
            for (int sl = 0; sl < kD / 32; ++sl)
                s = mfma16x32(*reinterpret_cast<const half8*>(kr + 32 * sl), qb[sl], s);
            float sc[4];
            float cmax = -__builtin_huge_valf();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = c * kCh + tb + 4 * quad + i;
                const bool ok = e < wl && L.row[e] != kNone;
                sc[i] = ok ? s[i] * A.scale : -__builtin_huge_valf();
                cmax = fmaxf(cmax, sc[i]);
            }
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
            const float mnew = fmaxf(mrun, cmax);
            const float mref = mnew == -__builtin_huge_valf() ? 0.0f : mnew;  // no token yet: nothing to scale
            const float alpha = __expf(mrun - mref);
            half4 pb;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pi = __expf(sc[i] - mref);
                psum += pi;
                pb[i] = (_Float16)pi;
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            lrun = lrun * alpha + psum;
            mrun = mnew;
            // O^T = alpha * O^T + V^T . P^T; V^T fragment: dim 16t + n, tokens 4*quad .. +3
            const _Float16* vr = &L.u.kv.v[(tb + 4 * quad) * kRow + n];
#pragma unroll
            for (int t = 0; t < kD / 16; ++t) {
                half4 va;
#pragma unroll
                for (int i = 0; i < 4; ++i) va[i] = vr[i * kRow + 16 * t];
                o[t] = mfma16x16(va, pb, o[t] * alpha);
            }
            __syncthreads();  // every wave is done with this chunk
            if (c + 1 < nch) stage();
            __syncthreads();
        }
    }

    // merge the waves: per head, M = max m_w, Lsum = sum l_w e^(m_w - M),
    // out = sum O_w e^(m_w - M) / Lsum (a head with no token gets zeros)
    if (quad == 0) {
        L.m[wave][n] = mrun;
        L.l[wave][n] = lrun;
    }
    __syncthreads();
    if (tid < 16) {
        float mall = -__builtin_huge_valf();
#pragma unroll
        for (int w = 0; w < 4; ++w) mall = fmaxf(mall, L.m[w][tid]);
        const float mref = mall == -__builtin_huge_valf() ? 0.0f : mall;
        float lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) lsum += L.l[w][tid] * __expf(L.m[w][tid] - mref);
        L.mh[tid] = mref;
        L.lh[tid] = lsum;
    }
    __syncthreads();
    const float f = __expf(mrun - L.mh[n]);
#pragma unroll
    for (int t = 0; t < kD / 16; ++t)
        *reinterpret_cast<float4v*>(&L.u.o[wave][n * kD + 16 * t + 4 * quad]) = o[t] * f;
    __syncthreads();
    if (A.splits == 1) {
        for (int e = tid; e < A.group * kD; e += kNT) {
            const int h = e / kD, d = e - h * kD;
            const float acc = (L.u.o[0][e] + L.u.o[1][e]) + (L.u.o[2][e] + L.u.o[3][e]);
            const float lsum = L.lh[h];
            A.out[((int64_t)row * A.q_heads + kvh * A.group + h) * kD + d] = lsum > 0.0f ? acc / lsum : 0.0f;
        }
        return;
    }
    // a split leaves its partial record for attend_merge_kernel
    AttendPart* P = reinterpret_cast<AttendPart*>(A.part) + blockIdx.x;
    if (tid < 16) {
        P->m[tid] = L.lh[tid] > 0.0f ? L.mh[tid] : -__builtin_huge_valf();
        P->l[tid] = L.lh[tid];
    }
    for (int e = tid; e < A.group * kD; e += kNT)
        P->o[e] = (L.u.o[0][e] + L.u.o[1][e]) + (L.u.o[2][e] + L.u.o[3][e]);
}

// One workgroup per (row, query head), one thread per output value: the
// splits' partial results merged with the same rescaling as between waves
// (every split's values are requested before any is used).
__global__ __launch_bounds__(kD) void attend_merge_kernel(AttendArgs A) {
    const int row = blockIdx.x / A.q_heads, h = blockIdx.x - row * A.q_heads;
    const int kvh = h / A.group, hh = h - kvh * A.group, d = threadIdx.x;
    const AttendPart* P = reinterpret_cast<const AttendPart*>(A.part) + ((int64_t)row * A.kv_heads + kvh) * A.splits;
    float ms[kMaxSplits], ls[kMaxSplits], os[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        const bool in = s < A.splits;
        const AttendPart* Ps = P + (in ? s : 0);
        ms[s] = Ps->m[hh];
        ls[s] = Ps->l[hh];
        os[s] = Ps->o[hh * kD + d];
        if (!in) ms[s] = -__builtin_huge_valf();
    }
    float mall = -__builtin_huge_valf();
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) mall = fmaxf(mall, ms[s]);
    float lsum = 0.0f, acc = 0.0f;
    if (mall > -__builtin_huge_valf()) {
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            // a split that saw no token (or lies past the list) adds nothing
            const float f = ms[s] == -__builtin_huge_valf() ? 0.0f : __expf(ms[s] - mall);
            lsum += ls[s] * f;
            acc += os[s] * f;
        }
    }
    A.out[((int64_t)row * A.q_heads + h) * kD + d] = lsum > 0.0f ? acc / lsum : 0.0f;
}

}  // namespace

// Splits per (row, KV head): enough workgroups to give every compute unit
// two (512 in all) when the rows alone do not, with at least two chunks (128
// list entries) per split and at most 16 splits.  Depends on the arguments
// only.  (Finer splits measured slower: each workgroup's fixed costs and the
// merge outweigh the added parallelism.)
static void attend_split_plan(int32_t rows, int32_t kv_heads, int32_t k, int32_t* splits, int32_t* span) {
    const int64_t wgs = (int64_t)rows * kv_heads;
    int64_t s = wgs >= 512 ? 1 : (512 + wgs - 1) / wgs;
    s = std::min<int64_t>(std::min<int64_t>(s, kMaxSplits), std::max<int64_t>(1, k / (2 * kCh)));
    int64_t sp = (k + s - 1) / s;
    sp = (sp + kCh - 1) / kCh * kCh;
    *span = (int32_t)sp;
    *splits = (int32_t)((k + sp - 1) / sp);
}

size_t attend_workspace_bytes(int32_t rows, int32_t kv_heads, int32_t k) {
    if (rows <= 0 || kv_heads <= 0 || k <= 0) return 0;
    int32_t splits, span;
    attend_split_plan(rows, kv_heads, k, &splits, &span);
    return splits > 1 ? (size_t)rows * kv_heads * splits * sizeof(AttendPart) : 0;
}

hipError_t launch_attend(const _Float16* q, const _Float16* kc, const _Float16* vc, const int32_t* page_table,
                         int64_t pt_stride, int32_t num_pages, int32_t num_reqs, const int32_t* row_req,
                         const int32_t* tokens, int32_t k, int32_t rows, int32_t q_heads, int32_t kv_heads,
                         int32_t page_size, float scale, float* out, void* workspace, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    AttendArgs A;
    A.q = q;
    A.kc = kc;
    A.vc = vc;
    A.page_table = page_table;
    A.pt_stride = pt_stride;
    A.num_pages = num_pages;
    A.num_reqs = num_reqs;
    A.row_req = row_req;
    A.tokens = tokens;
    A.k = k;
    A.rows = rows;
    A.q_heads = q_heads;
    A.kv_heads = kv_heads;
    A.group = q_heads / kv_heads;
    A.page_size = page_size;
    A.scale = scale;
    A.out = out;
    attend_split_plan(rows, kv_heads, k, &A.splits, &A.span);
    A.part = static_cast<float*>(workspace);
    if (A.splits > 1 && workspace == nullptr) return hipErrorInvalidValue;
    attend_kernel<<<dim3((unsigned)((int64_t)rows * kv_heads * A.splits)), kNT, 0, stream>>>(A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || A.splits == 1) return e;
    attend_merge_kernel<<<dim3((unsigned)((int64_t)rows * q_heads)), kD, 0, stream>>>(A);
    return hipGetLastError();
}

}  // namespace qsa
