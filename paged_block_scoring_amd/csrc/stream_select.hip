// stream_select.hip -- the streaming arm of qsa_select_paged_tokens, for
// batches with one row per request (decode): the score matrix is reduced to
// the rows' exact top-k on chip, chunk by chunk, so that it never reaches HBM.
//
// Sources: "qwen4_exp QSA cooperative_topk cannot launch on NVIDIA Thor
// (sm_110): cluster misconfiguration", section "What happens" (decode: one
// query row per request, each row streams its own keys; the score matrix is
// written and then re-read by a separate top-k op); "[Perf][Qwen4Exp] Admit
// the cuBLAS QSA indexer and exact top-k on Turing", sections "Purpose"
// (FP16 product with FP32 accumulation; the exact selector: higher score
// first, lower index on ties) and "Test Plan" (4 index heads, head dim 128).
//
// Two kernels.
//  1. Chunks: workgroup (row r, chunk c) -- 4 waves, several per compute unit --
//     scores keys c*C .. c*C+C-1 of row r (C = 8,192).  Its keys are cut into
//     segments of seg_len = min(512, 62 * keys per page) keys, so that a
//     segment spans at most 64 pages; wave w takes segments w, w + 4, ...
//     A wave reads a segment's page ids one per lane and scores 32-key tiles
//     with the next tile's loads in flight, with the windowed scorer's MFMA
//     chain, operands and order (score_group.hip), so the scores are the same
//     bits.  Lanes 0..31 then hold the chain
//     results of keys j0 + lane (default form: the score over the head-sum
//     factor f, a power of two, which ranks keys exactly as the score does).
//     Every key's order key goes to LDS at its place in the chunk; the
//     workgroup then holds the chunk in registers and selects its exact top
//     kb composites (order key, inverted index) -- distinct for distinct
//     keys, larger for the key that ranks first -- with select_top below, and
//     writes them in rank order to its slot of the workspace.  Chunks past
//     the row's visible keys exit.
//  2. Merge: one workgroup per row selects the min(kb, V) largest of its
//     chunks' lists the same way (or, for rows whose lists exceed the
//     registers, by repeated radix cuts in LDS) and writes them in rank
//     order.  The row's top kb lie in the union of its chunks' top kb, so the
//     result is exact.  Every chunk but a row's last holds 8,192 >= kb keys,
//     so a row's lists lie end to end in the workspace.
// The dispatcher hands chunks to compute units as they free up, so rows of
// different lengths share the chip evenly; a chunk writes kb composites
// (8 bytes) where the two-pass arm writes a score (4 bytes) per key.  On
// decode batches the arm runs level with the two-pass arm -- the score
// write it saves is a small share of the key reads -- and behind it on small
// batches, where a chunk's granularity leaves a longer tail; the library
// takes it only when forced.
#include <algorithm>

#include "qsa.h"
#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "qsa_select.hpp"

namespace qsa {
namespace {

constexpr int kStNT = 256;
constexpr int kStWaves = kStNT / 64;
constexpr int kStMaxSeg = 512;    // keys per segment at most
constexpr int kStChunk = 8192;    // keys per chunk
constexpr int kMgNT = 512;
constexpr int kMgBuf = 2 * QSA_MAX_SELECT;  // merge: after a cut to kb there is room for one more list

struct ChunkArgs {
    PagedArgs a;
    int32_t kb;
    int32_t seg_len;    // keys per segment (<= kStMaxSeg, spanning <= 64 pages)
    int32_t chunk;      // keys per chunk (kStChunk)
    int32_t nchunk;     // chunk slots per row: ceil(max_visible / chunk)
    int32_t kpp_shift;  // log2(kpp), or -1
    uint64_t* list;     // [rows][nchunk][kb] chunk top-kb composites (unsorted)
    int32_t* count;     // [rows][nchunk] entries of each list
};

// Keys a register select compacts at most: the largest kb (QSA_MAX_SELECT),
// so that a cut at a smaller kb fits unless many keys crowd around it.
constexpr int kTopCompact = QSA_MAX_SELECT;

template <int KBMAX>
struct TopLds {
    BoundSelectLds<KBMAX> s;
    uint64_t c[kTopCompact];
    int nc;
};

// Exact top-nsel of register-resident keys: thread t holds k[e], element
// e*NT + t with index idx(e); 0 marks an empty slot, slots e*NT >= nmax are
// skipped, 1 <= nsel <= the nonempty keys.  One histogram level over the keys
// (kSelBins bins between the smallest and largest) bounds the nsel-th
// largest (and, if that bin is crowded, a second level inside it); the keys at
// or above the bound are compacted into LDS and ranked by select_from_bound
// (qsa_select.hpp), or, if more than kTopCompact survive (ties), the keys are
// selected by select_exact_sorted.  emit(r, c) is called once for each rank
// r < nsel.  Contains barriers.
template <int NT, int EPT, int KBMAX, class IdxF, class EmitF>
__device__ __forceinline__ void select_top(const uint32_t (&k)[EPT], IdxF idx, int nmax, int nsel, TopLds<KBMAX>& L,
                                           EmitF emit) {
    const auto key = [&](int e) { return k[e]; };
    uint32_t mn, mx;
    block_minmax_u32<NT, EPT>(key, nmax, &mn, &mx, &L.s.hs);
    const int shift1 = max(0, bit_length32(mx - mn) - kSelBits);
    int above, cnt;
    const uint32_t b = hist_level32<NT, EPT>(key, nmax, mn, shift1, 32, 0u, nsel, &L.s.hs, nullptr, &above, &cnt);
    uint32_t lo = mn + (b << shift1);
    int surv = above + cnt;  // keys >= lo
    if (surv > kTopCompact && shift1 > 0) {  // (block-uniform) a crowded bin (outliers stretch the range): split it
        const int ns = max(0, shift1 - kSelBits);
        int above2, cnt2;
        const uint32_t b2 = hist_level32<NT, EPT>(key, nmax, mn, ns, shift1, b, nsel - above, &L.s.hs, nullptr,
                                                  &above2, &cnt2);
        lo += b2 << ns;
        surv = above + above2 + cnt2;
    }
    if (surv > kTopCompact) {  // (block-uniform)
        select_exact_sorted<NT, EPT, KBMAX>(key, idx, nmax, nsel, L.s, emit);
        return;
    }
    if (threadIdx.x == 0) L.nc = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const bool p = e * NT < nmax && k[e] >= lo;
        const uint64_t mk = __builtin_amdgcn_ballot_w64(p);
        if (mk) {  // (wave-uniform)
            int at = 0;
            if (lane == 0) at = atomicAdd(&L.nc, (int)__popcll(mk));
            at = __builtin_amdgcn_readfirstlane(at);
            if (p) L.c[at + (int)__popcll(mk & below)] = compose(k[e], idx(e));
        }
    }
    __syncthreads();
    constexpr int E2 = kTopCompact / NT;
    uint32_t k2[E2], i2[E2];
#pragma unroll
    for (int e = 0; e < E2; ++e) {
        const int p = e * NT + (int)threadIdx.x;
        const uint64_t ce = p < surv ? L.c[p] : 0ull;
        k2[e] = (uint32_t)(ce >> 32);
        i2[e] = composite_index(ce);
    }
    select_from_bound<NT, E2, KBMAX>(k2, [&](int e) { return i2[e]; }, surv, nsel, lo, L.s, emit);
}

// LDS of the chunk kernel: the chunk's order keys while it is scored, then
// the selection's scratch.
template <int KBMAX>
union ChunkLds {
    struct {
        uint32_t key[kStChunk];
        float stage[kStWaves][32];  // default form: a tile's 32 chain results
    } sc;
    TopLds<KBMAX> sel;
};

// Key of a 32-key tile loaded by MFMA row m in the default form (so that
// accumulator element v of lane l is the chain result of key 16*(l/32) + v);
// the relu form loads key m.
__device__ __forceinline__ int st_sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// The row's request and visible keys (a row of no valid request sees none).
__device__ __forceinline__ int st_row_visible(const PagedArgs& a, int row, int* req_out) {
    int req = a.row_req ? a.row_req[row] : 0;
    int V = 0;
    if (req >= 0 && req < a.num_reqs) V = visible_keys(a.pos[row], a.cr, a.max_visible);
    else req = 0;
    *req_out = __builtin_amdgcn_readfirstlane(req);
    return __builtin_amdgcn_readfirstlane(V);
}

template <bool RELU, bool POW2, int KBMAX>
__global__ __launch_bounds__(kStNT, 2) void stream_chunk_kernel(ChunkArgs A) {
    __shared__ ChunkLds<KBMAX> L;
    const PagedArgs& a = A.a;
    const int row = blockIdx.x / A.nchunk, ch = blockIdx.x - row * A.nchunk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 31, g = lane >> 5;
    int req;
    const int V = st_row_visible(a, row, &req);
    const int c0 = ch * A.chunk;
    if (c0 >= V) return;  // (block-uniform) the merge reads only the chunks below V
    const int c1 = min(c0 + A.chunk, V);

    // query fragments: the B operand column 0 (default form: the row's head
    // sum as an fp16 hi/lo pair, scaled by 1/f) or the A operand rows 0..3
    // (relu form: the row's four heads); zero elsewhere
    half8 qa[2 * kSlices];
    if (RELU) {
        const _Float16* qp = a.q + ((int64_t)row * kHeads + (m & 3)) * kHeadDim + 8 * g;
#pragma unroll
        for (int s = 0; s < kSlices; ++s) {
            const half8 v = *reinterpret_cast<const half8*>(qp + 16 * s);
            qa[s] = m < kHeads ? v : half8{};
        }
    } else {
        const _Float16* qp = a.q + (int64_t)row * kHeads * kHeadDim + 8 * g;
        auto load = [&](int s, int hh) { return *reinterpret_cast<const half8*>(qp + hh * kHeadDim + 16 * s); };
        float um = 0.0f;
#pragma unroll
        for (int s = 0; s < kSlices; ++s) um = fmaxf(um, head_sum_absmax(load(s, 0), load(s, 1), load(s, 2), load(s, 3)));
        um = fmaxf(um, __shfl_xor(um, 32, 64));
        const float inv_f = 1.0f / head_sum_factor(um);
#pragma unroll
        for (int s = 0; s < kSlices; ++s) {
            half8 hi, lo;
            head_sum_split(load(s, 0), load(s, 1), load(s, 2), load(s, 3), inv_f, hi, lo);
            qa[2 * s] = m == 0 ? hi : half8{};
            qa[2 * s + 1] = m == 0 ? lo : half8{};
        }
    }

    const int32_t* ptrow = a.page_table + (int64_t)req * a.pt_stride;
    const int mkey = RELU ? m : st_sigma(m);
    const int seg_len = A.seg_len;

    const int nsegs = (c1 - c0 + seg_len - 1) / seg_len;
    for (int sg = wave; sg < nsegs; sg += kStWaves) {  // (wave-uniform)
        const int k0 = c0 + sg * seg_len;
        const int k1 = min(k0 + seg_len, c1);
        const int pbase = POW2 ? (k0 >> A.kpp_shift) : k0 / a.kpp;
        const int plast = POW2 ? ((k1 - 1) >> A.kpp_shift) : (k1 - 1) / a.kpp;
        const int my_pg = min(max(ptrow[min(pbase + lane, plast)], 0), a.num_pages - 1);
        // lane l loads its eight 16-byte key pieces (tiles past the segment
        // load its last key)
        auto load_tile = [&](int j0, half8 (&kf)[kSlices]) {
            const int j = min(j0 + mkey, k1 - 1);
            const int lp = POW2 ? (j >> A.kpp_shift) : j / a.kpp;
            const int slot = j - lp * a.kpp;
            const int pg = __shfl(my_pg, lp - pbase, 64);
            const _Float16* key = a.kcache + ((int64_t)pg * a.kpp + slot) * kHeadDim + 8 * g;
#pragma unroll
            for (int s = 0; s < kSlices; ++s) kf[s] = *reinterpret_cast<const half8*>(key + 16 * s);
        };
        // one tile: lanes 0..31 take the result of key j0 + lane and store its
        // order key at the key's place in the chunk
        auto tile = [&](int j0, const half8 (&kf)[kSlices]) {
            float16v acc = {};
            float x;
            if (RELU) {
#pragma unroll
                for (int s = 0; s < kSlices; ++s) acc = mfma32(qa[s], kf[s], acc);
                x = combine_relu_heads(acc[0], acc[1], acc[2], acc[3]);
            } else {
#pragma unroll
                for (int s = 0; s < kSlices; ++s) {
                    acc = mfma32(kf[s], qa[2 * s], acc);
                    acc = mfma32(kf[s], qa[2 * s + 1], acc);
                }
                float* st = L.sc.stage[wave];
                if (m == 0) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) st[16 * g + v] = acc[v];
                }
                __builtin_amdgcn_wave_barrier();
                x = st[m];
                __builtin_amdgcn_wave_barrier();
            }
            const int j = j0 + m;
            if (g == 0 && j < k1) L.sc.key[j - c0] = order_key(x);
        };
        half8 b0[kSlices], b1[kSlices];
        load_tile(k0, b0);
        __builtin_amdgcn_sched_barrier(0);
        load_tile(k0 + 32, b1);
        __builtin_amdgcn_sched_barrier(0);
        int j0 = k0;
        for (; j0 + 32 < k1; j0 += 64) {
            tile(j0, b0);
            __builtin_amdgcn_sched_barrier(0);
            load_tile(j0 + 64, b0);
            __builtin_amdgcn_sched_barrier(0);
            tile(j0 + 32, b1);
            __builtin_amdgcn_sched_barrier(0);
            load_tile(j0 + 96, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (j0 < k1) tile(j0, b0);
    }
    __syncthreads();
    // the chunk's top min(kb, n) composites, in rank order
    const int n = c1 - c0;
    constexpr int EPT = kStChunk / kStNT;
    uint32_t k[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int p = e * kStNT + tid;
        k[e] = p < n ? L.sc.key[p] : 0u;
    }
    __syncthreads();  // (the selection reuses the LDS)
    const int64_t slot = (int64_t)row * A.nchunk + ch;
    uint64_t* dst = A.list + slot * A.kb;
    const int nsel = min(A.kb, n);
    select_top<kStNT, EPT, KBMAX>(k, [&](int e) { return (uint32_t)(c0 + e * kStNT + tid); }, n, nsel, L.sel,
                                  [&](int r, uint64_t c) { dst[r] = c; });
    if (tid == 0) A.count[slot] = nsel;
}

struct MergeArgs {
    PagedArgs a;
    int32_t kb, expand, out_len, chunk, nchunk;
    const uint64_t* list;
    const int32_t* count;
    int32_t* out;
};

constexpr int kMgEPT = 48;  // merge in registers: up to 24,576 list entries per row

template <int KBMAX>
union MergeLds {
    TopLds<KBMAX> top;
    struct {
        uint64_t buf[kMgBuf];
        uint64_t keep[QSA_MAX_SELECT];
        KthScratch ks;
        int nkeep;
    } it;
};

// Keeps the `keepn` largest of the n distinct composites buf[0 .. n) (n >
// keepn) at the front.  Contains barriers.
template <class ItLds>
__device__ __forceinline__ void keep_largest(ItLds& L, int n, int keepn) {
    const uint64_t cut = lds_kth_largest<kMgNT>(L.buf, n, keepn, &L.ks);
    if (threadIdx.x == 0) L.nkeep = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kMgNT) {
        const uint64_t v = L.buf[i];
        if (v >= cut) L.keep[atomicAdd(&L.nkeep, 1)] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < keepn; i += kMgNT) L.buf[i] = L.keep[i];
    __syncthreads();
}

template <int KBMAX>
__global__ __launch_bounds__(kMgNT) void stream_merge_kernel(MergeArgs A) {
    __shared__ MergeLds<KBMAX> L;
    const int row = blockIdx.x, tid = threadIdx.x;
    int req;
    const int V = st_row_visible(A.a, row, &req);
    const int nsel = min(A.kb, V);
    int32_t* orow = A.out + (int64_t)row * A.out_len;
    const bool vec4 = A.expand == 4 && (A.out_len & 3) == 0 && (reinterpret_cast<uintptr_t>(A.out) & 15) == 0;
    if (nsel > 0) {  // (block-uniform)
        const int parts = (V + A.chunk - 1) / A.chunk;
        // every list but the last holds exactly kb entries
        const uint64_t* lst = A.list + (int64_t)row * A.nchunk * A.kb;
        const int total = (parts - 1) * A.kb + min(max(A.count[(int64_t)row * A.nchunk + parts - 1], 0), A.kb);
        if (total <= kMgNT * kMgEPT) {
            uint32_t k[kMgEPT], ix[kMgEPT];
#pragma unroll
            for (int e = 0; e < kMgEPT; ++e) {
                const int p = e * kMgNT + tid;
                const uint64_t c = p < total ? lst[p] : 0ull;
                k[e] = (uint32_t)(c >> 32);
                ix[e] = composite_index(c);
            }
            select_top<kMgNT, kMgEPT, KBMAX>(k, [&](int e) { return ix[e]; }, total, nsel, L.top,
                                             [&](int r, uint64_t c) {
                                                 write_rank(orow, r, composite_index(c), A.expand, vec4);
                                             });
        } else {
            // lists beyond the registers: repeated radix cuts in LDS
            int n = 0;  // entries in buf (block-uniform)
            for (int p = 0; p < parts; ++p) {
                const int c = p + 1 < parts ? A.kb : total - (parts - 1) * A.kb;
                if (n + c > kMgBuf) {  // (then n > kb: a cut to kb leaves room for c <= kb)
                    __syncthreads();
                    keep_largest(L.it, n, A.kb);
                    n = A.kb;
                }
                const uint64_t* src = lst + (int64_t)p * A.kb;
                for (int i = tid; i < c; i += kMgNT) L.it.buf[n + i] = src[i];
                n += c;
            }
            __syncthreads();
            if (n > nsel) keep_largest(L.it, n, nsel);
            lds_sort_desc<kMgNT>(L.it.buf, nsel);
            for (int r = tid; r < nsel; r += kMgNT)
                write_rank(orow, r, composite_index(L.it.buf[r]), A.expand, vec4);
        }
    }
    for (int i = max(nsel, 0) * A.expand + tid; i < A.out_len; i += kMgNT) orow[i] = -1;
}

// Keys per segment: at most 62 pages' worth, so that a segment starting
// anywhere in a page spans at most 64 pages.
int32_t stream_seg_len(int32_t kpp) {
    return kpp < 1 ? 0 : (int32_t)std::min<int64_t>(kStMaxSeg, 62 * (int64_t)kpp);
}

}  // namespace

size_t stream_bytes(int32_t rows, int32_t max_visible, int32_t kb) {
    if (rows <= 0 || max_visible <= 0 || kb < 1) return 0;
    const int64_t nchunk = (max_visible + kStChunk - 1) / kStChunk;
    const size_t lists = (size_t)rows * (size_t)nchunk * (size_t)kb * sizeof(uint64_t);
    return ((lists + 255) & ~(size_t)255) + (size_t)rows * (size_t)nchunk * sizeof(int32_t);
}

hipError_t launch_stream_select(const PagedArgs& a, int32_t kb, int32_t expand, int32_t out_len, int32_t* out,
                                void* workspace, hipStream_t stream, hipError_t (*mark)(hipStream_t)) {
    if (a.rows <= 0) return hipSuccess;
    if (kb < 1 || kb > QSA_MAX_SELECT || a.kpp < 1) return hipErrorInvalidValue;
    ChunkArgs C;
    C.a = a;
    C.kb = kb;
    C.seg_len = stream_seg_len(a.kpp);
    C.chunk = kStChunk;
    C.nchunk = a.max_visible > 0 ? (a.max_visible + C.chunk - 1) / C.chunk : 1;
    C.kpp_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == a.kpp) C.kpp_shift = sh;
    const size_t lists = (size_t)a.rows * (size_t)C.nchunk * (size_t)kb * sizeof(uint64_t);
    C.list = static_cast<uint64_t*>(workspace);
    C.count = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) + ((lists + 255) & ~(size_t)255));
    hipError_t e;
    if (a.max_visible > 0) {
        const dim3 grid((unsigned)((int64_t)a.rows * C.nchunk));
        if (kb <= 1024) {
            if (a.relu) {
                if (C.kpp_shift >= 0) stream_chunk_kernel<true, true, 1024><<<grid, kStNT, 0, stream>>>(C);
                else stream_chunk_kernel<true, false, 1024><<<grid, kStNT, 0, stream>>>(C);
            } else {
                if (C.kpp_shift >= 0) stream_chunk_kernel<false, true, 1024><<<grid, kStNT, 0, stream>>>(C);
                else stream_chunk_kernel<false, false, 1024><<<grid, kStNT, 0, stream>>>(C);
            }
        } else {
            if (a.relu) {
                if (C.kpp_shift >= 0) stream_chunk_kernel<true, true, QSA_MAX_SELECT><<<grid, kStNT, 0, stream>>>(C);
                else stream_chunk_kernel<true, false, QSA_MAX_SELECT><<<grid, kStNT, 0, stream>>>(C);
            } else {
                if (C.kpp_shift >= 0) stream_chunk_kernel<false, true, QSA_MAX_SELECT><<<grid, kStNT, 0, stream>>>(C);
                else stream_chunk_kernel<false, false, QSA_MAX_SELECT><<<grid, kStNT, 0, stream>>>(C);
            }
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(stream)) != hipSuccess) return e;
    MergeArgs M;
    M.a = a;
    M.kb = kb;
    M.expand = expand;
    M.out_len = out_len;
    M.chunk = C.chunk;
    M.nchunk = C.nchunk;
    M.list = C.list;
    M.count = C.count;
    M.out = out;
    if (kb <= 1024)
        stream_merge_kernel<1024><<<dim3((unsigned)a.rows), kMgNT, 0, stream>>>(M);
    else
        stream_merge_kernel<QSA_MAX_SELECT><<<dim3((unsigned)a.rows), kMgNT, 0, stream>>>(M);
    return hipGetLastError();
}

}  // namespace qsa
