// score_group.hip -- the materialising scorer for calls with few query rows
// per request (decode: one row per request).
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", sections "Purpose" (FP16 product with FP32 accumulation; a paged
// scorer reading keys through the page table) and "Test Plan" (4 index heads,
// head dim 128, compress ratio 4); "qwen4_exp QSA cooperative_topk cannot
// launch on NVIDIA Thor (sm_110): cluster misconfiguration", section "What
// happens" (decode: one query row per request, so each row streams its own
// keys).
//
// Why a second scorer.  The tiled scorer shares every staged key among the
// 128 (or 64) rows of a tile, which is what a prefill chunk needs.  With one
// row per request each key is used by one row only: the work is a stream of
// the cache (256 bytes per key, HBM-bound) and a tile would hold rows of 128
// different requests.  Here every wave (a one-wave workgroup, so that waves
// are dispatched and retired independently) works alone on an item = (window
// of G consecutive rows, segment of about 1,024 keys -- shorter, down to 256,
// when there are few windows -- starting on a page boundary and spanning at
// most 64 pages), G chosen by the host from the rows per request; a window whose rows belong to several requests is done in one
// pass per request, as in the tiled scorer.  The page ids of a segment are
// read once, one per lane, and handed to the key loads by lane shuffles.
//
// A 32-key tile.  Each lane loads its MFMA key fragments straight from the
// cache into registers -- eight 16-byte pieces of one key, the ones the
// canonical arrangement (qsa_device.hpp) gives that lane -- while the tile
// before it is scored.  The chain, its operands and their order are exactly
// those of the tiled scorer, so both produce the same bits:
//   default form -- keys are the MFMA rows; lane l loads key sigma(l%32) of
//     the tile (sigma as in the tiled scorer), so that accumulator element v
//     of lane l is the score of window row l%32 and key 16*(l/32) + v;
//   relu form -- keys are the MFMA columns; lane l loads key l%32 and element
//     group i (elements 4i..4i+3) holds the four head dots of window row
//     2i + l/32 (windows of at most 8 rows).
// Scores collect in the wave's LDS buffer (1,024 per wave, rows of 1024/G
// keys) and leave it in whole-wave 16-byte stores: with one row per window a
// tile has just two lanes' worth of scores, and storing them directly would
// cost four nearly empty store instructions per tile.
//
// Memory-level parallelism.  vmcnt counts loads and stores in issue order, so
// the compiler's waits are exact only if (a) the loads of tile t are issued
// before those of tile t+1 (scheduling barriers), (b) no store is issued
// behind a prefetch (scores are buffered, and flushed, before the next loads)
// and (c) the loop has one exit and wave-uniform bounds (readfirstlane), so
// that every path into the loop head carries the same pending loads.  Then the
// wait for tile t leaves tile t+1 in flight.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

#include <algorithm>

namespace qsa {
namespace {

constexpr int kGroupNT = 64;
constexpr int kGroupWaves = kGroupNT / 64;
constexpr int kSeg = 1024;  // target keys per item
constexpr int kBufFloats = 1024;  // buffered scores per wave

struct GroupArgs {
    PagedArgs a;
    int32_t G;        // rows per window
    int32_t windows;  // ceil(rows / G)
    int32_t nseg;     // ceil(max_visible / seg_len)
    float* out;
    int64_t ld;
    int32_t vec_store;
    int32_t kpp_shift;  // log2(kpp), or -1
    int32_t seg_len;    // keys per item: a multiple of 32 and of kpp, spanning <= 64 pages
};

// Key of a 32-key tile loaded by MFMA row m in the default form (see the
// header comment); the relu form loads key m.
__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

template <bool RELU, bool POW2>
__global__ __launch_bounds__(kGroupNT, 2) void score_group_kernel(GroupArgs A) {
    const PagedArgs& a = A.a;
    const int lane = threadIdx.x & 63;
    // wave-uniform item (the compiler cannot see that tid/64 is uniform)
    const int64_t item = (int64_t)blockIdx.x * kGroupWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= (int64_t)A.windows * A.nseg) return;
    const int seg = (int)(item / A.windows);
    const int win = (int)(item - (int64_t)seg * A.windows);
    const int k0 = seg * A.seg_len;
    const int r0 = win * A.G;
    const int m = lane & 31, g = lane >> 5;
    __shared__ __attribute__((aligned(16))) float s_sc[kGroupWaves][kBufFloats + 4 * 32];

    // This lane's window row (column of the default form's MFMA): its request
    // and visible keys.  Rows beyond the window are inactive (req -1).
    const int c = m;
    int req_c = -1, v_c = 0;
    if (c < A.G && r0 + c < a.rows) {
        const int r = r0 + c;
        const int q = a.row_req ? a.row_req[r] : 0;
        if (q >= 0 && q < a.num_reqs) {
            req_c = q;
            v_c = visible_keys(a.pos[r], a.cr, a.max_visible);
        }
    }
    bool todo = req_c >= 0 && v_c > k0;
    half8 qa[2 * kSlices];
    float fac = 1.0f;  // head-sum factor of this lane's row (default form)

    for (;;) {
        // one pass per request among the window's pending rows, smallest first
        int act = todo ? req_c : 0x7FFFFFFF;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) act = min(act, __shfl_xor(act, o, 64));
        act = __builtin_amdgcn_readfirstlane(act);  // wave-uniform: scalar control flow below
        if (act == 0x7FFFFFFF) break;
        const bool on = todo && req_c == act;
        todo = todo && !on;
        const int lim_c = on ? v_c : 0;  // this column's key bound in this pass
        int vmax = lim_c;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) vmax = max(vmax, __shfl_xor(vmax, o, 64));
        vmax = __builtin_amdgcn_readfirstlane(vmax);
        const int k1 = min(k0 + A.seg_len, vmax);

        // query fragments of the active rows (zero elsewhere); inactive
        // lanes read row r0 (a valid row) and discard it
        if (RELU) {
            // A operand row m = 4 * (window row m/4) + head m%4; window row
            // m/4's activity is held by lane m/4
            const int rw = m >> 2;
            const bool row_on = __shfl(on ? 1 : 0, rw, 64) != 0;
            const _Float16* qp = a.q + ((int64_t)(row_on ? r0 + rw : r0) * kHeads + (m & 3)) * kHeadDim + 8 * g;
#pragma unroll
            for (int s = 0; s < kSlices; ++s) {
                const half8 v = *reinterpret_cast<const half8*>(qp + 16 * s);
                qa[s] = row_on ? v : half8{};
            }
        } else {
            const _Float16* qp = a.q + (int64_t)(on ? r0 + c : r0) * kHeads * kHeadDim + 8 * g;
            auto load = [&](int s, int hh) {
                const half8 v = *reinterpret_cast<const half8*>(qp + hh * kHeadDim + 16 * s);
                return on ? v : half8{};
            };
            // the row's head-sum factor (lanes l and l^32 hold its two halves)
            float um = 0.0f;
#pragma unroll
            for (int s = 0; s < kSlices; ++s) um = fmaxf(um, head_sum_absmax(load(s, 0), load(s, 1), load(s, 2), load(s, 3)));
            um = fmaxf(um, __shfl_xor(um, 32, 64));
            fac = head_sum_factor(um);
#pragma unroll
            for (int s = 0; s < kSlices; ++s)
                head_sum_split(load(s, 0), load(s, 1), load(s, 2), load(s, 3), 1.0f / fac, qa[2 * s], qa[2 * s + 1]);
        }

        const int32_t* ptrow = a.page_table + (int64_t)act * a.pt_stride;
        const int mkey = RELU ? m : sigma(m);
        // page ids of the segment's first 64 pages, page pbase + i in lane i
        const int pbase = k0 / a.kpp;  // segments start on a page boundary and span <= 64 pages
        const int plast = (k1 - 1) / a.kpp;
        const int my_pg = min(max(ptrow[min(pbase + lane, plast)], 0), a.num_pages - 1);
        // Each lane loads its MFMA key fragments: eight 16-byte pieces of
        // key sigma(m) (default form) or m (relu form) of the tile.
        auto load_tile = [&](int j0, half8 (&kf)[kSlices]) {
            const int j = min(j0 + mkey, k1 - 1);
            const int lp = POW2 ? (j >> A.kpp_shift) : j / a.kpp;
            const int slot = j - lp * a.kpp;
            const int pg = __shfl(my_pg, lp - pbase, 64);
            const _Float16* key = a.kcache + ((int64_t)pg * a.kpp + slot) * kHeadDim + 8 * g;
#pragma unroll
            for (int s = 0; s < kSlices; ++s) kf[s] = *reinterpret_cast<const half8*>(key + 16 * s);
        };
        auto chain = [&](const half8 (&kf)[kSlices]) {
            float16v acc = {};
#pragma unroll
            for (int s = 0; s < kSlices; ++s) {
                if (RELU) {
                    acc = mfma32(qa[s], kf[s], acc);
                } else {
                    acc = mfma32(kf[s], qa[2 * s], acc);
                    acc = mfma32(kf[s], qa[2 * s + 1], acc);
                }
            }
            return acc;
        };
        // Scores go to this wave's LDS buffer (rows of kbuf keys, padded by
        // 4 floats against bank conflicts) and leave it in whole-wave 16-byte
        // stores once kbuf keys of every row are in (or the item ends).
        const int kbuf = kBufFloats / A.G;  // keys per buffered row (a multiple of 32)
        const int rstride = kbuf + 4;
        float* const sb = s_sc[threadIdx.x >> 6];
        auto put = [&](int j0, int wbase, const float16v& acc) {
            const int off = j0 - wbase;
            if (RELU) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (2 * i + g < A.G)  // the buffer holds A.G rows
                        sb[(2 * i + g) * rstride + off + m] =
                            combine_relu_heads(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
            } else if (c < A.G) {
                // chain result x head-sum factor = score
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<float4v*>(sb + c * rstride + off + 16 * g + 4 * i) =
                        float4v{acc[4 * i] * fac, acc[4 * i + 1] * fac, acc[4 * i + 2] * fac, acc[4 * i + 3] * fac};
            }
        };
        auto flush = [&](int wbase) {
            const int q4n = kbuf >> 2;  // float4s per buffered row
#pragma unroll
            for (int i = 0; i < kBufFloats / 256; ++i) {
                const int f = 64 * i + lane;
                const int row = f / q4n, q4 = f - row * q4n;
                // the row's bound, and the item's end: a segment shorter than
                // the buffer leaves the buffer's tail unwritten
                const int lim = min(__shfl(lim_c, row & 31, 64), k1);
                const int key = wbase + 4 * q4;
                if (row < A.G && key < lim) {
                    const float4v v = *reinterpret_cast<const float4v*>(sb + row * rstride + 4 * q4);
                    float* dst = A.out + (int64_t)(r0 + row) * A.ld + key;
                    if (key + 4 <= lim && A.vec_store) {
                        *reinterpret_cast<float4v*>(dst) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (key + e < lim) dst[e] = v[e];
                    }
                }
            }
        };
        // the tile at j0 is done: buffer it, flush a full buffer
        int wbase = k0;
        auto store = [&](int j0, const float16v& acc) {
            put(j0, wbase, acc);
            if (j0 + 32 - wbase == kbuf) {
                flush(wbase);
                wbase += kbuf;
            }
        };
        // Tile t+1 (and t+2 in the relu form) is in flight while tile t is
        // scored; a tile's scores are buffered (and possibly flushed) before
        // the next loads are issued,
        // so that no wait for a tile can drain the loads behind it.  The loop
        // has a single exit so that the waits are the same on every path.
        // Tiles past the segment load its last key.
        // (the relu form keeps two tiles in flight: it runs at two waves per
        // SIMD with three buffers as at three with two, and streams faster)
        constexpr int NB = RELU ? 3 : 2;
        half8 b[NB][kSlices];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            load_tile(k0 + 32 * i, b[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
        int j0 = k0;
        for (; j0 + 32 * (NB - 1) < k1; j0 += 32 * NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const float16v acc = chain(b[i]);
                __builtin_amdgcn_sched_barrier(0);
                store(j0 + 32 * i, acc);
                __builtin_amdgcn_sched_barrier(0);
                load_tile(j0 + 32 * (NB + i), b[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last tiles (fewer than NB), already loaded in order
#pragma unroll
        for (int i = 0; i < NB - 1; ++i) {
            if (j0 < k1) {
                const float16v acc = chain(b[i]);
                store(j0, acc);
                j0 += 32;
            }
        }
        if (j0 != wbase) flush(wbase);
    }
}

}  // namespace

int32_t group_rows_for(int32_t rows, int32_t num_reqs, bool relu) {
    const int32_t per = (rows + (num_reqs > 0 ? num_reqs : 1) - 1) / (num_reqs > 0 ? num_reqs : 1);
    int32_t G = 1;
    while (G < per) G <<= 1;
    const int32_t cap = relu ? 8 : 32;
    return G > cap ? cap : G;
}

hipError_t launch_score_group(const PagedArgs& a, float* out, int64_t ld, int32_t cus, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    GroupArgs A;
    A.a = a;
    A.G = group_rows_for(a.rows, a.num_reqs, a.relu);
    A.windows = (a.rows + A.G - 1) / A.G;
    A.out = out;
    A.ld = ld;
    A.vec_store = (ld % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) ? 1 : 0;
    A.kpp_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == a.kpp) A.kpp_shift = sh;
    // whole multiples of lcm(32, kpp), at most 64 pages and (where that
    // allows more than one multiple) about kSeg keys
    int64_t gcd = 32, b = a.kpp;
    while (b) { const int64_t t = gcd % b; gcd = b; b = t; }
    const int64_t L = 32 / gcd * a.kpp;
    int64_t nl = std::min<int64_t>(64 * (int64_t)a.kpp / L, kSeg / L);
    if (nl < 1) nl = 1;
    // with few windows, shorter segments (down to 256 keys) spread the keys
    // of a handful of rows over the compute units
    while (nl > 1 && nl % 2 == 0 && L * (nl / 2) >= 256 &&
           (int64_t)A.windows * ((a.max_visible + L * nl - 1) / (L * nl)) < 2 * (int64_t)cus)
        nl /= 2;
    A.seg_len = (int32_t)(L * nl);
    A.nseg = (a.max_visible + A.seg_len - 1) / A.seg_len;
    const int64_t items = (int64_t)A.windows * A.nseg;
    const int64_t blocks = (items + kGroupWaves - 1) / kGroupWaves;
    const dim3 grid((unsigned)blocks);
    if (a.relu) {
        if (A.kpp_shift >= 0) score_group_kernel<true, true><<<grid, kGroupNT, 0, stream>>>(A);
        else score_group_kernel<true, false><<<grid, kGroupNT, 0, stream>>>(A);
    } else {
        if (A.kpp_shift >= 0) score_group_kernel<false, true><<<grid, kGroupNT, 0, stream>>>(A);
        else score_group_kernel<false, false><<<grid, kGroupNT, 0, stream>>>(A);
    }
    return hipGetLastError();
}

}  // namespace qsa
