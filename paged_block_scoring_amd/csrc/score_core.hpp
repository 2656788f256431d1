// score_core.hpp -- the tiled paged MQA scoring kernel shared by every arm.
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", sections "Purpose" (FP16 product with FP32 accumulation and an
// epilogue; a paged scorer reading keys through the page table) and "Test
// Plan" (4 index heads, head dim 128, compress ratio 4); "spec(MODEL-MM-QWEN4-
// EXP) ...", section "The component deep-dives, and two corrections to the
// above" (one key per ratio tokens shared by all heads; one score per query
// token summed over heads).
//
// Work.  Rows are cut into tiles of 64 consecutive rows; the logical keys
// (logical key i is key stride*i of the request; stride is 1 except for the
// sampling pass) are cut into 8 stripes, one per XCD.  Workgroup w runs on
// XCD w % 8 (the hardware's round-robin dispatch) and owns a contiguous,
// equal share of that XCD's (tile, key) positions, so every XCD streams only
// its stripe of keys (which stays in its L2) and every workgroup does the
// same amount of work.  A share is processed as pieces of one tile and at
// most kMaxPiece keys.
//
// A piece.  Each of the 4 waves holds the fp16 query fragments of its 16 rows
// in registers (loaded once per tile).  Keys are staged 64 at a time: a
// per-piece table gives every logical key's slot in the cache; each thread
// prefetches its 16-byte pieces of the next 64 keys into registers while the
// current ones are consumed from one half of a double-buffered, XOR-swizzled
// LDS tile (one barrier per 64 keys = two 32-key MFMA column tiles, whose
// MFMA chains are interleaved).  The MFMA arrangements are the canonical ones
// of qsa_device.hpp.  Each visible score goes to the epilogue:
//   Store  -- out[row*ld + i] = score (two-pass arm, sampling pass);
//   Filter -- keep (score, key) if score >= the row's threshold score: one
//             compare per score; kept entries get slots from wave-uniform
//             per-row counters (ballot + mbcnt), are staged per row in LDS
//             as (score bits, key) and appended to the row's global list with
//             one atomic per row and piece.
// Rows of different requests in one tile are processed in successive passes.
#pragma once

#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

enum class Epi { Store, Filter };

constexpr int kSub = 2;                // 32-key column tiles per LDS stage
constexpr int kStepKeys = 32 * kSub;   // keys per LDS stage
constexpr int kMaxPiece = 1024;        // logical keys per piece (slot-table size)
constexpr int kLCap = 64;              // per-row LDS staging slots of the Filter epilogue
constexpr int kTileRows = 64;          // rows per tile
constexpr int kXcds = 8;               // XCDs of an MI355X (256 CUs = 8 x 32)

struct ScoreKernelArgs {
    PagedArgs a;
    int32_t stride;    // logical key i is key stride*i
    int32_t lmax;      // logical keys of the longest row: ceil(max_visible / stride)
    int32_t tiles;     // ceil(rows / kTileRows)
    int32_t xcd_keys;  // logical keys per XCD stripe
    int64_t seg_len;   // (tile, key) positions per workgroup
    // Store
    float* out;
    int64_t ld;
    // Filter
    const uint64_t* thresh;  // [rows] threshold composite; only its score is used
    uint64_t* cand;          // [rows][cand_cap] entries (score bits << 32 | key)
    int32_t* cand_count;     // [rows]
    int32_t cand_cap;
};

struct ScoreShape {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int RPW = kTileRows / WAVES;                    // rows per wave
    static constexpr int NLOAD = kStepKeys * kChunksPerKey / NT;     // 16-byte pieces per thread per stage
    static constexpr int NOUT = 8;                                   // scores per lane per 32 keys
    static constexpr int NQ = 2 * kSlices;                           // query fragments per lane
};

// Row (within the wave's 16) of output o of a lane in lane half 0; lane half
// 1 adds out_half_offset.  Default form: MFMA rows 8*(v/4) + (v%4) hold
// (row, pair) = (m/2, m%2), so outputs o = v/2 are rows 4*(o/2) + o%2 and the
// upper lane half (MFMA rows +4) is rows +2.  Relu form: outputs o = 4*mt + g
// of MFMA tile mt are rows 8*mt + 2*g, and the upper lane half is rows +1.
template <bool RELU>
__device__ __forceinline__ constexpr int out_row_offset(int o) {
    return RELU ? 8 * (o >> 2) + 2 * (o & 3) : 4 * (o >> 1) + (o & 1);
}
template <bool RELU>
__device__ __forceinline__ constexpr int out_half_offset() {
    return RELU ? 1 : 2;
}
template <bool RELU>
__device__ __forceinline__ int out_tile_row(int o, int wave, int lane) {
    return wave * ScoreShape::RPW + out_half_offset<RELU>() * (lane >> 5) + out_row_offset<RELU>(o);
}

// Filter epilogue for one output index o of a wave: `c` is this lane's keep
// decision for (tile row tr, key jn).  The two 32-lane halves of the wave
// hold two different rows, each owned by this wave alone, so the slot of a
// kept entry is the row's running count (a wave-uniform value) plus the
// lane's rank among the kept lanes of its half; no atomics unless the row's
// LDS staging is full.
__device__ __forceinline__ void filter_append(const ScoreKernelArgs& A, bool c, float sc, int tr, int r0, int jn,
                                              int lane, int& cnt_lo, int& cnt_hi, uint64_t* s_lbuf) {
    const uint64_t m = __ballot(c);
    if (m == 0ull) return;
    const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
    const bool upper = lane >= 32;
    const int rank = (int)__builtin_amdgcn_mbcnt_hi(upper ? hi : 0u, __builtin_amdgcn_mbcnt_lo(upper ? 0u : lo, 0u));
    const int slot = (upper ? cnt_hi : cnt_lo) + rank;
    cnt_lo += __popc(lo);
    cnt_hi += __popc(hi);
    if (c) {
        const uint64_t e = ((uint64_t)__float_as_uint(sc) << 32) | (uint32_t)jn;
        if (slot < kLCap) {
            s_lbuf[tr * kLCap + slot] = e;
        } else {
            const int g = atomicAdd(&A.cand_count[r0 + tr], 1);
            if (g < A.cand_cap) A.cand[(int64_t)(r0 + tr) * A.cand_cap + g] = e;
        }
    }
}

template <bool RELU, Epi EPI>
__global__ __launch_bounds__(ScoreShape::NT, 2) void score_tiles_kernel(ScoreKernelArgs A) {
    using S = ScoreShape;
    constexpr int NT = S::NT, NOUT = S::NOUT;
    constexpr bool FILTER = EPI == Epi::Filter;

    __shared__ __attribute__((aligned(16))) unsigned char s_keys[2][kStepKeys * kKeyBytes];
    __shared__ uint32_t s_slot[kMaxPiece];
    __shared__ int32_t s_req[kTileRows], s_lv[kTileRows], s_todo[kTileRows], s_lim[kTileRows];
    __shared__ float s_fT[FILTER ? kTileRows : 1];
    __shared__ int32_t s_lc[FILTER ? kTileRows : 1];
    __shared__ uint64_t s_lbuf[FILTER ? kTileRows * kLCap : 1];
    __shared__ int32_t s_act, s_vmax;

    const PagedArgs& a = A.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
    const int xk0 = xcd * A.xcd_keys;
    const int span = min(A.xcd_keys, A.lmax - xk0);
    if (span <= 0) return;
    const int64_t total = (int64_t)A.tiles * span;
    int64_t p = (int64_t)loc * A.seg_len;
    const int64_t pend = min(p + A.seg_len, total);

    half8 qa[S::NQ];
    float fT[NOUT];
    int loaded_tile = -1;

    while (p < pend) {
        const int tile = (int)(p / span);
        const int off = (int)(p - (int64_t)tile * span);
        const int len = (int)min<int64_t>(min<int64_t>((int64_t)(span - off), pend - p), (int64_t)kMaxPiece);
        const int c0 = xk0 + off, c1 = c0 + len;
        p += len;
        const int r0 = tile * kTileRows;
        const bool new_tile = tile != loaded_tile;

        for (int t = tid; t < kTileRows; t += NT) {
            const int r = r0 + t;
            int req = -1, lv = 0;
            if (r < a.rows) {
                req = a.row_req ? a.row_req[r] : 0;
                if (req < 0 || req >= a.num_reqs) {
                    req = -1;
                } else {
                    const int v = visible_keys(a.pos[r], a.cr, a.max_visible);
                    lv = (v + A.stride - 1) / A.stride;
                }
            }
            s_req[t] = req;
            s_lv[t] = lv;
            s_todo[t] = (req >= 0 && lv > c0) ? 1 : 0;
            // the threshold composite's score (an all-ones composite decodes
            // to NaN, which no score reaches)
            if (FILTER && new_tile) s_fT[t] = req >= 0 ? key_to_float((uint32_t)(A.thresh[r] >> 32)) : 0.0f;
        }
        if (new_tile) {
            // query fragments of this wave's 16 rows
#pragma unroll
            for (int t = 0; t < S::NQ; ++t) {
                const int m = lane & 31;
                int row, h, s;
                if (RELU) {  // MFMA tile t/8: rows 8*(t/8) + m/4, head m%4; slice t%8
                    row = wave * S::RPW + (t / kSlices) * 8 + (m >> 2);
                    h = m & 3;
                    s = t % kSlices;
                } else {     // MFMA row m = (row m/2, pair m%2); step t = (slice t/2, head 2*pair + t%2)
                    row = wave * S::RPW + (m >> 1);
                    h = 2 * (m & 1) + (t & 1);
                    s = t >> 1;
                }
                row += r0;
                half8 v = {};
                if (row < a.rows)
                    v = *reinterpret_cast<const half8*>(a.q + ((int64_t)row * kHeads + h) * kHeadDim + 16 * s +
                                                        8 * (lane >> 5));
                qa[t] = v;
            }
        }
        __syncthreads();
        if (FILTER && new_tile) {
#pragma unroll
            for (int o = 0; o < NOUT; ++o) fT[o] = s_fT[out_tile_row<RELU>(o, wave, lane)];
        }
        loaded_tile = tile;

        // kept-entry counts of this wave's 16 rows (output o, lane half)
        int cnt_lo[NOUT], cnt_hi[NOUT];
#pragma unroll
        for (int o = 0; o < NOUT; ++o) cnt_lo[o] = cnt_hi[o] = 0;

        for (;;) {
            // one pass per request present among the tile's pending rows
            // (smallest request id first): wave 0 elects it and marks the rows
            if (wave == 0) {
                int best = 0x7FFFFFFF;
                for (int t = lane; t < kTileRows; t += 64)
                    if (s_todo[t]) best = min(best, s_req[t]);
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, 64));
                int vmax = 0;
                for (int t = lane; t < kTileRows; t += 64) {
                    const bool on = s_todo[t] && s_req[t] == best;
                    s_lim[t] = on ? min(s_lv[t], c1) : 0;
                    if (on) {
                        s_todo[t] = 0;
                        vmax = max(vmax, s_lv[t]);
                    }
                }
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) vmax = max(vmax, __shfl_xor(vmax, o, 64));
                if (lane == 0) {
                    s_act = best == 0x7FFFFFFF ? -1 : best;
                    s_vmax = vmax;
                }
            }
            __syncthreads();
            const int act = s_act;
            if (act < 0) break;
            const int cend = min(c1, s_vmax);

            const int32_t* ptrow = a.page_table + (int64_t)act * a.pt_stride;
            for (int i = tid; i < cend - c0; i += NT) {
                const int j = (c0 + i) * A.stride;
                const int lp = j / a.kpp;
                const int slot = j - lp * a.kpp;
                const int pg = min(max(ptrow[lp], 0), a.num_pages - 1);
                s_slot[i] = (uint32_t)pg * (uint32_t)a.kpp + (uint32_t)slot;
            }
            // smallest visible bound over this wave's rows: column tiles
            // entirely below it need no per-row mask
            int wlim = 0x7FFFFFFF;
            for (int t = lane; t < S::RPW; t += 64) wlim = min(wlim, s_lim[wave * S::RPW + t]);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) wlim = min(wlim, __shfl_xor(wlim, o, 64));
            __syncthreads();

            // Step: barrier (tile staged) -> issue the loads of the next tile
            // -> MFMAs -> wait for the next tile and stage it in the other
            // buffer -> epilogue.  The epilogue's global stores are issued
            // after the wait, so they drain during the next step's MFMAs.
            const _Float16* kc = a.kcache;
            u32x4 pf[S::NLOAD];
#pragma unroll
            for (int i = 0; i < S::NLOAD; ++i) {
                const int flat = i * NT + tid, n = flat >> 4, c = flat & 15;
                const int li = min(c0 + n, cend - 1) - c0;
                pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)s_slot[li] * kHeadDim + c * 8);
            }
#pragma unroll
            for (int i = 0; i < S::NLOAD; ++i) {
                const int flat = i * NT + tid, n = flat >> 4, c = flat & 15;
                *reinterpret_cast<u32x4*>(s_keys[0] + lds_key_chunk(n, c)) = pf[i];
            }
            const int tr0 = out_tile_row<RELU>(0, wave, lane);
            int buf = 0;
            for (int j0 = c0; j0 < cend; j0 += kStepKeys) {
                __syncthreads();
                const unsigned char* sk = s_keys[buf];
#pragma unroll
                for (int i = 0; i < S::NLOAD; ++i) {
                    const int flat = i * NT + tid, n = flat >> 4, c = flat & 15;
                    const int li = min(j0 + kStepKeys + n, cend - 1) - c0;
                    pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)s_slot[li] * kHeadDim + c * 8);
                }
                // keep the prefetch issued here, ahead of the MFMAs that hide it
                __builtin_amdgcn_sched_barrier(0);

                float sc[kSub][NOUT];
                if (RELU) {
                    float16v acc[kSub][2];
#pragma unroll
                    for (int st = 0; st < kSub; ++st) acc[st][0] = acc[st][1] = float16v{};
#pragma unroll
                    for (int s = 0; s < kSlices; ++s) {
                        half8 kbs[kSub];
#pragma unroll
                        for (int st = 0; st < kSub; ++st)
                            kbs[st] = *reinterpret_cast<const half8*>(
                                sk + lds_key_chunk(32 * st + (lane & 31), 2 * s + (lane >> 5)));
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int st = 0; st < kSub; ++st)
                                acc[st][mt] = mfma32(qa[mt * kSlices + s], kbs[st], acc[st][mt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int st = 0; st < kSub; ++st)
#pragma unroll
                        for (int o = 0; o < NOUT; ++o) {
                            const int mt = o >> 2, g = o & 3;
                            sc[st][o] = combine_relu_heads(acc[st][mt][4 * g], acc[st][mt][4 * g + 1],
                                                           acc[st][mt][4 * g + 2], acc[st][mt][4 * g + 3]);
                        }
                } else {
                    float16v acc[kSub];
#pragma unroll
                    for (int st = 0; st < kSub; ++st) acc[st] = float16v{};
#pragma unroll
                    for (int s = 0; s < kSlices; ++s) {
                        half8 kbs[kSub];
#pragma unroll
                        for (int st = 0; st < kSub; ++st)
                            kbs[st] = *reinterpret_cast<const half8*>(
                                sk + lds_key_chunk(32 * st + (lane & 31), 2 * s + (lane >> 5)));
#pragma unroll
                        for (int t = 2 * s; t < 2 * s + 2; ++t)
#pragma unroll
                            for (int st = 0; st < kSub; ++st) acc[st] = mfma32(qa[t], kbs[st], acc[st]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int st = 0; st < kSub; ++st)
#pragma unroll
                        for (int o = 0; o < NOUT; ++o) sc[st][o] = combine_pairs(acc[st][2 * o], acc[st][2 * o + 1]);
                }
                // stage the prefetched tile in the idle buffer (after the last
                // step this fills a buffer no wave reads any more: every wave
                // has passed this step's barrier)
#pragma unroll
                for (int i = 0; i < S::NLOAD; ++i) {
                    const int flat = i * NT + tid, n = flat >> 4, c = flat & 15;
                    *reinterpret_cast<u32x4*>(s_keys[buf ^ 1] + lds_key_chunk(n, c)) = pf[i];
                }

#pragma unroll
                for (int st = 0; st < kSub; ++st) {
                    const int jn = j0 + 32 * st + (lane & 31);  // this lane's key (logical index)
                    const bool full = j0 + 32 * (st + 1) <= wlim;
                    if (!FILTER) {
                        float* base = A.out + (int64_t)(r0 + tr0) * A.ld + jn;
                        if (full) {
#pragma unroll
                            for (int o = 0; o < NOUT; ++o) base[(int64_t)out_row_offset<RELU>(o) * A.ld] = sc[st][o];
                        } else {
#pragma unroll
                            for (int o = 0; o < NOUT; ++o)
                                if (jn < s_lim[tr0 + out_row_offset<RELU>(o)])
                                    base[(int64_t)out_row_offset<RELU>(o) * A.ld] = sc[st][o];
                        }
                    } else {
#pragma unroll
                        for (int o = 0; o < NOUT; ++o) {
                            const int tr = tr0 + out_row_offset<RELU>(o);
                            bool c = sc[st][o] >= fT[o];
                            if (!full) c = c && jn < s_lim[tr];
                            filter_append(A, c, sc[st][o], tr, r0, jn, lane, cnt_lo[o], cnt_hi[o], s_lbuf);
                        }
                    }
                }
                buf ^= 1;
            }
            // every wave is done with this pass's s_lim before wave 0 rewrites it
            __syncthreads();
        }

        if (FILTER) {
            // flush the staged entries: one global atomic per row
            if (lane == 0) {
#pragma unroll
                for (int o = 0; o < NOUT; ++o) {
                    s_lc[out_tile_row<RELU>(o, wave, 0)] = cnt_lo[o];
                    s_lc[out_tile_row<RELU>(o, wave, 32)] = cnt_hi[o];
                }
            }
            __syncthreads();
            for (int t = wave; t < kTileRows; t += S::WAVES) {
                const int n = min(s_lc[t], kLCap);
                if (n == 0) continue;
                const int row = r0 + t;
                int base = 0;
                if (lane == 0) base = atomicAdd(&A.cand_count[row], n);
                base = __shfl(base, 0, 64);
                for (int i = lane; i < n; i += 64)
                    if (base + i < A.cand_cap) A.cand[(int64_t)row * A.cand_cap + base + i] = s_lbuf[t * kLCap + i];
            }
        }
        __syncthreads();
    }
}

}  // namespace qsa
