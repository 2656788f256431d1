// score_core.hpp -- the tiled paged scorer of the relu form (QSA_SCORE_RELU:
// per-head dots, each through relu, summed, times the fp32 value nearest
// 1/sqrt(128)); the default form has its own kernel in score_rows.hpp.
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", sections "Purpose" (FP16 product with FP32 accumulation and an
// epilogue; a paged scorer reading keys through the page table) and "Test
// Plan" (4 index heads, head dim 128, compress ratio 4); "spec(MODEL-MM-QWEN4-
// EXP) ...", section "The component deep-dives, and two corrections to the
// above" (one key per ratio tokens shared by all heads; relu per head and the
// 1/sqrt(head_dim) scale).
//
// Work.  Rows are cut into tiles of 64 consecutive rows (4 waves of 16); the
// logical keys (logical key i is key stride*i of the request; stride is 1
// except for the sampling pass) are cut into 8 stripes, one per XCD.
// Workgroup w runs on XCD w % 8 (the hardware's round-robin dispatch) and
// owns a contiguous, equal share of that XCD's (tile, key) positions, so every
// XCD streams only its stripe of keys (which stays in its L2) and every
// workgroup does the same amount of work.  With several requests and the
// tiles' visible-key counts, each tile's own keys are striped instead and the
// stripes shared evenly (TileShares, score_rows.hpp), so that tiles of short
// rows cost nothing.  A share is processed as pieces of one tile and at most
// kMaxPiece keys.
//
// A piece.  Each of the 4 waves holds the fp16 query fragments of its rows
// in registers (loaded once per tile): MFMA row m = 4*row + head, 8 rows x 4
// heads per MFMA tile, two tiles per wave.  Keys are staged 64 at a time: a
// per-piece table gives every logical key's slot in the cache; each thread
// prefetches its 16-byte pieces of the next 64 keys into registers while the
// current ones are consumed from one half of a double-buffered, XOR-swizzled
// LDS tile (one barrier per 64 keys = two 32-key MFMA column tiles, whose
// MFMA chains are interleaved).  The MFMA arrangement is the canonical one of
// qsa_device.hpp.
//
// Epilogue.  The head-combined scores of a 32-key column tile are spread over
// rows, so the wave transposes them through a small LDS buffer of its own
// until lane l holds row l/4 and 8 consecutive keys.  Then
//   Store  -- out[row*ld + i] = score with 16-byte stores (two-pass arm,
//             sampling pass);
//   Filter -- keep (score, key) if score >= the row's threshold score: one
//             compare per score against a per-lane threshold, whose ballot is
//             the exec mask of that score's append (no branch); a prefix sum
//             over the row's 4 lanes gives each lane its first slot in the
//             row's LDS staging list (score bits, key), which the lanes move
//             to the row's global list -- one atomic per row -- when it would
//             overflow and when the workgroup leaves the tile.
// Rows of different requests in one tile are processed in successive passes.
#pragma once

#include <type_traits>

#include "qsa_device.hpp"
#include "qsa_internal.hpp"
#include "score_rows.hpp"

namespace qsa {

constexpr int kLCap = 32;              // per-row LDS staging slots of the Filter epilogue (>= 32)

struct ScoreKernelArgs {
    PagedArgs a;
    const _Float16* qsum;  // default form only: prepared head sums, or null
    int32_t stride;    // logical key i is key stride*i
    int32_t lmax;      // logical keys of the longest row: ceil(max_visible / stride)
    int32_t tiles;     // ceil(rows / rows per tile)
    const int32_t* tile_v;  // relu form: [tiles] visible keys of each tile's longest row, or null (see below)
    int32_t xcd_keys;  // logical keys per XCD stripe (a multiple of the stage size)
    int64_t seg_len;   // (tile, key) positions per workgroup (a multiple of the stage size)
    // Store
    float* out;
    int64_t ld;
    int32_t vec_store;  // out and ld allow 16-byte stores
    int32_t true_scores;  // default form: store scores, else chain results (score / head-sum factor)
    // Filter
    const uint64_t* thresh;  // [rows] threshold composite; only its score is used
    uint64_t* cand;          // [rows][cand_cap] entries (score bits << 32 | key)
    int32_t* cand_count;     // [rows * kCountStride]
    int32_t cand_cap;
};

struct ScoreShape {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
};

// The relu form's MFMA arrangement (qsa_device.hpp) as seen by the tiled
// kernel: heads in M, two MFMA tiles of 8 rows x 4 heads per wave; the
// head-combined outputs o = 4*mt + g are rows 8*mt + 2*g (+1 for lane half
// 1), transposed to lane l = row l/4, keys 8*(l%4) .. 8*(l%4)+7.
struct ReluForm {
    static constexpr int RPW = 16;                 // rows per wave
    static constexpr int TILE = 4 * RPW;           // rows per tile
    static constexpr int NQ = 2 * kSlices;         // query fragments per lane: (MFMA tile, slice)
    static constexpr int SUB = 2;                  // 32-key column tiles per LDS stage
    static constexpr int STEP = 32 * SUB;          // keys per LDS stage
    static constexpr int NLOAD = STEP * kChunksPerKey / ScoreShape::NT;  // 16-byte pieces per thread per stage
    static constexpr int MAXPIECE = 1024;          // logical keys per piece (slot-table size)
    static constexpr int WG_PER_CU = 2;            // resident workgroups per compute unit
    static_assert(NLOAD * ScoreShape::NT == STEP * kChunksPerKey, "whole keys per thread");
    __device__ static constexpr int out_row(int o) { return 8 * (o >> 2) + 2 * (o & 3); }
    __device__ static int lane_row(int lane) { return lane >> 2; }
};

// Quad (lanes 4k..4k+3) exclusive prefix sum of x; *total gets the quad sum.
__device__ __forceinline__ int quad_exclusive_sum(int x, int* total) {
    const int q = threadIdx.x & 3;
    // quad_perm(0,0,1,2): lane q reads lane q-1 (lane 0 reads itself)
    const int a = __builtin_amdgcn_mov_dpp(x, 0x90, 0xF, 0xF, false);
    const int s1 = x + (q >= 1 ? a : 0);
    // quad_perm(0,0,0,1): lanes 2, 3 read lanes 0, 1
    const int b = __builtin_amdgcn_mov_dpp(s1, 0x40, 0xF, 0xF, false);
    const int incl = s1 + (q >= 2 ? b : 0);
    // quad_perm(3,3,3,3): everyone reads lane 3
    *total = __builtin_amdgcn_mov_dpp(incl, 0xFF, 0xF, 0xF, false);
    return incl - x;
}

// Moves the staged entries of one row per lane group (the `gsize` lanes that
// share `row`; `leader` is the group's member 0) to the rows' global
// candidate lists: the leader reserves space with one atomic, the group
// copies.  Wave-local.
__device__ __forceinline__ void flush_staged(const ScoreKernelArgs& A, const uint64_t* lb, int row, int& cnt,
                                             int leader, int member, int gsize) {
    int base = 0;
    if (member == 0 && cnt > 0) base = atomicAdd(&A.cand_count[(int64_t)row * kCountStride], cnt);
    base = __shfl(base, leader, 64);
    uint64_t* dst = A.cand + (int64_t)row * A.cand_cap;
    for (int i = member; i < cnt; i += gsize)
        if (base + i < A.cand_cap) dst[base + i] = lb[i];
    cnt = 0;
}

__device__ __forceinline__ uint64_t cand_entry(float score, int key) {
    return ((uint64_t)__float_as_uint(score) << 32) | (uint32_t)key;
}

template <Epi EPI>
__global__ __launch_bounds__(ScoreShape::NT, ReluForm::WG_PER_CU) void score_tiles_kernel(ScoreKernelArgs A) {
    using F = ReluForm;
    constexpr int NT = ScoreShape::NT, TILE = F::TILE, RPW = F::RPW;
    constexpr int kSub = F::SUB, kStepKeys = F::STEP, NLOAD = F::NLOAD;
    constexpr int kMaxPiece = F::MAXPIECE;
    constexpr bool FILTER = EPI == Epi::Filter;

    __shared__ __attribute__((aligned(16))) unsigned char s_keys[2][kStepKeys * kKeyBytes];
    __shared__ __attribute__((aligned(16))) uint32_t s_slot[kMaxPiece];
    // per-wave transpose buffer (16 rows)
    __shared__ __attribute__((aligned(16))) float s_tr[ScoreShape::WAVES][RPW * kTrStride];
    __shared__ int32_t s_req[TILE], s_lv[TILE], s_todo[TILE], s_lim[TILE];
    __shared__ float s_fT[FILTER ? TILE : 1];
    __shared__ uint64_t s_lbuf[FILTER ? TILE * kLCap : 1];
    __shared__ int32_t s_act, s_vmax;

    const PagedArgs& a = A.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
    // Work positions of this XCD: without tile counts, keys xk0 .. xk0+span of
    // the XCD's stripe of the longest row for every tile, padded to whole
    // stages so that every piece starts on a stage boundary (keys past the end
    // are invisible to every row); with them (tile_v, several requests), each
    // tile's own stripes laid end to end and shared evenly (TileShares).
    const bool bal = A.tile_v != nullptr;
    const int xk0 = xcd * A.xcd_keys;
    const int span = min(A.xcd_keys, (A.lmax - xk0 + kStepKeys - 1) / kStepKeys * kStepKeys);
    if (!bal && span <= 0) return;
    TileShares<NT, kStepKeys> ts{A.tile_v, A.tiles, A.stride, xcd};
    int64_t p, pend;
    if (bal) {
        ts.begin(loc, gridDim.x / kXcds, &p, &pend);
    } else {
        const int64_t total = (int64_t)A.tiles * span;
        p = (int64_t)loc * A.seg_len;
        pend = min(p + A.seg_len, total);
    }

    // staging: this thread's NLOAD consecutive keys of a stage and its chunk
    const int pk = NLOAD * (tid >> 4), pc = tid & 15;
    // epilogue: the tile row this lane works on, and its lane group
    const int erow = wave * RPW + F::lane_row(lane);
    const int g_leader = lane & ~3, g_member = lane & 3;
    constexpr int g_size = 4;

    // every slot-table entry always holds a valid cache slot, so the prefetch
    // may read entries past the end of a pass's table
    for (int i = tid; i < kMaxPiece; i += NT) s_slot[i] = 0u;

    half8 qa[F::NQ];
    float fT_r = 0.0f;  // threshold score of this lane's row (Filter)
    int cnt_r = 0;      // staged entries of this lane's row (Filter)
    int tile_r0 = -1;   // first row of the tile held in registers

    while (p < pend) {
        int tile, len, c0;
        if (bal) {
            ts.piece(p, pend, kMaxPiece, &tile, &c0, &len);
        } else {
            tile = (int)(p / span);
            const int off = (int)(p - (int64_t)tile * span);
            len = (int)min<int64_t>(min<int64_t>((int64_t)(span - off), pend - p), (int64_t)kMaxPiece);
            c0 = xk0 + off;
        }
        const int c1 = c0 + len;
        p += len;
        const int r0 = tile * TILE;
        const bool new_tile = r0 != tile_r0;
        if (FILTER && new_tile && tile_r0 >= 0)
            flush_staged(A, s_lbuf + erow * kLCap, tile_r0 + erow, cnt_r, g_leader, g_member, g_size);

        for (int t = tid; t < TILE; t += NT) {
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
            // query fragments of this wave's rows (A operand: MFMA tile t/8
            // rows 8*(t/8) + m/4, head m%4; slice t%8)
#pragma unroll
            for (int t = 0; t < F::NQ; ++t) {
                const int m = lane & 31;
                const int row = r0 + wave * RPW + (t / kSlices) * 8 + (m >> 2);
                half8 v = {};
                if (row < a.rows)
                    v = *reinterpret_cast<const half8*>(a.q + ((int64_t)row * kHeads + (m & 3)) * kHeadDim +
                                                        16 * (t % kSlices) + 8 * (lane >> 5));
                qa[t] = v;
            }
        }
        __syncthreads();
        if (FILTER && new_tile) fT_r = s_fT[erow];
        tile_r0 = r0;

        for (;;) {
            // one pass per request present among the tile's pending rows
            // (smallest request id first): wave 0 elects it and marks the rows
            if (wave == 0) {
                int best = 0x7FFFFFFF;
                for (int t = lane; t < TILE; t += 64)
                    if (s_todo[t]) best = min(best, s_req[t]);
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, 64));
                int vmax = 0;
                for (int t = lane; t < TILE; t += 64) {
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
            // this lane's row bound, and the smallest over the wave's rows:
            // column tiles entirely below it need no per-row mask
            const int lim_r = s_lim[erow];
            int wlim = lim_r;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) wlim = min(wlim, __shfl_xor(wlim, o, 64));
            wlim = __builtin_amdgcn_readfirstlane(wlim);
            __syncthreads();

            // Step i: barrier (stage i staged) -> issue the loads of stage i+2
            // -> MFMAs on stage i -> wait for the loads of stage i+1 (issued
            // one step earlier) and stage them in the other buffer ->
            // epilogue.  Loads thus have two steps to arrive; the slot of
            // stage i+3 is read from LDS during step i so that the next
            // step's loads issue right after its barrier.  Two register sets
            // alternate (the loop is unrolled by two).
            const _Float16* kc = a.kcache;
            using SlotVec = typename std::conditional<NLOAD == 4, u32x4, u32x2>::type;
            auto slots_of = [&](int stage) {
                const int li = min(stage * kStepKeys + pk, kMaxPiece - NLOAD);
                return *reinterpret_cast<const SlotVec*>(&s_slot[li]);
            };
            auto issue = [&](const SlotVec& sl, u32x4 (&pf)[NLOAD]) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i)
                    pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)sl[i] * kHeadDim + pc * 8);
            };
            auto stage_in = [&](int b, const u32x4 (&pf)[NLOAD]) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i)
                    *reinterpret_cast<u32x4*>(s_keys[b] + lds_key_chunk(pk + i, pc)) = pf[i];
            };
            u32x4 pfA[NLOAD], pfB[NLOAD];
            issue(slots_of(0), pfA);
            stage_in(0, pfA);
            issue(slots_of(1), pfA);
            SlotVec sl_next = slots_of(2);
            const int nsteps = (cend - c0 + kStepKeys - 1) / kStepKeys;
            auto step = [&](int si, const u32x4 (&pf_wait)[NLOAD], u32x4 (&pf_issue)[NLOAD]) {
                const int j0 = c0 + si * kStepKeys;
                const int buf = si & 1;
                __syncthreads();
                const unsigned char* sk = s_keys[buf];
                issue(sl_next, pf_issue);
                sl_next = slots_of(si + 3);
                // keep the prefetch issued here, ahead of the MFMAs that hide it
                __builtin_amdgcn_sched_barrier(0);

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
                float sc[kSub][8];
#pragma unroll
                for (int st = 0; st < kSub; ++st)
#pragma unroll
                    for (int o = 0; o < 8; ++o) {
                        const int mt = o >> 2, g = o & 3;
                        sc[st][o] = combine_relu_heads(acc[st][mt][4 * g], acc[st][mt][4 * g + 1],
                                                       acc[st][mt][4 * g + 2], acc[st][mt][4 * g + 3]);
                    }
                // stage the prefetched tile in the idle buffer (after the
                // last step this fills a buffer no wave reads any more:
                // every wave has passed this step's barrier)
                stage_in(buf ^ 1, pf_wait);

                float* const tw = s_tr[wave];
                const int rr = lane >> 2, cq = lane & 3;
#pragma unroll
                for (int st = 0; st < kSub; ++st) {
                    // transpose: lane (row rr, keys 8cq..8cq+7) of this column tile
#pragma unroll
                    for (int o = 0; o < 8; ++o)
                        tw[(F::out_row(o) + (lane >> 5)) * kTrStride + (lane & 31)] = sc[st][o];
                    __builtin_amdgcn_wave_barrier();
                    const float4v v0 = *reinterpret_cast<const float4v*>(tw + rr * kTrStride + 8 * cq);
                    const float4v v1 = *reinterpret_cast<const float4v*>(tw + rr * kTrStride + 8 * cq + 4);
                    __builtin_amdgcn_wave_barrier();
                    const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    const int key0 = j0 + 32 * st + 8 * cq;
                    const bool full = j0 + 32 * (st + 1) <= wlim;
                    if (!FILTER) {
                        float* dst = A.out + (int64_t)(r0 + erow) * A.ld + key0;
                        if (full && A.vec_store) {
                            *reinterpret_cast<float4v*>(dst) = v0;
                            *reinterpret_cast<float4v*>(dst + 4) = v1;
                        } else {
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                if (full || key0 + i < lim_r) dst[i] = v[i];
                        }
                    } else {
                        // the ballot of each compare is the exec mask of that
                        // score's append (no branch); bounds only on a tile
                        // that crosses a row's end
                        uint64_t m[16];
                        if (full) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) m[i] = __builtin_amdgcn_ballot_w64(v[i] >= fT_r);
                        } else {
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                m[i] = __builtin_amdgcn_ballot_w64(v[i] >= fT_r && key0 + i < lim_r);
                        }
#pragma unroll
                        for (int i = 8; i < 16; ++i) m[i] = 0ull;
                        int n = 0;
                        count_masks8(m, 0, n);
                        int tot;
                        const int excl = quad_exclusive_sum(n, &tot);
                        uint64_t* lb = s_lbuf + erow * kLCap;
                        if (__any(cnt_r + tot > kLCap))
                            flush_staged(A, lb, r0 + erow, cnt_r, g_leader, g_member, g_size);
                        // entries (key, score bits) from this lane's slot of the row's list on
                        uint32_t ad = (uint32_t)reinterpret_cast<uintptr_t>(static_cast<void*>(lb + cnt_r + excl));
                        const float16v sv = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7],
                                             0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                        append_masks8(m, sv, 0, key0, ad);
                        cnt_r += tot;
                    }
                }
            };
            for (int si = 0; si < nsteps; si += 2) {
                step(si, pfA, pfB);
                if (si + 1 < nsteps) step(si + 1, pfB, pfA);
            }
            // every wave is done with this pass's s_lim before wave 0 rewrites it
            __syncthreads();
        }
        __syncthreads();
    }
    if (FILTER && tile_r0 >= 0)
        flush_staged(A, s_lbuf + erow * kLCap, tile_r0 + erow, cnt_r, g_leader, g_member, g_size);
}

}  // namespace qsa
