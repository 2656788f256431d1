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
// Work.  Rows are cut into tiles of consecutive rows (128 in the default
// form, 64 in the relu form: 4 waves of 32 or 16 rows); the logical keys
// (logical key i is key stride*i of the request; stride is 1 except for the
// sampling pass) are cut into 8 stripes, one per XCD.  Workgroup w runs on
// XCD w % 8 (the hardware's round-robin dispatch) and owns a contiguous,
// equal share of that XCD's (tile, key) positions, so every XCD streams only
// its stripe of keys (which stays in its L2) and every workgroup does the
// same amount of work.  A share is processed as pieces of one tile and at
// most kMaxPiece keys.
//
// A piece.  Each of the 4 waves holds the fp16 query fragments of its rows
// in registers (loaded once per tile).  Keys are staged 64 at a time: a
// per-piece table gives every logical key's slot in the cache; each thread
// prefetches its 16-byte pieces of the next 64 keys into registers while the
// current ones are consumed from one half of a double-buffered, XOR-swizzled
// LDS tile (one barrier per 64 keys = two 32-key MFMA column tiles, whose
// MFMA chains are interleaved).  The MFMA arrangements are the canonical ones
// of qsa_device.hpp.
//
// Epilogue.  A 32-key column tile leaves each wave 32 (or 16) rows x 32
// scores spread over the MFMA output layout.  The wave transposes them, 16
// rows at a time, through a small LDS buffer of its own so that each lane
// holds 8 consecutive keys of one row (lanes 4r..4r+3 share row r):
//   Store  -- out[row*ld + i] = score with two 16-byte stores per lane
//             (two-pass arm, sampling pass);
//   Filter -- keep (score, key) if score >= the row's threshold score: one
//             compare per score against a per-lane threshold; a quad prefix
//             sum gives each kept entry its slot in the row's LDS staging list
//             (score bits, key), which the wave moves to the row's global
//             list -- one atomic per row -- when it would overflow and when
//             the workgroup leaves the tile.  No other synchronisation.
// Rows of different requests in one tile are processed in successive passes.
#pragma once

#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

enum class Epi { Store, Filter };

constexpr int kSub = 2;                // 32-key column tiles per LDS stage
constexpr int kStepKeys = 32 * kSub;   // keys per LDS stage
constexpr int kMaxPiece = 1024;        // logical keys per piece (slot-table size)
constexpr int kLCap = 32;              // per-row LDS staging slots of the Filter epilogue (>= 32)
constexpr int kMaxTileRows = 128;      // rows per tile, largest form
constexpr int kXcds = 8;               // XCDs of an MI355X (256 CUs = 8 x 32)
constexpr int kTrStride = 36;          // floats per row of the transpose buffer (32 + 4: conflict-free reads)

struct ScoreKernelArgs {
    PagedArgs a;
    int32_t stride;    // logical key i is key stride*i
    int32_t lmax;      // logical keys of the longest row: ceil(max_visible / stride)
    int32_t tiles;     // ceil(rows / rows per tile)
    int32_t xcd_keys;  // logical keys per XCD stripe (a multiple of kStepKeys)
    int64_t seg_len;   // (tile, key) positions per workgroup (a multiple of kStepKeys)
    // Store
    float* out;
    int64_t ld;
    int32_t vec_store;  // out and ld allow 16-byte stores
    // Filter
    const uint64_t* thresh;  // [rows] threshold composite; only its score is used
    uint64_t* cand;          // [rows][cand_cap] entries (score bits << 32 | key)
    int32_t* cand_count;     // [rows]
    int32_t cand_cap;
};

struct ScoreShape {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int NLOAD = kStepKeys * kChunksPerKey / NT;     // 16-byte pieces per thread per stage
};
static_assert(ScoreShape::NLOAD == 4, "each thread stages 4 consecutive keys per stage");

// The two MFMA arrangements (qsa_device.hpp), as seen by the tiled kernel.
// A lane's MFMA outputs for a 32-key column tile come in rounds of 8 scores
// that cover 16 rows of the wave; out_row(o) is the row (within the round) of
// output o in lane half 0, and lane half 1 adds HALF.
template <bool RELU>
struct Form;
// default form: heads in K; MFMA row = query row (32 per wave); output
// element v of the 16 is row 8*(v/4) + 4*(lane/32) + v%4, i.e. round v/8
template <>
struct Form<false> {
    static constexpr int RPW = 32;                 // rows per wave
    static constexpr int TILE = 4 * RPW;           // rows per tile
    static constexpr int NQ = kHeads * kSlices;    // query fragments per lane: (slice, head)
    static constexpr int ROUNDS = 2;
    static constexpr int HALF = 4;
    __device__ static constexpr int out_row(int o) { return 8 * (o >> 2) + (o & 3); }
};
// relu form: heads in M; two MFMA tiles of 8 rows x 4 heads per wave; the
// head-combined outputs o = 4*mt + g are rows 8*mt + 2*g (+1 for lane half 1)
template <>
struct Form<true> {
    static constexpr int RPW = 16;
    static constexpr int TILE = 4 * RPW;
    static constexpr int NQ = 2 * kSlices;
    static constexpr int ROUNDS = 1;
    static constexpr int HALF = 1;
    __device__ static constexpr int out_row(int o) { return 8 * (o >> 2) + 2 * (o & 3); }
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

// Moves this wave's staged entries of tile rows (one row per quad, `row` =
// its global row) to the rows' global candidate lists: the quad's first lane
// reserves space with one atomic, the quad copies.  Wave-local.
__device__ __forceinline__ void flush_staged(const ScoreKernelArgs& A, const uint64_t* lb, int row, int& cnt) {
    int base = 0;
    if ((threadIdx.x & 3) == 0 && cnt > 0) base = atomicAdd(&A.cand_count[row], cnt);
    base = __builtin_amdgcn_mov_dpp(base, 0x00, 0xF, 0xF, false);  // quad_perm(0,0,0,0)
    uint64_t* dst = A.cand + (int64_t)row * A.cand_cap;
    for (int i = threadIdx.x & 3; i < cnt; i += 4)
        if (base + i < A.cand_cap) dst[base + i] = lb[i];
    cnt = 0;
}

template <bool RELU, Epi EPI>
__global__ __launch_bounds__(ScoreShape::NT, 2) void score_tiles_kernel(ScoreKernelArgs A) {
    using S = ScoreShape;
    using F = Form<RELU>;
    constexpr int NT = S::NT, TILE = F::TILE, RPW = F::RPW, ROUNDS = F::ROUNDS;
    constexpr bool FILTER = EPI == Epi::Filter;

    __shared__ __attribute__((aligned(16))) unsigned char s_keys[2][kStepKeys * kKeyBytes];
    __shared__ __attribute__((aligned(16))) uint32_t s_slot[kMaxPiece];
    __shared__ __attribute__((aligned(16))) float s_tr[S::WAVES][16 * kTrStride];
    __shared__ int32_t s_req[TILE], s_lv[TILE], s_todo[TILE], s_lim[TILE];
    __shared__ float s_fT[FILTER ? TILE : 1];
    __shared__ uint64_t s_lbuf[FILTER ? TILE * kLCap : 1];
    __shared__ int32_t s_act, s_vmax;

    const PagedArgs& a = A.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
    const int xk0 = xcd * A.xcd_keys;
    // keys of this XCD's stripe, padded to whole stages so that every piece
    // starts on a stage boundary (keys past the end are invisible to every row)
    const int span = min(A.xcd_keys, (A.lmax - xk0 + kStepKeys - 1) / kStepKeys * kStepKeys);
    if (span <= 0) return;
    const int64_t total = (int64_t)A.tiles * span;
    int64_t p = (int64_t)loc * A.seg_len;
    const int64_t pend = min(p + A.seg_len, total);

    // staging: this thread's 4 consecutive keys of a stage and its chunk
    const int pk = 4 * (tid >> 4), pc = tid & 15;
    // transposed epilogue: this lane's rows of the wave (rr + 16*round) and
    // its 8 keys of a column tile
    const int rr = lane >> 2, cq = lane & 3;
    int trow[ROUNDS];
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) trow[h] = wave * RPW + 16 * h + rr;
    float* const tw = s_tr[wave];

    // every slot-table entry always holds a valid cache slot, so the prefetch
    // may read entries past the end of a pass's table
    for (int i = tid; i < kMaxPiece; i += NT) s_slot[i] = 0u;

    half8 qa[F::NQ];
    float fT_r[ROUNDS];  // threshold scores of this lane's rows (Filter)
    int cnt_r[ROUNDS];   // staged entries of this lane's rows (Filter)
#pragma unroll
    for (int h = 0; h < ROUNDS; ++h) {
        fT_r[h] = 0.0f;
        cnt_r[h] = 0;
    }
    int tile_r0 = -1;    // first row of the tile held in registers

    while (p < pend) {
        const int tile = (int)(p / span);
        const int off = (int)(p - (int64_t)tile * span);
        const int len = (int)min<int64_t>(min<int64_t>((int64_t)(span - off), pend - p), (int64_t)kMaxPiece);
        const int c0 = xk0 + off, c1 = c0 + len;
        p += len;
        const int r0 = tile * TILE;
        const bool new_tile = r0 != tile_r0;
        if (FILTER && new_tile && tile_r0 >= 0) {
#pragma unroll
            for (int h = 0; h < ROUNDS; ++h) flush_staged(A, s_lbuf + trow[h] * kLCap, tile_r0 + trow[h], cnt_r[h]);
        }

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
            // query fragments of this wave's rows
#pragma unroll
            for (int t = 0; t < F::NQ; ++t) {
                const int m = lane & 31;
                int row, h, s;
                if (RELU) {  // MFMA tile t/8: rows 8*(t/8) + m/4, head m%4; slice t%8
                    row = wave * RPW + (t / kSlices) * 8 + (m >> 2);
                    h = m & 3;
                    s = t % kSlices;
                } else {     // MFMA row m = row m; step t = (slice t/4, head t%4)
                    row = wave * RPW + m;
                    h = t & 3;
                    s = t >> 2;
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
            for (int h = 0; h < ROUNDS; ++h) fT_r[h] = s_fT[trow[h]];
        }
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
            // this lane's row bounds, and the smallest over the wave's rows:
            // column tiles entirely below it need no per-row mask
            int lim_r[ROUNDS];
            int wlim = 0x7FFFFFFF;
#pragma unroll
            for (int h = 0; h < ROUNDS; ++h) {
                lim_r[h] = s_lim[trow[h]];
                wlim = min(wlim, lim_r[h]);
            }
#pragma unroll
            for (int o = 4; o < 64; o <<= 1) wlim = min(wlim, __shfl_xor(wlim, o, 64));
            wlim = __builtin_amdgcn_readfirstlane(wlim);
            __syncthreads();

            // Step: barrier (tile staged) -> issue the loads of the next tile
            // -> MFMAs -> wait for the next tile and stage it in the other
            // buffer -> epilogue.  The epilogue's global stores are issued
            // after the wait, so they drain during the next step's MFMAs.
            const _Float16* kc = a.kcache;
            u32x4 pf[S::NLOAD];
            {
                const u32x4 sl = *reinterpret_cast<const u32x4*>(&s_slot[pk]);
#pragma unroll
                for (int i = 0; i < S::NLOAD; ++i)
                    pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)sl[i] * kHeadDim + pc * 8);
#pragma unroll
                for (int i = 0; i < S::NLOAD; ++i)
                    *reinterpret_cast<u32x4*>(s_keys[0] + lds_key_chunk(pk + i, pc)) = pf[i];
            }
            int buf = 0;
            for (int j0 = c0; j0 < cend; j0 += kStepKeys) {
                __syncthreads();
                const unsigned char* sk = s_keys[buf];
                {
                    const int li = min(j0 + kStepKeys - c0 + pk, kMaxPiece - 4);
                    const u32x4 sl = *reinterpret_cast<const u32x4*>(&s_slot[li]);
#pragma unroll
                    for (int i = 0; i < S::NLOAD; ++i)
                        pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)sl[i] * kHeadDim + pc * 8);
                }
                // keep the prefetch issued here, ahead of the MFMAs that hide it
                __builtin_amdgcn_sched_barrier(0);

                float sc[kSub][ROUNDS][8];
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
                        for (int o = 0; o < 8; ++o) {
                            const int mt = o >> 2, g = o & 3;
                            sc[st][0][o] = combine_relu_heads(acc[st][mt][4 * g], acc[st][mt][4 * g + 1],
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
                        for (int h = 0; h < kHeads; ++h)
#pragma unroll
                            for (int st = 0; st < kSub; ++st) acc[st] = mfma32(qa[kHeads * s + h], kbs[st], acc[st]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int st = 0; st < kSub; ++st)
#pragma unroll
                        for (int h = 0; h < ROUNDS; ++h)
#pragma unroll
                            for (int o = 0; o < 8; ++o) sc[st][h][o] = acc[st][8 * h + o];
                }
                // stage the prefetched tile in the idle buffer (after the last
                // step this fills a buffer no wave reads any more: every wave
                // has passed this step's barrier)
#pragma unroll
                for (int i = 0; i < S::NLOAD; ++i)
                    *reinterpret_cast<u32x4*>(s_keys[buf ^ 1] + lds_key_chunk(pk + i, pc)) = pf[i];

#pragma unroll
                for (int st = 0; st < kSub; ++st) {
                    const int key0 = j0 + 32 * st + 8 * cq;
                    const bool full = j0 + 32 * (st + 1) <= wlim;
#pragma unroll
                    for (int h = 0; h < ROUNDS; ++h) {
                        // transpose: lane (row rr, keys 8cq..8cq+7) of this round
                        const int wr = F::HALF * (lane >> 5);
#pragma unroll
                        for (int o = 0; o < 8; ++o) tw[(wr + F::out_row(o)) * kTrStride + (lane & 31)] = sc[st][h][o];
                        __builtin_amdgcn_wave_barrier();
                        const float4v v0 = *reinterpret_cast<const float4v*>(tw + rr * kTrStride + 8 * cq);
                        const float4v v1 = *reinterpret_cast<const float4v*>(tw + rr * kTrStride + 8 * cq + 4);
                        __builtin_amdgcn_wave_barrier();
                        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                        if (!FILTER) {
                            float* dst = A.out + (int64_t)(r0 + trow[h]) * A.ld + key0;
                            if (full && A.vec_store) {
                                *reinterpret_cast<float4v*>(dst) = v0;
                                *reinterpret_cast<float4v*>(dst + 4) = v1;
                            } else {
#pragma unroll
                                for (int i = 0; i < 8; ++i)
                                    if (full || key0 + i < lim_r[h]) dst[i] = v[i];
                            }
                        } else {
                            bool kp[8];
                            int n = 0;
#pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                kp[i] = v[i] >= fT_r[h] && (full || key0 + i < lim_r[h]);
                                n += kp[i] ? 1 : 0;
                            }
                            int tot;
                            const int excl = quad_exclusive_sum(n, &tot);
                            uint64_t* lb = s_lbuf + trow[h] * kLCap;
                            if (__any(cnt_r[h] + tot > kLCap)) flush_staged(A, lb, r0 + trow[h], cnt_r[h]);
                            int slot = cnt_r[h] + excl;
#pragma unroll
                            for (int i = 0; i < 8; ++i)
                                if (kp[i]) lb[slot++] = ((uint64_t)__float_as_uint(v[i]) << 32) | (uint32_t)(key0 + i);
                            cnt_r[h] += tot;
                        }
                    }
                }
                buf ^= 1;
            }
            // every wave is done with this pass's s_lim before wave 0 rewrites it
            __syncthreads();
        }
        __syncthreads();
    }
    if (FILTER && tile_r0 >= 0) {
#pragma unroll
        for (int h = 0; h < ROUNDS; ++h) flush_staged(A, s_lbuf + trow[h] * kLCap, tile_r0 + trow[h], cnt_r[h]);
    }
}

}  // namespace qsa
