// score_rows.hpp -- the tiled paged scorer of the default score form (the
// plain head sum), used by the sampling and filtering passes of the fused arm
// and by the materialising scorer.
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", sections "Purpose" (FP16 product with FP32 accumulation and an
// epilogue; a paged scorer reading keys through the page table) and "Test
// Plan" (4 index heads, head dim 128, compress ratio 4); "spec(MODEL-MM-QWEN4-
// EXP) ...", section "The component deep-dives, and two corrections to the
// above" (one key per ratio tokens shared by all heads; one score per query
// token summed over heads).
//
// Work.  Rows are cut into tiles of 128 consecutive rows (4 waves of 32); the
// logical keys (logical key i is key stride*i of the request; stride is 1
// except for the sampling pass) are cut into 8 stripes, one per XCD.
// Workgroup w runs on XCD w % 8 (the hardware's round-robin dispatch) and
// owns a contiguous, equal share of that XCD's (tile, key) positions, so every
// XCD streams only its stripe of keys (which stays in its L2) and every
// workgroup does the same amount of work.  A share is processed as pieces of
// one tile and at most kRowsPiece keys; rows of different requests in one
// tile are processed in successive passes over the piece (with a single
// request there is one pass, set up before the piece's first barrier: the
// page ids are loaded first and the slot table written as soon as they are
// in, while the row and query loads are still on their way).
//
// A piece.  Each wave holds the head-sum query fragments (hi and lo halves,
// qsa_device.hpp) of its 32 rows in registers: read from the prepared head
// sums when the caller has them (coalesced), else formed from q.  A per-piece table in LDS
// gives every logical key's slot in the cache.  Keys go through LDS 32 at a
// time (8 KB, double-buffered, XOR-swizzled).  Step i: barrier -> issue the
// global loads of stage i+2 into registers -> read the 8 key fragments of
// stage i -> 16 MFMAs (keys as MFMA rows, the wave's rows as columns) ->
// wait for the loads of stage i+1 (issued one step earlier) and write them to
// the idle buffer -> epilogue.  Two register sets alternate, so a load has two
// steps to arrive; the slot of stage i+3 is read during step i.  The LDS row
// of key n of a stage is sigma^-1(n) (see Form), which makes lane l's
// accumulator element v the score of row l%32 and key 16*(l/32) + v.
//
// Epilogues.
//   Store  -- out[row*ld + i] = score (or, for the sampling pass, the chain
//             result score / f of the row's head-sum factor f, the unit the
//             filtering pass compares in): the wave transposes its 32 x 32 tile
//             through LDS so that 8 consecutive lanes store 32 consecutive
//             keys (128 bytes) of one row with 16-byte stores;
//   Filter -- keep (key, score) if score >= the row's threshold score.  Each
//             lane keeps its own list in LDS (kLaneCap entries).  A step
//             compares the lane's 16 scores (the ballot of each compare is the
//             exec mask of that score's append) and counts them; a lane whose
//             list would overflow makes the wave move every lane's list to the
//             rows' global candidate lists (one atomic per lane), as does
//             leaving a tile.  The appends themselves run without branches:
//             exec is set to the score's ballot around one LDS store; they
//             are issued in the gaps of the next stage's MFMA chain.  A row
//             with no key in a pass (another request's, or a padding row)
//             compares against NaN, so only the pass's own rows bound the
//             column tiles that need a per-key mask, and a wave none of whose
//             rows is in the pass skips its MFMA chain.
#pragma once

#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {

enum class Epi { Store, Filter };

constexpr int kXcds = 8;         // XCDs of an MI355X (256 CUs = 8 x 32)
constexpr int kTrStride = 36;    // floats per row of a transpose buffer (32 + 4: conflict-free reads)
constexpr int kRowsPiece = 2048; // logical keys per piece (slot-table entries)
constexpr int kLaneCap = 24;     // entries of a lane's LDS candidate list (>= 16)

struct RowsArgs {
    PagedArgs a;
    const _Float16* qsum;  // head sums in fragment order (qsa_internal.hpp), or null
    const float* qfac;     // with qsum: each row slot's head-sum factor
    int32_t stride;    // logical key i is key stride*i
    int32_t lmax;      // logical keys of the longest row: ceil(max_visible / stride)
    int32_t tiles;     // ceil(rows / 128)
    const int32_t* tile_v; // [tiles] visible keys of each tile's longest row, or null (see below)
    int32_t xcd_keys;  // logical keys per XCD stripe (a multiple of 32)
    int32_t kpp_shift; // log2(keys per page) when that is a power of two, else -1
    int64_t seg_len;   // (tile, key) positions per workgroup (a multiple of 32)
    // Store
    float* out;
    int64_t ld;
    int32_t vec_store;  // out and ld allow 16-byte stores
    int32_t true_scores;  // store scores (chain result x head-sum factor), else chain results
    // Filter
    const uint64_t* thresh;  // [rows] threshold composite; only its score is used
    uint64_t* cand;          // [rows][cand_cap] entries (score bits << 32 | key)
    int32_t* cand_count;     // [rows * kCountStride]
    int32_t cand_cap;
};

struct RowsShape {
    static constexpr int WAVES = 4;
    static constexpr int NT = 64 * WAVES;
    static constexpr int RPW = 32;               // rows per wave
    static constexpr int TILE = WAVES * RPW;     // rows per tile
    static constexpr int STEP = 32;              // keys per stage
    static constexpr int NLOAD = STEP * kChunksPerKey / NT;  // 16-byte pieces per thread per stage
    static_assert(NLOAD == 2, "two consecutive keys per thread");
    // LDS row of key n of a stage: sigma^-1, sigma(m) = 16*((m/4)%2) + 4*(m/8) + m%4
    __device__ static int stage_row(int n) {
        const int k = n & 31;
        return (n & ~31) | (8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3));
    }
};

// n += the number of masks among m0..m7 that hold this lane (one add with
// carry-in per mask).  The masks come from VALU compares, and a VALU-written
// SGPR read as a carry needs two wait states: the block starts with them.
__device__ __forceinline__ void count_masks8(const uint64_t (&m)[16], int o, int& n) {
    uint64_t junk;
    asm volatile(
        "s_nop 1\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m0]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m1]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m2]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m3]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m4]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m5]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m6]\n\t"
        "v_addc_co_u32_e64 %[n], %[j], %[n], 0, %[m7]"
        : [n] "+v"(n), [j] "=&s"(junk)
        : [m0] "s"(m[o]), [m1] "s"(m[o + 1]), [m2] "s"(m[o + 2]), [m3] "s"(m[o + 3]), [m4] "s"(m[o + 4]),
          [m5] "s"(m[o + 5]), [m6] "s"(m[o + 6]), [m7] "s"(m[o + 7]));
}

// Appends (key kb+v, score sv) for v = o..o+7 at LDS byte address addr
// (advanced by 8 per entry) in the lanes of mask m[v]: exec is set to m[v]
// around each entry's store, so lanes outside it neither store nor advance,
// without a branch.  The caller runs with a full exec, which is restored.
__device__ __forceinline__ void append_masks8(const uint64_t (&m)[16], const float16v& sc, int o, int kb,
                                              uint32_t& addr) {
    int tk;
#define QSA_APPEND_ONE(V)                                      \
    "s_mov_b64 exec, %[m" #V "]\n\t"                           \
    "v_add_u32 %[tk], " #V ", %[kb]\n\t"                       \
    "ds_write2_b32 %[ad], %[tk], %[s" #V "] offset1:1\n\t"     \
    "v_add_u32 %[ad], 8, %[ad]\n\t"
    asm volatile(
        QSA_APPEND_ONE(0) QSA_APPEND_ONE(1) QSA_APPEND_ONE(2) QSA_APPEND_ONE(3)
        QSA_APPEND_ONE(4) QSA_APPEND_ONE(5) QSA_APPEND_ONE(6) QSA_APPEND_ONE(7)
        "s_mov_b64 exec, -1"
        : [ad] "+v"(addr), [tk] "=&v"(tk)
        : [kb] "v"(kb + o), [m0] "s"(m[o]), [m1] "s"(m[o + 1]), [m2] "s"(m[o + 2]), [m3] "s"(m[o + 3]),
          [m4] "s"(m[o + 4]), [m5] "s"(m[o + 5]), [m6] "s"(m[o + 6]), [m7] "s"(m[o + 7]), [s0] "v"(sc[o]),
          [s1] "v"(sc[o + 1]), [s2] "v"(sc[o + 2]), [s3] "v"(sc[o + 3]), [s4] "v"(sc[o + 4]),
          [s5] "v"(sc[o + 5]), [s6] "v"(sc[o + 6]), [s7] "v"(sc[o + 7])
        : "memory");
#undef QSA_APPEND_ONE
}

// A quarter (4 MFMAs, chain steps t = 4b..4b+3) of a 32-key stage's MFMA
// chain, with 4 of the previous stage's appends (scores v = 4b..4b+3) placed
// in the gaps the dependent chain leaves: after each MFMA the append's exec
// is set to its ballot, the key formed, the entry stored, the address
// advanced and exec restored.  Quarter 0 starts the chain from zero; quarter
// 3 ends with the wait states an MFMA result needs before a VALU may read it
// and also names every key fragment of the stage as an input, so that no
// fragment register is reused (written) while an MFMA of the chain may still
// read it.  Nothing else in a block touches the chain's accumulators.
template <int B>
__device__ __forceinline__ void mfma_quarter_appends(float16v& acc, const half8 (&kf)[8], const half8& k0,
                                                     const half8& k1, const half8 (&qa)[16],
                                                     const uint64_t (&m)[16], const float16v& ps, int pkb,
                                                     uint32_t& pad) {
    int tk;
#define QSA_APP(V)                                          \
    "s_mov_b64 exec, %[m" #V "]\n\t"                        \
    "v_add_u32 %[tk], " #V ", %[kb]\n\t"                    \
    "ds_write2_b32 %[ad], %[tk], %[s" #V "] offset1:1\n\t"  \
    "v_add_u32 %[ad], 8, %[ad]\n\t"                         \
    "s_mov_b64 exec, -1\n\t"
#define QSA_OPS                                                                                      \
    [k0] "v"(k0), [k1] "v"(k1), [q0] "v"(qa[4 * B]), [q1] "v"(qa[4 * B + 1]), [q2] "v"(qa[4 * B + 2]),  \
        [q3] "v"(qa[4 * B + 3]), [m0] "s"(m[4 * B]), [m1] "s"(m[4 * B + 1]), [m2] "s"(m[4 * B + 2]),     \
        [m3] "s"(m[4 * B + 3]), [s0] "v"(ps[4 * B]), [s1] "v"(ps[4 * B + 1]), [s2] "v"(ps[4 * B + 2]),   \
        [s3] "v"(ps[4 * B + 3]), [kb] "v"(pkb + 4 * B)
    if (B == 0) {
        asm volatile(
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q0], 0\n\t" QSA_APP(0)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q1], %[acc]\n\t" QSA_APP(1)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q2], %[acc]\n\t" QSA_APP(2)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q3], %[acc]\n\t" QSA_APP(3)
            : [acc] "=&v"(acc), [ad] "+v"(pad), [tk] "=&v"(tk)
            : QSA_OPS
            : "memory");
    } else if (B < 3) {
        asm volatile(
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q0], %[acc]\n\t" QSA_APP(0)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q1], %[acc]\n\t" QSA_APP(1)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q2], %[acc]\n\t" QSA_APP(2)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q3], %[acc]\n\t" QSA_APP(3)
            : [acc] "+v"(acc), [ad] "+v"(pad), [tk] "=&v"(tk)
            : QSA_OPS
            : "memory");
    } else {
        asm volatile(
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q0], %[acc]\n\t" QSA_APP(0)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k0], %[q1], %[acc]\n\t" QSA_APP(1)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q2], %[acc]\n\t" QSA_APP(2)
            "v_mfma_f32_32x32x16_f16 %[acc], %[k1], %[q3], %[acc]\n\t" QSA_APP(3)
            "s_nop 7\n\ts_nop 7\n\ts_nop 7"
            : [acc] "+v"(acc), [ad] "+v"(pad), [tk] "=&v"(tk)
            : QSA_OPS, [f0] "v"(kf[0]), [f1] "v"(kf[1]), [f2] "v"(kf[2]), [f3] "v"(kf[3]), [f4] "v"(kf[4]),
              [f5] "v"(kf[5])
            : "memory");
    }
#undef QSA_OPS
#undef QSA_APP
}

// Balanced (tile, key) positions of the tiled scorers, for calls with several
// requests.  tile_v[t] is the visible-key count of tile t's longest row; its
// logical keys (logical key i is key stride*i) are cut into kXcds stripes
// padded to whole stages of STEP keys, and this XCD's stripe of every tile is
// laid end to end.  The XCD's workgroups share that total evenly, in whole
// stages, so that tiles of short rows cost nothing.  A cursor follows the
// tile that holds the current position.
template <int NT, int STEP>
struct TileShares {
    const int32_t* tile_v;
    int tiles, stride, xcd;
    int tcur = 0, ucur = 0, stcur = 0;  // the tile holding the cursor, its share and its stripe
    int64_t pbase = 0;                  // the position where that share starts

    // this XCD's stage-padded share of tile t's keys; *st = the tile's stripe
    __device__ __forceinline__ int share(int t, int* st) const {
        const int lv = (tile_v[t] + stride - 1) / stride;
        *st = ((lv + kXcds - 1) / kXcds + STEP - 1) / STEP * STEP;
        const int u = min(max(lv - xcd * *st, 0), *st);
        return (u + STEP - 1) / STEP * STEP;
    }

    // Positions [*p, *pend) of workgroup `loc` of the XCD's `per`, and the
    // cursor on the tile that holds *p.  Called by the whole workgroup (one
    // block scan of the shares); contains barriers.
    __device__ __forceinline__ void begin(int loc, int64_t per, int64_t* p, int64_t* pend) {
        __shared__ int32_t s_ws[NT / 64];
        __shared__ int64_t s_found;
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        // an inclusive block scan of the shares of tiles t0 .. t0+NT-1
        auto scan = [&](int t0, int& u, int& incl, int& chunk) {
            int st;
            u = t0 + tid < tiles ? share(t0 + tid, &st) : 0;
            incl = u;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int nb = __shfl_up(incl, o, 64);
                if (lane >= o) incl += nb;
            }
            if (lane == 63) s_ws[wave] = incl;
            __syncthreads();
            chunk = 0;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) {
                incl += w < wave ? s_ws[w] : 0;
                chunk += s_ws[w];
            }
            __syncthreads();
        };
        int64_t total = 0;
        int u0 = 0, incl0 = 0;  // the first chunk's scan, kept for the search below
        for (int t0 = 0; t0 < tiles; t0 += NT) {
            int u, incl, chunk;
            scan(t0, u, incl, chunk);
            if (t0 == 0) {
                u0 = u;
                incl0 = incl;
            }
            total += chunk;
        }
        const int64_t seg = max<int64_t>(STEP, ((total + per - 1) / per + STEP - 1) / STEP * STEP);
        *p = (int64_t)loc * seg;
        *pend = min(*p + seg, total);
        if (*p < *pend) {
            const int64_t q = *p;
            // the tile whose share holds q (exactly one thread finds it); with
            // at most NT tiles the first scan already holds every prefix
            if (tid == 0) s_found = -1;
            __syncthreads();
            if (tiles <= NT) {
                if (u0 > 0 && incl0 - u0 <= q && q < incl0)
                    s_found = ((int64_t)tid << 32) | (uint64_t)(uint32_t)(incl0 - u0);
            } else {
                int64_t base = 0;
                for (int t0 = 0; t0 < tiles; t0 += NT) {
                    int u, incl, chunk;
                    scan(t0, u, incl, chunk);
                    if (u > 0 && base + incl - u <= q && q < base + incl)
                        s_found = ((int64_t)(t0 + tid) << 32) | (uint64_t)(uint32_t)(base + incl - u);
                    base += chunk;
                }
            }
            __syncthreads();
            tcur = (int)(s_found >> 32);
            pbase = (int64_t)(uint32_t)(s_found & 0xFFFFFFFFll);
            ucur = share(tcur, &stcur);
        }
    }

    // The piece at position p (< pend): its tile, its first logical key and
    // its length, at most maxlen keys and not past pend.
    __device__ __forceinline__ void piece(int64_t p, int64_t pend, int maxlen, int* tile, int* c0, int* len) {
        while (p >= pbase + ucur) {  // on to the next tile with keys on this XCD
            pbase += ucur;
            ++tcur;
            ucur = share(tcur, &stcur);
        }
        *tile = tcur;
        const int off = (int)(p - pbase);
        *len = (int)min<int64_t>(min<int64_t>((int64_t)(ucur - off), pend - p), (int64_t)maxlen);
        *c0 = xcd * stcur + off;
    }
};

template <Epi EPI>
__global__ __launch_bounds__(RowsShape::NT, 2) void score_rows_kernel(RowsArgs A) {
    using S = RowsShape;
    constexpr int NT = S::NT, TILE = S::TILE, RPW = S::RPW, STEP = S::STEP, NLOAD = S::NLOAD;
    constexpr bool FILTER = EPI == Epi::Filter;

    __shared__ __attribute__((aligned(16))) unsigned char s_keys[2][STEP * kKeyBytes];
    __shared__ __attribute__((aligned(16))) uint32_t s_slot[kRowsPiece];
    __shared__ __attribute__((aligned(16))) float s_tr[FILTER ? 1 : S::WAVES][FILTER ? 4 : RPW * kTrStride];
    __shared__ __attribute__((aligned(16))) uint2 s_list[FILTER ? NT * kLaneCap : 1];
    __shared__ int32_t s_req[TILE], s_lv[TILE], s_todo[TILE], s_lim[TILE];
    __shared__ float s_fT[FILTER ? TILE : 1];
    __shared__ int32_t s_act, s_vmax;
    __shared__ int32_t s_wv[TILE / 64];  // one request: per wave of row threads, the longest active row

    const PagedArgs& a = A.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
    // Work positions of this XCD.  Without tile counts: keys xk0 .. xk0+span
    // of the XCD's stripe of the longest row, for every tile.  With them
    // (tile_v): each tile's own visible keys cut into 8 stripes, this XCD's
    // stripe of every tile laid end to end, and the workgroups of the XCD
    // share that total evenly, so that tiles of short rows cost nothing.
    // Stripes are padded to whole stages so that every piece starts on a
    // stage boundary (keys past the end are invisible to every row).
    const bool bal = A.tile_v != nullptr;
    const int xk0 = xcd * A.xcd_keys;
    const int span = min(A.xcd_keys, (A.lmax - xk0 + STEP - 1) / STEP * STEP);
    if (!bal && span <= 0) return;
    TileShares<NT, STEP> ts{A.tile_v, A.tiles, A.stride, xcd};
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
    // epilogue: the tile row of this lane
    const int erow = wave * RPW + (lane & 31);

    // every slot-table entry always holds a valid cache slot, so the prefetch
    // may read entries past the end of a pass's table
    for (int i = tid; i < kRowsPiece; i += NT) s_slot[i] = 0u;

    half8 qa[2 * kSlices];
    float fac = 1.0f;  // head-sum factor of this lane's row (Store with true_scores)
    float fT = 0.0f;  // threshold chain result of this lane's row (Filter)
    int cnt = 0;      // entries in this lane's list (Filter)
    const uint32_t list0 =
        (uint32_t)reinterpret_cast<uintptr_t>(static_cast<void*>(&s_list[0])) + (uint32_t)(tid * kLaneCap * 8);
    int tile_r0 = -1;  // first row of the tile held in registers

    // moves every lane's list to its row's global candidate list: lanes l and
    // l+32 hold the same row, lane l reserves room for both with one atomic
    // and lane l+32's entries follow lane l's (the list is read from LDS 16
    // bytes at a time).  Called by whole waves.
    auto flush = [&](int row) {
        const int other = __shfl_xor(cnt, 32, 64);
        int base = 0;
        if (lane < 32 && cnt + other > 0) base = atomicAdd(&A.cand_count[(int64_t)row * kCountStride], cnt + other);
        base = __shfl(base, lane & 31, 64) + (lane >= 32 ? other : 0);
        const int lim = min(cnt, A.cand_cap - base);
        uint64_t* dst = A.cand + (int64_t)row * A.cand_cap + base;
        const u32x4* src = reinterpret_cast<const u32x4*>(&s_list[tid * kLaneCap]);
        u32x4 e[kLaneCap / 2];
#pragma unroll
        for (int i = 0; i < kLaneCap / 2; ++i) e[i] = src[i];
#pragma unroll
        for (int i = 0; i < kLaneCap / 2; ++i) {
            if (2 * i < lim) dst[2 * i] = ((uint64_t)e[i][1] << 32) | e[i][0];
            if (2 * i + 1 < lim) dst[2 * i + 1] = ((uint64_t)e[i][3] << 32) | e[i][2];
        }
        cnt = 0;
    };
    // the single-request case builds a piece's slot table while its rows load
    const bool one_req = a.num_reqs == 1;
    // cache slot of every key of the piece (page ids clamped into the cache);
    // all page ids are loaded before any is used (lanes past the piece in its
    // last group reload its last key's page and write nothing)
    auto build_slots = [&](int act, int k0, int k1) {
        constexpr int U = kRowsPiece / NT;
        const int n = k1 - k0;
        if (n <= 0) return;
        const int32_t* ptrow = a.page_table + (int64_t)act * a.pt_stride;
        int32_t pg[U];
        int sl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u * NT >= n) break;
            const int j = (k0 + min(tid + u * NT, n - 1)) * A.stride;
            const int lp = A.kpp_shift >= 0 ? (j >> A.kpp_shift) : j / a.kpp;
            sl[u] = j - lp * a.kpp;
            pg[u] = ptrow[lp];
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (tid + u * NT < n)
                s_slot[tid + u * NT] = (uint32_t)min(max(pg[u], 0), a.num_pages - 1) * (uint32_t)a.kpp + (uint32_t)sl[u];
    };

    while (p < pend) {
        int tile, len, c0;
        if (bal) {
            ts.piece(p, pend, kRowsPiece, &tile, &c0, &len);
        } else {
            tile = (int)(p / span);
            const int off = (int)(p - (int64_t)tile * span);
            len = (int)min<int64_t>(min<int64_t>((int64_t)(span - off), pend - p), (int64_t)kRowsPiece);
            c0 = xk0 + off;
        }
        const int c1 = c0 + len;
        p += len;
        const int r0 = tile * TILE;
        const bool new_tile = r0 != tile_r0;
        if (FILTER && new_tile && tile_r0 >= 0) flush(tile_r0 + erow);

        // (the stripe end c1 is padded to whole stages and may lie up to 31
        // keys past the last visible key; the table stops at that key, so no
        // page-table entry beyond the request's visible pages is read)
        // (one request: the page ids first, in two halves -- loads now, the
        // table once they, and only they, are in)
        constexpr int U = kRowsPiece / NT;
        const int sn = one_req ? min(c1, A.lmax) - c0 : 0;
        int32_t pg1[U];
        int sl1[U];
        if (sn > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (u * NT >= sn) break;
                const int j = (c0 + min(tid + u * NT, sn - 1)) * A.stride;
                const int lp = A.kpp_shift >= 0 ? (j >> A.kpp_shift) : j / a.kpp;
                sl1[u] = j - lp * a.kpp;
                pg1[u] = a.page_table[lp];
            }
        }
        // the tile's rows (threads < 128), then the queries: the slot table
        // below waits only for the page ids, the rows' bounds only for the
        // rows, and the queries are first needed by the first MFMA
        int req = -1, ps = 0;
        uint64_t th = 0ull;
        const int rr = r0 + tid;
        if (tid < TILE) {
            const int rc = rr < a.rows ? rr : a.rows - 1;
            req = a.row_req ? a.row_req[rc] : 0;
            ps = a.pos[rc];
            if (FILTER && new_tile) th = A.thresh[rc];
        }
        if (new_tile && A.qsum) {
            // prepared head sums: 16 coalesced 16-byte loads per lane
            const half8* qs = reinterpret_cast<const half8*>(A.qsum) + ((int64_t)tile * S::WAVES + wave) * 16 * 64 + lane;
#pragma unroll
            for (int t = 0; t < 2 * kSlices; ++t) qa[t] = qs[64 * t];
            if (!FILTER && A.true_scores) fac = A.qfac[r0 + erow];
        } else if (new_tile) {
            // B operand: column m = row m; step t of the chain = (slice t/2, hi/lo t%2)
            const int row = r0 + wave * RPW + (lane & 31);
            const int rowc = row < a.rows ? row : a.rows - 1;
            const _Float16* qr = a.q + (int64_t)rowc * kHeads * kHeadDim + 8 * (lane >> 5);
            auto load = [&](int s, int hh) {
                const half8 v = *reinterpret_cast<const half8*>(qr + hh * kHeadDim + 16 * s);
                return row < a.rows ? v : half8{};
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
            if (!A.true_scores) fac = 1.0f;
        }
        if (sn > 0) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (tid + u * NT < sn)
                    s_slot[tid + u * NT] = (uint32_t)min(max(pg1[u], 0), a.num_pages - 1) * (uint32_t)a.kpp + (uint32_t)sl1[u];
        }
        if (tid < TILE) {
            int lv = 0;
            if (rr >= a.rows || req < 0 || req >= a.num_reqs) {
                req = -1;
            } else {
                const int v = visible_keys(ps, a.cr, a.max_visible);
                lv = (v + A.stride - 1) / A.stride;
            }
            s_req[tid] = req;
            s_lv[tid] = lv;
            s_todo[tid] = (req >= 0 && lv > c0) ? 1 : 0;
            // the threshold composite's score (an all-ones composite decodes
            // to NaN, which no score reaches)
            if (FILTER && new_tile) s_fT[tid] = req >= 0 ? key_to_float((uint32_t)(th >> 32)) : 0.0f;
            if (one_req) {
                // a single pass over every active row: its bounds now, and the
                // longest active row per wave (TILE row threads = whole waves)
                const bool on = req >= 0 && lv > c0;
                s_lim[tid] = on ? min(lv, c1) : 0;
                int wv = on ? lv : 0;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) wv = max(wv, __shfl_xor(wv, o, 64));
                if (lane == 0) s_wv[wave] = wv;
            }
        }
        __syncthreads();
        if (FILTER && new_tile) fT = s_fT[erow];
        tile_r0 = r0;

        bool one_done = false;
        for (;;) {
            int act = 0, vm = 0;
            if (one_req) {
                if (one_done) break;
                one_done = true;
#pragma unroll
                for (int w = 0; w < TILE / 64; ++w) vm = max(vm, s_wv[w]);
                if (vm <= c0) break;
            } else {
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
                act = s_act;
                if (act < 0) break;
                vm = s_vmax;
            }
            const int cend = min(c1, vm);

            if (!one_req) build_slots(act, c0, cend);
            // this lane's row bound, and the smallest over the wave's rows:
            // column tiles entirely below it need no per-row mask
            const int lim_r = s_lim[erow];
            // (Filter: a row with no key in this pass -- another request's, one
            // that ends before the piece, or a padding row -- takes a NaN
            // threshold, which no score reaches, and does not bound the
            // wave's unmasked column tiles)
            const bool row_on = lim_r > c0;
            int wlim = FILTER && !row_on ? 0x7FFFFFFF : lim_r;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) wlim = min(wlim, __shfl_xor(wlim, o, 64));
            wlim = __builtin_amdgcn_readfirstlane(wlim);
            const float fTp = row_on ? fT : __builtin_nanf("");
            const bool wave_on = wlim != 0x7FFFFFFF;
            // (with one request the slot table and bounds were in place at the first barrier)
            if (!one_req) __syncthreads();

            const _Float16* kc = a.kcache;
            auto slots_of = [&](int stage) {
                const int li = min(stage * STEP + pk, kRowsPiece - NLOAD);
                return *reinterpret_cast<const u32x2*>(&s_slot[li]);
            };
            auto issue = [&](const u32x2& sl, u32x4 (&pf)[NLOAD]) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i)
                    pf[i] = *reinterpret_cast<const u32x4*>(kc + (size_t)sl[i] * kHeadDim + pc * 8);
            };
            auto stage_in = [&](int b, const u32x4 (&pf)[NLOAD]) {
#pragma unroll
                for (int i = 0; i < NLOAD; ++i)
                    *reinterpret_cast<u32x4*>(s_keys[b] + lds_key_chunk(S::stage_row(pk + i), pc)) = pf[i];
            };
            // stages 0 and 1 load together; stage 0 goes to LDS, stage 1 is
            // the first step's pending set
            u32x4 pfA[NLOAD], pfB[NLOAD];
            issue(slots_of(0), pfB);
            issue(slots_of(1), pfA);
            stage_in(0, pfB);
            u32x2 sl_next = slots_of(2);
            const int nsteps = (cend - c0 + STEP - 1) / STEP;

            auto step_store = [&](int si, const u32x4 (&pf_wait)[NLOAD], u32x4 (&pf_issue)[NLOAD]) {
                const int j0 = c0 + si * STEP;
                const int buf = si & 1;
                __syncthreads();
                const unsigned char* sk = s_keys[buf];
                issue(sl_next, pf_issue);
                sl_next = slots_of(si + 3);
                // keep the prefetch issued here, ahead of the MFMAs that hide it
                __builtin_amdgcn_sched_barrier(0);
                half8 kf[kSlices];
#pragma unroll
                for (int s = 0; s < kSlices; ++s)
                    kf[s] = *reinterpret_cast<const half8*>(sk + lds_key_chunk(lane & 31, 2 * s + (lane >> 5)));
                __builtin_amdgcn_sched_barrier(0);
                float16v acc = {};
#pragma unroll
                for (int s = 0; s < kSlices; ++s) {
                    acc = mfma32(kf[s], qa[2 * s], acc);
                    acc = mfma32(kf[s], qa[2 * s + 1], acc);
                }
                __builtin_amdgcn_sched_barrier(0);
                // stage i+1 into the idle buffer (after the last step this fills a
                // buffer no wave reads any more: every wave has passed this step's barrier)
                stage_in(buf ^ 1, pf_wait);

                // element v: key kb + v of row erow
                const int kb = j0 + 16 * (lane >> 5);
                const bool full = j0 + STEP <= wlim;
                if (A.true_scores) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[v] *= fac;
                }
                {
                    // transpose so that lane l holds keys 4*(l%8) .. +3 of rows l/8 + 8i
                    float* const tw = s_tr[wave];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<float4v*>(tw + (lane & 31) * kTrStride + 16 * (lane >> 5) + 4 * j) =
                            float4v{acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]};
                    __builtin_amdgcn_wave_barrier();
                    float4v w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        w[i] = *reinterpret_cast<const float4v*>(tw + ((lane >> 3) + 8 * i) * kTrStride + 4 * (lane & 7));
                    __builtin_amdgcn_wave_barrier();
                    const int key0 = j0 + 4 * (lane & 7);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int trow = wave * RPW + (lane >> 3) + 8 * i;
                        float* dst = A.out + (int64_t)(r0 + trow) * A.ld + key0;
                        if (full && A.vec_store) {
                            *reinterpret_cast<float4v*>(dst) = w[i];
                        } else {
                            const int lim = s_lim[trow];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (full || key0 + e < lim) dst[e] = w[i][e];
                        }
                    }
                }
            };

            // Filter: the appends of a stage ride in the next stage's MFMA chain.
            // Two sets (scores, ballots, list address, key base) alternate: the
            // step writes one and appends the other's entries.
            auto step_filter = [&](int si, const u32x4 (&pf_wait)[NLOAD], u32x4 (&pf_issue)[NLOAD], float16v& acc,
                                   uint64_t (&m)[16], uint32_t& ad, int& kbw, const float16v& pacc,
                                   const uint64_t (&pm)[16], uint32_t pad, int pkb) {
                const int j0 = c0 + si * STEP;
                const int buf = si & 1;
                __syncthreads();
                const unsigned char* sk = s_keys[buf];
                issue(sl_next, pf_issue);
                sl_next = slots_of(si + 3);
                __builtin_amdgcn_sched_barrier(0);
                // (a wave with no row in this pass has nothing to score or append)
                if (wave_on) {
                    half8 kf[kSlices];
#pragma unroll
                    for (int s = 0; s < kSlices; ++s)
                        kf[s] = *reinterpret_cast<const half8*>(sk + lds_key_chunk(lane & 31, 2 * s + (lane >> 5)));
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(1);
                    mfma_quarter_appends<0>(acc, kf, kf[0], kf[1], qa, pm, pacc, pkb, pad);
                    mfma_quarter_appends<1>(acc, kf, kf[2], kf[3], qa, pm, pacc, pkb, pad);
                    mfma_quarter_appends<2>(acc, kf, kf[4], kf[5], qa, pm, pacc, pkb, pad);
                    mfma_quarter_appends<3>(acc, kf, kf[6], kf[7], qa, pm, pacc, pkb, pad);
                    __builtin_amdgcn_s_setprio(0);
                }
                __builtin_amdgcn_sched_barrier(0);
                stage_in(buf ^ 1, pf_wait);

                // element v: key kb + v of row erow
                const int kb = j0 + 16 * (lane >> 5);
                // a column tile that crosses a row bound: scores past it cannot pass
                if (j0 + STEP > wlim) {
                    const int nv = min(max(lim_r - kb, 0), 16);
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (v >= nv) acc[v] = -__builtin_huge_valf();
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) m[v] = __builtin_amdgcn_ballot_w64(acc[v] >= fTp);
                int n = 0;
                count_masks8(m, 0, n);
                count_masks8(m, 8, n);
                // the lists now hold every entry up to the previous stage
                if (__any(cnt + n > kLaneCap)) flush(r0 + erow);
                ad = list0 + (uint32_t)(cnt * 8);
                kbw = kb;
                cnt += n;
            };

            if (!FILTER) {
                for (int si = 0; si < nsteps; si += 2) {
                    step_store(si, pfA, pfB);
                    if (si + 1 < nsteps) step_store(si + 1, pfB, pfA);
                }
            } else {
                float16v accA, accB;
                uint64_t mA[16], mB[16];
                uint32_t adA = list0, adB = list0;
                int kbA = 0, kbB = 0;
#pragma unroll
                for (int v = 0; v < 16; ++v) mB[v] = 0ull;  // nothing pending before the first stage
                int si = 0;
                for (; si + 1 < nsteps; si += 2) {
                    step_filter(si, pfA, pfB, accA, mA, adA, kbA, accB, mB, adB, kbB);
                    step_filter(si + 1, pfB, pfA, accB, mB, adB, kbB, accA, mA, adA, kbA);
                }
                // the last stage's entries
                if (si < nsteps) {
                    step_filter(si, pfA, pfB, accA, mA, adA, kbA, accB, mB, adB, kbB);
                    append_masks8(mA, accA, 0, kbA, adA);
                    append_masks8(mA, accA, 8, kbA, adA);
                } else {
                    append_masks8(mB, accB, 0, kbB, adB);
                    append_masks8(mB, accB, 8, kbB, adB);
                }
            }
            // every wave is done with this pass's s_lim before wave 0 rewrites it
            __syncthreads();
        }
        __syncthreads();
    }
    if (FILTER && tile_r0 >= 0) flush(tile_r0 + erow);
}

}  // namespace qsa
