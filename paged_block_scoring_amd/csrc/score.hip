// score.hip -- paged MQA index scorer on gfx950 MFMA (fp16 inputs, fp32
// accumulation), writing one fp32 score per (row, visible key).
//
// Sources: "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
// Turing", section "Purpose" (the scorer is an FP16 product with FP32
// accumulation followed by an epilogue; the paged scorer reads keys through
// the page table) and "Test Plan" (4 index heads, head dim 128, compress
// ratio 4); "spec(MODEL-MM-QWEN4-EXP) ...", section "The component
// deep-dives, and two corrections to the above" (one key per ratio tokens
// shared by all index heads; one score per query token, summed over heads).
//
// Work decomposition.  A workgroup of 4 waves owns a tile of TR = 16*MT
// consecutive rows and a chunk of `chunk` consecutive key indices.  Wave w
// holds the query fragments of MT groups of 4 rows (16 MFMA rows: 4 rows x 4
// heads) in registers for the whole chunk.  Keys are staged 64 at a time in
// LDS (16 KB): each 16-byte chunk of a key is fetched by one thread through
// the page table, so a page's keys are read as contiguous 4 KB runs, and
// stored XOR-swizzled.  Each wave then runs 4 MFMAs (K = 128) per 16 keys per
// row group, sums the heads in registers and writes the visible scores.
// Rows of different requests in one tile are handled in successive passes
// over the chunk, one request per pass.
#include "qsa_device.hpp"
#include "qsa_internal.hpp"

namespace qsa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileKeys = 64;

template <int MT, bool RELU>
__global__ __launch_bounds__(kThreads) void score_paged_kernel(PagedArgs a, float* __restrict__ scores,
                                                               int64_t ld, int32_t chunk) {
    constexpr int TR = 4 * MT * kWaves;
    __shared__ __attribute__((aligned(16))) unsigned char s_keys[kTileKeys * kKeyBytes];
    __shared__ int64_t s_keyoff[kTileKeys];
    __shared__ int32_t s_req[TR], s_vis[TR], s_todo[TR], s_active[TR];
    __shared__ int32_t s_act, s_vmax;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = blockIdx.x * TR;
    const int c0 = blockIdx.y * chunk;
    if (c0 >= a.max_visible) return;
    const int c1 = min(c0 + chunk, a.max_visible);

    if (tid < TR) {
        int r = r0 + tid, req = -1, vis = 0;
        if (r < a.rows) {
            req = a.row_req ? a.row_req[r] : 0;
            if (req < 0 || req >= a.num_reqs) req = -1;
            else vis = visible_keys(a.pos[r], a.cr, a.max_visible);
        }
        s_req[tid] = req;
        s_vis[tid] = vis;
        s_todo[tid] = (req >= 0 && vis > c0) ? 1 : 0;
    }
    __syncthreads();

    for (;;) {
        // One pass per distinct request among the tile's rows that still have
        // visible keys in this chunk.
        if (tid == 0) {
            int act = -1, vmax = 0;
            for (int t = 0; t < TR; ++t)
                if (s_todo[t]) { act = s_req[t]; break; }
            for (int t = 0; t < TR; ++t) {
                int on = (act >= 0 && s_todo[t] && s_req[t] == act) ? 1 : 0;
                s_active[t] = on;
                if (on) { s_todo[t] = 0; vmax = max(vmax, s_vis[t]); }
            }
            s_act = act;
            s_vmax = vmax;
        }
        __syncthreads();
        const int act = s_act;
        if (act < 0) break;
        const int cend = min(c1, s_vmax);

        half8 qa[MT][4];
        int lim[MT];     // keys this lane may write for its output row (0: none)
        int orow[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int tr_a = wave * 4 * MT + 4 * mt + ((lane & 15) >> 2);
            const int h = lane & 3;
            const int r = r0 + tr_a;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                half8 v = {};
                if (r < a.rows)
                    v = *reinterpret_cast<const half8*>(a.q + ((int64_t)r * kHeads + h) * kHeadDim + 32 * s +
                                                        8 * (lane >> 4));
                qa[mt][s] = v;
            }
            const int tr_o = wave * 4 * MT + 4 * mt + (lane >> 4);
            orow[mt] = r0 + tr_o;
            lim[mt] = s_active[tr_o] ? min(s_vis[tr_o], c1) : 0;
        }

        const int32_t* ptrow = a.page_table + (int64_t)act * a.pt_stride;
        for (int j0 = c0; j0 < cend; j0 += kTileKeys) {
            if (tid < kTileKeys) {
                const int j = j0 + tid;
                int64_t off = -1;
                if (j < cend) {
                    const int lp = j / a.kpp;
                    const int slot = j - lp * a.kpp;
                    int p = ptrow[lp];
                    p = min(max(p, 0), a.num_pages - 1);
                    off = ((int64_t)p * a.kpp + slot) * kHeadDim;
                }
                s_keyoff[tid] = off;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kTileKeys * kChunksPerKey / kThreads; ++i) {
                const int flat = i * kThreads + tid, n = flat >> 4, c = flat & 15;
                const int64_t off = s_keyoff[n];
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (off >= 0) v = *reinterpret_cast<const uint4*>(a.kcache + off + c * 8);
                *reinterpret_cast<uint4*>(s_keys + lds_key_chunk(n, c)) = v;
            }
            __syncthreads();
#pragma unroll
            for (int nt = 0; nt < kTileKeys / 16; ++nt) {
                const int n = nt * 16 + (lane & 15);
                half8 kb[4];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    kb[s] = *reinterpret_cast<const half8*>(s_keys + lds_key_chunk(n, 4 * s + (lane >> 4)));
                const int j = j0 + n;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma16(qa[mt][s], kb[s], acc);
                    if (j < lim[mt]) scores[(int64_t)orow[mt] * ld + j] = combine_heads<RELU>(acc);
                }
            }
            __syncthreads();
        }
    }
}

template <int MT>
hipError_t launch_mt(const PagedArgs& a, float* scores, int64_t ld, hipStream_t stream) {
    constexpr int TR = 16 * MT;
    int64_t chunk = 1024;
    const int64_t min_chunk = ((int64_t)a.max_visible + 65534) / 65535;
    if (chunk < min_chunk) chunk = (min_chunk + kTileKeys - 1) / kTileKeys * kTileKeys;
    dim3 grid((unsigned)((a.rows + TR - 1) / TR), (unsigned)((a.max_visible + chunk - 1) / chunk));
    if (a.relu)
        score_paged_kernel<MT, true><<<grid, kThreads, 0, stream>>>(a, scores, ld, (int32_t)chunk);
    else
        score_paged_kernel<MT, false><<<grid, kThreads, 0, stream>>>(a, scores, ld, (int32_t)chunk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_score_paged(const PagedArgs& a, float* scores, int64_t ld, hipStream_t stream) {
    if (a.rows <= 0 || a.max_visible <= 0) return hipSuccess;
    // Many rows per request: 64-row tiles share every staged key tile.
    // Few rows per request (decode): 16-row tiles keep the grid wide.
    const int64_t rows_per_req = a.rows / (a.num_reqs > 0 ? a.num_reqs : 1);
    if (rows_per_req >= 32) return launch_mt<4>(a, scores, ld, stream);
    return launch_mt<1>(a, scores, ld, stream);
}

}  // namespace qsa
