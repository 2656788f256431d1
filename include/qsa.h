/*
 * qsa.h -- C ABI of the paged block-scoring indexer (QSA-style sparse
 * attention indexer) for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  Each query row r (one token of a prefill chunk
 * or of a decode step) belongs to a request and sits at absolute position
 * pos[r].  The request owns a paged side cache of compressed index keys: one
 * fp16 key of head_dim values per block of compress_ratio (cr) tokens, shared
 * by all index heads (MQA with a single key head).  Key j covers tokens
 * cr*j .. cr*j+cr-1 and becomes visible to row r once its last token exists,
 * i.e. for j < V_r = (pos[r]+1) / cr.  Every visible key is scored against the
 * row's index-head queries; the per-head dot products (fp16 inputs, fp32
 * accumulation) are summed over heads into one fp32 score per (row, key).
 * The row keeps its exact top k/cr blocks under the lexicographic rule
 * "higher score first, lower index on ties", and each block expands to its cr
 * raw token positions; unused output slots hold -1.
 *
 * Sources (cited by page title and section):
 *  [thor]   "qwen4_exp QSA cooperative_topk cannot launch on NVIDIA Thor
 *           (sm_110): cluster misconfiguration", section "What happens" (the
 *           indexer's forward calls qsa_select_paged_tokens, which runs a
 *           top-k op over (logits, visible_blocks, blocks, workspace,
 *           block_topk, columns); a failed launch surfaces as an error that
 *           names the source location and the launch error).
 *  [turing] "[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on
 *           Turing", sections "Purpose" (FP16 scorer with FP32 accumulation;
 *           exact lexicographic top-k with a deterministic tie rule), "Test
 *           Plan" (4 index heads, head dim 128, compress ratio 4, top-k 2,048
 *           tokens), "Path coverage" (block top-k 512, int32 indices).
 *  [spec]   "spec(MODEL-MM-QWEN4-EXP): Qwen3.8-Flash-Next is a new
 *           architecture vLLM does not implement, so the port splits its
 *           oracle", section "The component deep-dives, and two corrections to
 *           the above" (one key head of dim 128 shared by the index heads,
 *           relu(q.k) summed over heads and scaled by 1/sqrt(head_dim), no
 *           head axis in the result, the (position+1) % ratio boundary, one
 *           stored state per ratio tokens, raw tokens selected at ratio
 *           granularity, every candidate selected below the budget).
 *
 * Conventions for every entry point.
 *  - Pointers named as device data must point to device memory (HIP
 *    allocations) of the current device; host scalars are passed by value.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream).  Nothing is synchronised.
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    retains a pointer after returning; buffers must stay alive until the
 *    enqueued work completes.  Scratch memory is a caller-provided workspace
 *    sized by the matching *_workspace_size query ([thor]: the top-k op takes
 *    a caller workspace).
 *  - Argument errors are detected on the host before anything is enqueued
 *    and return a non-zero qsa_status; qsa_last_error() then describes the
 *    failure as "file:line: message".  Launch failures return QSA_ERR_DEVICE
 *    with the HIP error text.  Faults of already-enqueued work surface at the
 *    caller's next synchronisation.
 *  - Supported geometry: heads == 4 and head_dim == 128 ([turing] "Test
 *    Plan"); anything else returns QSA_ERR_UNSUPPORTED.  page_size must be a
 *    positive multiple of compress_ratio.
 *  - Device-side data outside its contract (a page-table entry outside
 *    [0, num_pages), a row_req entry outside [0, num_reqs), a row with
 *    V_r > max_visible) never causes an out-of-bounds access: page ids are
 *    clamped into range, rows with an invalid request select nothing, and V_r
 *    is clamped to max_visible.  The results for such rows are unspecified.
 *  - Inputs must be finite (any finite fp16 value, up to +-65504 in every
 *    head; NaN and Inf are outside the contract).  Scores are exact fp16
 *    products accumulated in fp32, so no finite input overflows them; the
 *    default form stays exact when the per-dimension sum over heads leaves
 *    the fp16 range (it is carried divided by 2 or 4, a power of two).
 *  - Calls are thread-safe.  Library state is a per-device properties cache
 *    and a thread-local error string.
 *  - Indices are logical positions within the request (key j, token t); the
 *    mapping to physical cache slots is the consumer's.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad stride, k not a multiple of cr, unknown flag */
    QSA_ERR_UNSUPPORTED = 2,        /* heads != 4, head_dim != 128, k beyond the selector's limit, device not gfx950 */
    QSA_ERR_WORKSPACE_TOO_SMALL = 3,
    QSA_ERR_DEVICE = 4              /* a HIP call or kernel launch failed */
} qsa_status;

/* flags */
#define QSA_SCORE_RELU 0x1u  /* [spec] form: sum_h relu(q_h . k) times the fp32 value nearest 1/sqrt(head_dim);
                                default is the plain sum_h q_h . k */
#define QSA_OUT_KEYS   0x2u  /* k counts keys and the output holds key indices (no expansion to tokens) */
#define QSA_STREAM_SELECT 0x8u /* qsa_select_paged_tokens: take the streaming arm -- each range of 8,192 keys
                                  reduced to its top-k on chip, then a merge per row -- in place of the
                                  library's choice.  Measured faster for batches of one row per request whose
                                  rows are all long (64k+ tokens) and number 320 or more (about level at
                                  256); slower with short or few rows.  The workspace query must be given the
                                  same flag. */

/* Largest number of selected entries per row (blocks, or keys with
 * QSA_OUT_KEYS) that the selector supports. */
#define QSA_MAX_SELECT 4096

/*
 * qsa_score_paged -- the scorer alone ([turing] "Purpose": FP16 inputs, FP32
 * accumulation; [spec]: one score per (row, key), summed over index heads).
 *
 *  q            device fp16 [rows][heads][head_dim], row-major, contiguous.
 *  kcache       device fp16 [num_pages][page_size/compress_ratio][head_dim]:
 *               page p holds keys slot 0.. page_size/cr-1 contiguously.
 *  page_table   device int32 [num_reqs][pt_stride]: logical page i of
 *               request q is physical page page_table[q*pt_stride + i]; key j
 *               of request q is slot j % (page_size/cr) of logical page
 *               j / (page_size/cr).  Entries for logical pages at or beyond
 *               ceil(V/(page_size/cr)) of a request's longest row are never read.
 *  pt_stride    row stride of page_table in entries; must be >=
 *               ceil(max_visible / (page_size/cr)).
 *  num_pages    number of physical pages in kcache (>= 1).
 *  num_reqs     number of page-table rows (>= 1).
 *  row_req      device int32 [rows]: request of each row; NULL means every
 *               row belongs to request 0.
 *  pos          device int32 [rows]: absolute token position of each row.
 *               V_r = (pos[r]+1)/compress_ratio keys are visible (0 if pos<0).
 *  rows         number of query rows (0 is a no-op).
 *  max_visible  host upper bound on every V_r (the top-k op's `columns` in
 *               [thor]); sizes the launch.
 *  flags        0 or QSA_SCORE_RELU.
 *  scores       device fp32 [rows][ld_scores]: entry (r, j) is written for
 *               j < V_r only; every other entry is left untouched.
 *  ld_scores    row stride of scores in floats, >= max_visible.
 */
qsa_status qsa_score_paged(const void* q, const void* kcache, const int32_t* page_table,
                           int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                           const int32_t* row_req, const int32_t* pos, int32_t rows,
                           int32_t heads, int32_t head_dim, int32_t page_size,
                           int32_t compress_ratio, int32_t max_visible, uint32_t flags,
                           float* scores, int64_t ld_scores, void* stream);

/*
 * qsa_topk_rows -- the exact selector alone ([thor] "What happens": the top-k
 * op over the score matrix, the per-row visible count, k and the column
 * count; [turing] "Purpose": exact, lexicographic, deterministic on ties).
 *
 *  scores       device fp32 [rows][ld_scores]; only entries j < visible[r]
 *               are read.  -0 and +0 are equal (a tie broken by index).
 *  visible      device int32 [rows] or NULL (then every row has max_visible
 *               candidates); values are clamped to [0, max_visible].
 *  rows         number of rows (0 is a no-op).
 *  max_visible  host upper bound on visible[r]; ld_scores >= max_visible.
 *  k            entries to select per row, 1 <= k <= QSA_MAX_SELECT.
 *  out          device int32 [rows][k]: out[r][i] is the key index of rank i
 *               (higher score first, lower index on ties), -1 for
 *               i >= min(k, visible[r]).
 *  workspace    device scratch of at least qsa_topk_rows_workspace_size(...)
 *               bytes (may be NULL when that size is 0); its contents on entry
 *               and exit are unspecified.
 */
qsa_status qsa_topk_rows(const float* scores, int64_t ld_scores, const int32_t* visible,
                         int32_t rows, int32_t max_visible, int32_t k, int32_t* out,
                         void* workspace, size_t workspace_bytes, void* stream);

size_t qsa_topk_rows_workspace_size(int32_t rows, int32_t max_visible, int32_t k);

/*
 * qsa_select_paged_tokens -- the whole indexer ([thor] "What happens": the
 * indexer forward's entry point; [turing] "Test Plan": 4 heads, head dim 128,
 * compress ratio 4, top-k 2,048 tokens; [spec]: raw tokens at ratio
 * granularity, every candidate selected below the budget).
 *
 *  q .. max_visible   as for qsa_score_paged.
 *  k            output entries per row.  Default: tokens; k must be a
 *               multiple of compress_ratio and k/cr blocks are selected
 *               (1 <= k/cr <= QSA_MAX_SELECT).  With QSA_OUT_KEYS: keys,
 *               1 <= k <= QSA_MAX_SELECT.
 *  flags        QSA_SCORE_RELU, QSA_OUT_KEYS and/or QSA_STREAM_SELECT.
 *  out          device int32 [rows][k]: rank-ordered blocks, each expanded to
 *               tokens cr*j .. cr*j+cr-1 ascending (or key j with
 *               QSA_OUT_KEYS); -1 after the min(k/cr, V_r) selected blocks.
 *  workspace    device scratch of at least
 *               qsa_select_paged_tokens_workspace_size(...) bytes, queried
 *               with the same flags and under the same debug-force mask as
 *               the call (the arms' workspaces differ in size).
 */
qsa_status qsa_select_paged_tokens(const void* q, const void* kcache, const int32_t* page_table,
                                   int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                                   const int32_t* row_req, const int32_t* pos, int32_t rows,
                                   int32_t heads, int32_t head_dim, int32_t page_size,
                                   int32_t compress_ratio, int32_t max_visible, int32_t k,
                                   uint32_t flags, int32_t* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

size_t qsa_select_paged_tokens_workspace_size(int32_t rows, int32_t num_reqs, int32_t max_visible,
                                              int32_t compress_ratio, int32_t k, uint32_t flags);

/*
 * qsa_select_paged_tokens_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): qsa_select_paged_tokens with the same arguments and
 * results, minus the workspace.  Its scratch is a static device array of
 * QSA_NOALLOC_SCRATCH_BYTES per device, held from the library's first use on
 * that device until the process ends; the call allocates nothing.
 *
 *  - Returns QSA_ERR_UNSUPPORTED, enqueuing nothing, when the call needs more
 *    scratch than that (qsa_select_paged_tokens_workspace_size(...) bytes;
 *    every benchmark configuration of this library fits).
 *  - Every call on one device shares that device's array.  Calls that may
 *    overlap on one device (other streams, other threads, unordered graph
 *    nodes) race on it and give undefined results; calls ordered on one
 *    stream are safe.  The array's contents carry over between calls and are
 *    never relied on: each call writes what it reads.
 */
#define QSA_NOALLOC_SCRATCH_BYTES (96ull << 20)
qsa_status qsa_select_paged_tokens_noalloc(const void* q, const void* kcache, const int32_t* page_table,
                                           int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                                           const int32_t* row_req, const int32_t* pos, int32_t rows,
                                           int32_t heads, int32_t head_dim, int32_t page_size,
                                           int32_t compress_ratio, int32_t max_visible, int32_t k,
                                           uint32_t flags, int32_t* out, void* stream);

/*
 * qsa_sparse_attention -- the consumer of the selection ([spec] op survey:
 * plain GQA, 24 query heads over 2 KV heads, head_dim 256; [spec] "The
 * component deep-dives, and two corrections to the above": the consumer
 * attends to the raw tokens the indexer selected).  For every row r and query
 * head h: out[r][h] = sum_t softmax_t(scale * q[r][h] . K[t]) V[t] over the
 * tokens t listed in tokens[r], K and V of KV head h / (q_heads / kv_heads).
 *
 *  q            device fp16 [rows][q_heads][head_dim].
 *  k_cache      device fp16 [num_pages][page_size][kv_heads][head_dim]: token t
 *               of request q is slot t % page_size of page
 *               page_table[q][t / page_size].
 *  v_cache      device fp16, the same layout.
 *  page_table, pt_stride, num_pages, num_reqs, row_req   as for
 *               qsa_score_paged (row_req NULL: every row is request 0).
 *  tokens       device int32 [rows][k]: logical token positions (for example
 *               the output of qsa_select_paged_tokens); entries < 0 are
 *               skipped.  Positions past the page table and page ids outside
 *               [0, num_pages) are clamped (never an out-of-bounds access).
 *  scale        softmax scale, e.g. 1/sqrt(head_dim).
 *  out          device fp32 [rows][q_heads][head_dim]; a row with no token
 *               gets zeros.
 *  workspace    device scratch of at least
 *               qsa_sparse_attention_workspace_size(rows, q_heads, kv_heads,
 *               head_dim, k) bytes, 16-byte aligned (may be NULL when that
 *               size is 0).  With fewer than 512 (row, KV head) pairs each
 *               row's list is split over several workgroups, whose partial
 *               softmax states a second kernel merges; the workspace holds
 *               them.
 *  Supported: head_dim == 256, q_heads a multiple of kv_heads with at most 16
 *  query heads per KV head, num_pages * page_size * kv_heads < 2^32.
 *  Asynchronous on `stream`.
 */
size_t qsa_sparse_attention_workspace_size(int32_t rows, int32_t q_heads, int32_t kv_heads,
                                           int32_t head_dim, int32_t k);
qsa_status qsa_sparse_attention(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* page_table, int64_t pt_stride, int32_t num_pages,
                                int32_t num_reqs, const int32_t* row_req, const int32_t* tokens,
                                int32_t k, int32_t rows, int32_t q_heads, int32_t kv_heads,
                                int32_t head_dim, int32_t page_size, float scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_compress_keys -- the producer of the side cache the scorer reads
 * ([spec] "The component deep-dives, and two corrections to the above": one
 * stored state per compress_ratio tokens, written at the token whose
 * (position + 1) is a multiple of the ratio; a pooled key, RMSNorm on it, RoPE
 * at the block-start position).  The pages name no pooling for this model;
 * the library takes the mean.  For block c of request q (tokens cr*c ..
 * cr*c+cr-1, raw keys x_0 .. x_{cr-1}):
 *   m = (x_0 + ... + x_{cr-1}) / cr;  y_i = w_i m_i / sqrt(mean_j m_j^2 + eps);
 *   RoPE on y's leading rope_dim values at p0 = cr*c: the pair (a, b) at
 *   frequency index i turns into (a cos - b sin, b cos + a sin),
 *   angle p0 * rope_base^(-2i/rope_dim); pairs (i, i + rope_dim/2), or
 *   (2i, 2i+1) with QSA_ROPE_INTERLEAVED;
 * rounded to fp16 and stored in slot c % (page_size/cr) of physical page
 * page_table[q][c / (page_size/cr)] of kcache (the layout qsa_score_paged
 * reads).
 *
 *  k_tok        device fp16 [tokens][head_dim]: the raw index keys of this
 *               call's tokens.  Each request's tokens form one run of
 *               consecutive positions in consecutive slots (a prefill chunk,
 *               or a decode token); across calls a request's positions
 *               arrive in order, each once.
 *  tok_req      device int32 [tokens]: request of each token; NULL means
 *               request 0.  Tokens with a request outside [0, num_reqs) or a
 *               negative position are ignored.
 *  tok_pos      device int32 [tokens]: absolute position of each token.
 *  head_dim     must be 128.
 *  norm_w       device fp32 [head_dim] RMSNorm weights, or NULL for 1.
 *  eps          RMSNorm epsilon (finite, >= 0).
 *  rope_dim     0 (no rotation) .. head_dim, a multiple of 16.
 *  rope_base    RoPE base (finite, > 0; unused when rope_dim is 0).
 *  flags        0 or QSA_ROPE_INTERLEAVED.
 *  state        device fp16 [num_reqs][compress_ratio][head_dim], owned by
 *               the caller and kept between calls: the raw keys of each
 *               request's open block.  Read and written by the call; its
 *               initial contents never matter for a request whose positions
 *               start at 0.  May be NULL when compress_ratio is 1.
 *  kcache       device fp16 [num_pages][page_size/cr][head_dim]: written at
 *               the slots of the blocks that close in this call only.
 *  page_table, pt_stride, num_pages, num_reqs   as for qsa_score_paged;
 *               a block whose logical page is >= pt_stride is not stored,
 *               page ids are clamped into [0, num_pages).
 *  Supported: 1 <= compress_ratio <= 64, page_size a multiple of it.
 *  Two kernels on `stream`; no workspace.
 */
#define QSA_ROPE_INTERLEAVED 0x4u
qsa_status qsa_compress_keys(const void* k_tok, const int32_t* tok_req, const int32_t* tok_pos,
                             int32_t tokens, int32_t head_dim, const float* norm_w, float eps,
                             int32_t rope_dim, double rope_base, uint32_t flags, void* state,
                             void* kcache, const int32_t* page_table, int64_t pt_stride,
                             int32_t num_pages, int32_t num_reqs, int32_t page_size,
                             int32_t compress_ratio, void* stream);

/* Description of the last failure on the calling thread, "file:line: message"
 * ("" if none).  The pointer stays valid until the thread's next library call. */
const char* qsa_last_error(void);

/* Name of the execution arm the calling thread's last successful
 * qsa_select_paged_tokens call used ("two_pass", "fused" or "stream"); ""
 * before any call. */
const char* qsa_last_path(void);

/* Library version string. */
const char* qsa_version(void);

/* Instrumentation for benchmarks and profilers.  Arms the calling thread's
 * next qsa_select_paged_tokens or qsa_compress_keys call to record events[0]
 * on its stream before its first kernel and events[i] after its i-th kernel,
 * for at most n events (hipEvent_t handles created and owned by the caller,
 * passed as void*; they must stay valid until that call returns).  The call
 * disarms the hook; qsa_debug_events_recorded() then returns how many events
 * it recorded.  Kernel order: two-pass arm = scorer, selector; fused arm =
 * head-sum preparation (default form; in the relu form the tile counts of
 * calls with several requests, else nothing), sampling
 * scorer, threshold, filtering scorer, final select; streaming arm = chunk
 * top-k, merge; producer = block compression, staging of open
 * blocks (none when compress_ratio is 1). */
qsa_status qsa_debug_record_events(void* const* events, int32_t n);
int32_t qsa_debug_events_recorded(void);

/* Overrides of the library's own choices, for tests and benchmarks that must
 * drive one execution arm or one scorer deliberately.  Process-wide (every
 * thread and device) until the next qsa_debug_force call; mask 0 restores the
 * library's choices.  The workspace-size queries follow the forced arm.
 * Conflicting or unknown bits return QSA_ERR_INVALID_ARGUMENT and change
 * nothing.  The library reads no environment variables. */
#define QSA_DEBUG_FORCE_TWO_PASS 0x1u   /* qsa_select_paged_tokens: the two-pass arm */
#define QSA_DEBUG_FORCE_FUSED    0x2u   /* ... the fused arm */
#define QSA_DEBUG_FORCE_FALLBACK 0x4u   /* the fused arm, every row on its exact recompute path */
#define QSA_DEBUG_FORCE_TILES    0x8u   /* materialising scorer: the row-tiled kernel */
#define QSA_DEBUG_FORCE_GROUPS   0x10u  /* materialising scorer: the windowed kernel */
#define QSA_DEBUG_FORCE_REDO     0x20u  /* the fused arm, every row's final select in its second pass */
#define QSA_DEBUG_FORCE_STREAM   0x40u  /* qsa_select_paged_tokens: the streaming arm */
qsa_status qsa_debug_force(uint32_t mask);
uint32_t qsa_debug_forced(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
