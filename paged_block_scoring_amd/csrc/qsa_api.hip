// qsa_api.hip -- the C ABI declared in include/qsa.h: argument validation,
// device check, workspace carving and kernel launches.
//
// Error behaviour follows "qwen4_exp QSA cooperative_topk cannot launch on
// NVIDIA Thor (sm_110): cluster misconfiguration", section "What happens": a
// failure is reported with the source location and the launch error text.
// Here every argument is checked on the host before anything is enqueued, and
// the device is identified by its real architecture name and limits rather
// than a capability proxy (the same page, section "What the source says").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/qsa.h"
#include "qsa_internal.hpp"

#define QSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[1024] = "";
thread_local const char* g_path = "";
thread_local void* const* g_events = nullptr;  // armed instrumentation events
thread_local int32_t g_nevents = 0;
thread_local int32_t g_recorded = 0;

// Records the next armed event (if any) on `s`.
hipError_t mark(hipStream_t s) {
    if (g_events && g_recorded < g_nevents) return hipEventRecord(static_cast<hipEvent_t>(g_events[g_recorded++]), s);
    return hipSuccess;
}

qsa_status fail_at(const char* file, int line, qsa_status code, const char* fmt, ...) {
    const char* base = strrchr(file, '/');
    base = base ? base + 1 : file;
    int n = snprintf(g_err, sizeof g_err, "%s:%d: ", base, line);
    if (n < 0 || n >= (int)sizeof g_err) n = 0;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err + n, sizeof g_err - (size_t)n, fmt, ap);
    va_end(ap);
    return code;
}

#define FAIL(code, ...) return fail_at(__FILE__, __LINE__, (code), __VA_ARGS__)
#define REQUIRE(cond, code, ...) \
    do {                         \
        if (!(cond)) FAIL((code), __VA_ARGS__); \
    } while (0)
#define HIP_CHECK(expr)                                                                         \
    do {                                                                                        \
        hipError_t e_ = (expr);                                                                 \
        if (e_ != hipSuccess) FAIL(QSA_ERR_DEVICE, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

constexpr int kMaxDevices = 64;
struct DeviceInfo {
    std::atomic<bool> probed{false};  // set (release) once the fields below are final
    bool supported = false;
    int cus = 0;
    size_t lds = 0;
    char arch[64] = "";
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Arm and scorer overrides set by qsa_debug_force (QSA_DEBUG_FORCE_* bits).
std::atomic<uint32_t> g_force{0};

// Identify the current device once: the kernels are written for gfx950
// (CDNA4) and its 64-wide wavefronts, 16x16x32 f16 MFMA and 160 KB LDS.
// After the first call per device this is one hipGetDevice and one load.
qsa_status check_device(const DeviceInfo** out) {
    int dev = -1;
    HIP_CHECK(hipGetDevice(&dev));
    REQUIRE(dev >= 0 && dev < kMaxDevices, QSA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    DeviceInfo& d = g_dev[dev];
    if (!d.probed.load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(g_dev_mu);
        if (!d.probed.load(std::memory_order_relaxed)) {
            hipDeviceProp_t p;
            HIP_CHECK(hipGetDeviceProperties(&p, dev));
            snprintf(d.arch, sizeof d.arch, "%s", p.gcnArchName);
            d.cus = p.multiProcessorCount;
            d.lds = p.sharedMemPerBlock;
            d.supported = strncmp(d.arch, "gfx950", 6) == 0 && p.warpSize == 64 && d.lds >= 64 * 1024;
            d.probed.store(true, std::memory_order_release);
        }
    }
    REQUIRE(d.supported, QSA_ERR_UNSUPPORTED,
            "device %d is %s; this library is built for gfx950 (MI355X)", dev, d.arch);
    *out = &d;
    return QSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Common checks of the paged inputs (everything qsa_score_paged and
// qsa_select_paged_tokens share).
qsa_status check_paged(const void* q, const void* kcache, const int32_t* page_table, int64_t pt_stride,
                       int32_t num_pages, int32_t num_reqs, const int32_t* pos, int32_t rows,
                       int32_t heads, int32_t head_dim, int32_t page_size, int32_t compress_ratio,
                       int32_t max_visible) {
    REQUIRE(rows >= 0, QSA_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %d)", rows);
    REQUIRE(heads == 4, QSA_ERR_UNSUPPORTED, "heads must be 4 (got %d)", heads);
    REQUIRE(head_dim == 128, QSA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
    REQUIRE(compress_ratio >= 1, QSA_ERR_INVALID_ARGUMENT, "compress_ratio must be >= 1 (got %d)",
            compress_ratio);
    REQUIRE(page_size >= 1 && page_size % compress_ratio == 0, QSA_ERR_INVALID_ARGUMENT,
            "page_size (%d) must be a positive multiple of compress_ratio (%d)", page_size, compress_ratio);
    REQUIRE(max_visible >= 0, QSA_ERR_INVALID_ARGUMENT, "max_visible must be >= 0 (got %d)", max_visible);
    REQUIRE(num_pages >= 1, QSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", num_pages);
    REQUIRE(num_reqs >= 1, QSA_ERR_INVALID_ARGUMENT, "num_reqs must be >= 1 (got %d)", num_reqs);
    const int64_t kpp = page_size / compress_ratio;
    REQUIRE(pt_stride >= ceil_div(max_visible, kpp) && pt_stride >= 1, QSA_ERR_INVALID_ARGUMENT,
            "pt_stride (%lld) must be >= ceil(max_visible / keys_per_page) = %lld", (long long)pt_stride,
            (long long)ceil_div(max_visible, kpp));
    REQUIRE((int64_t)num_pages * kpp <= (int64_t)UINT32_MAX, QSA_ERR_UNSUPPORTED,
            "num_pages * keys_per_page (%lld) exceeds 2^32 keys", (long long)num_pages * kpp);
    if (rows == 0) return QSA_OK;
    REQUIRE(q && kcache && page_table && pos, QSA_ERR_INVALID_ARGUMENT,
            "null pointer: q=%p kcache=%p page_table=%p pos=%p", q, kcache, (const void*)page_table,
            (const void*)pos);
    REQUIRE(aligned16(q) && aligned16(kcache), QSA_ERR_INVALID_ARGUMENT,
            "q and kcache must be 16-byte aligned");
    return QSA_OK;
}

qsa::PagedArgs make_paged(const void* q, const void* kcache, const int32_t* page_table, int64_t pt_stride,
                          int32_t num_pages, int32_t num_reqs, const int32_t* row_req, const int32_t* pos,
                          int32_t rows, int32_t page_size, int32_t compress_ratio, int32_t max_visible,
                          uint32_t flags) {
    qsa::PagedArgs a;
    a.q = static_cast<const _Float16*>(q);
    a.kcache = static_cast<const _Float16*>(kcache);
    a.page_table = page_table;
    a.pt_stride = pt_stride;
    a.num_pages = num_pages;
    a.num_reqs = num_reqs;
    a.row_req = row_req;
    a.pos = pos;
    a.rows = rows;
    a.kpp = page_size / compress_ratio;
    a.cr = compress_ratio;
    a.max_visible = max_visible;
    a.relu = (flags & QSA_SCORE_RELU) != 0;
    return a;
}

// Two-pass arm: fp32 scores [rows][ld] in the workspace, then the selector.
int64_t two_pass_ld(int32_t max_visible) { return ceil_div(max_visible > 0 ? max_visible : 1, 64) * 64; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// scores, then the prepared query head sums
size_t two_pass_scores_bytes(int32_t rows, int32_t max_visible) {
    return align256((size_t)rows * (size_t)two_pass_ld(max_visible) * sizeof(float));
}
size_t two_pass_bytes(int32_t rows, int32_t max_visible) {
    return two_pass_scores_bytes(rows, max_visible) + qsa::qsum_bytes(rows);
}

// Fused arm: sample scores, per-row threshold and candidate count, candidate lists.
struct FusedLayout {
    qsa::FusedPlan plan;
    size_t off_qsum, off_samp, off_thresh, off_count, off_redo, off_cand, total;
};

FusedLayout fused_layout(int32_t rows, int32_t max_visible, int32_t kb) {
    FusedLayout L;
    L.plan = qsa::plan_fused(max_visible, kb);
    size_t o = 0;
    L.off_qsum = o;
    o = align256(o + qsa::qsum_bytes(rows));
    L.off_samp = o;
    o = align256(o + (size_t)rows * (size_t)L.plan.ld_s * sizeof(float));
    L.off_thresh = o;
    o = align256(o + (size_t)rows * sizeof(uint64_t));
    L.off_count = o;
    o = align256(o + (size_t)rows * (size_t)qsa::kCountStride * sizeof(int32_t));
    L.off_redo = o;
    o = align256(o + qsa::redo_bytes(rows));
    L.off_cand = o;
    o = align256(o + (size_t)rows * (size_t)L.plan.cand_cap * sizeof(uint64_t));
    L.total = o;
    return L;
}

enum class Path { TwoPass, Fused, Stream };

// The fused arm scores every key twice over a 1/16 sample but never writes
// the score matrix; it pays off when many rows share each request's keys and
// there is enough work to cover its five launches (measured crossover: rows x
// longest row between 4.2 M and 6.6 M keys).  Few rows per request (decode),
// and small batches, take the two-pass arm.  The streaming arm (chunk top-k
// on chip, then a merge) is taken when the caller asks for it
// (QSA_STREAM_SELECT) or a test forces it: it measured faster on decode
// batches whose rows are all long and slower once short rows join, which the
// row count and the longest row do not tell apart.
constexpr int64_t kFusedMinWork = 5000000;

Path choose_path(int32_t rows, int32_t num_reqs, int32_t max_visible, uint32_t flags) {
    const uint32_t f = g_force.load(std::memory_order_relaxed);
    if (f & QSA_DEBUG_FORCE_TWO_PASS) return Path::TwoPass;
    if (f & (QSA_DEBUG_FORCE_FUSED | QSA_DEBUG_FORCE_FALLBACK | QSA_DEBUG_FORCE_REDO)) return Path::Fused;
    if ((f & QSA_DEBUG_FORCE_STREAM) || (flags & QSA_STREAM_SELECT)) return Path::Stream;
    if (max_visible <= 0) return Path::TwoPass;
    if (rows / (num_reqs > 0 ? num_reqs : 1) < 32) return Path::TwoPass;
    return (int64_t)rows * max_visible >= kFusedMinWork ? Path::Fused : Path::TwoPass;
}

bool force_fallback() { return (g_force.load(std::memory_order_relaxed) & QSA_DEBUG_FORCE_FALLBACK) != 0; }
bool force_redo() { return (g_force.load(std::memory_order_relaxed) & QSA_DEBUG_FORCE_REDO) != 0; }

qsa::ScorerChoice scorer_choice() {
    const uint32_t f = g_force.load(std::memory_order_relaxed);
    if (f & QSA_DEBUG_FORCE_TILES) return qsa::ScorerChoice::Tiles;
    if (f & QSA_DEBUG_FORCE_GROUPS) return qsa::ScorerChoice::Groups;
    return qsa::ScorerChoice::Auto;
}

}  // namespace

QSA_EXPORT const char* qsa_last_error(void) { return g_err; }
QSA_EXPORT const char* qsa_last_path(void) { return g_path; }
QSA_EXPORT const char* qsa_version(void) { return "qsa-mi355x 0.1.0 (gfx950)"; }

QSA_EXPORT qsa_status qsa_debug_record_events(void* const* events, int32_t n) {
    g_err[0] = 0;
    REQUIRE(n >= 0 && (events != nullptr || n == 0), QSA_ERR_INVALID_ARGUMENT, "bad event list");
    g_events = n > 0 ? events : nullptr;
    g_nevents = n;
    g_recorded = 0;
    return QSA_OK;
}

QSA_EXPORT int32_t qsa_debug_events_recorded(void) { return g_recorded; }

QSA_EXPORT qsa_status qsa_debug_force(uint32_t mask) {
    g_err[0] = 0;
    constexpr uint32_t known = QSA_DEBUG_FORCE_TWO_PASS | QSA_DEBUG_FORCE_FUSED | QSA_DEBUG_FORCE_FALLBACK |
                               QSA_DEBUG_FORCE_TILES | QSA_DEBUG_FORCE_GROUPS | QSA_DEBUG_FORCE_REDO |
                               QSA_DEBUG_FORCE_STREAM;
    constexpr uint32_t fused = QSA_DEBUG_FORCE_FUSED | QSA_DEBUG_FORCE_FALLBACK | QSA_DEBUG_FORCE_REDO;
    REQUIRE((mask & ~known) == 0, QSA_ERR_INVALID_ARGUMENT, "unknown debug bits 0x%x", mask & ~known);
    REQUIRE(((mask & QSA_DEBUG_FORCE_TWO_PASS) ? 1 : 0) + ((mask & fused) ? 1 : 0) +
                    ((mask & QSA_DEBUG_FORCE_STREAM) ? 1 : 0) <= 1,
            QSA_ERR_INVALID_ARGUMENT, "at most one of the two-pass, fused and streaming arms can be forced (0x%x)",
            mask);
    REQUIRE(!((mask & QSA_DEBUG_FORCE_TILES) && (mask & QSA_DEBUG_FORCE_GROUPS)), QSA_ERR_INVALID_ARGUMENT,
            "the tiled and the windowed scorer cannot both be forced (0x%x)", mask);
    g_force.store(mask, std::memory_order_relaxed);
    return QSA_OK;
}

QSA_EXPORT uint32_t qsa_debug_forced(void) { return g_force.load(std::memory_order_relaxed); }

QSA_EXPORT qsa_status qsa_score_paged(const void* q, const void* kcache, const int32_t* page_table,
                                      int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                                      const int32_t* row_req, const int32_t* pos, int32_t rows, int32_t heads,
                                      int32_t head_dim, int32_t page_size, int32_t compress_ratio,
                                      int32_t max_visible, uint32_t flags, float* scores, int64_t ld_scores,
                                      void* stream) {
    g_err[0] = 0;
    qsa_status st = check_paged(q, kcache, page_table, pt_stride, num_pages, num_reqs, pos, rows, heads,
                                head_dim, page_size, compress_ratio, max_visible);
    if (st != QSA_OK) return st;
    REQUIRE((flags & ~QSA_SCORE_RELU) == 0, QSA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x for the scorer",
            flags);
    REQUIRE(ld_scores >= max_visible && ld_scores >= 1, QSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) must be >= max_visible (%d)", (long long)ld_scores, max_visible);
    if (rows == 0 || max_visible == 0) return QSA_OK;
    REQUIRE(scores != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: scores");
    const DeviceInfo* dev = nullptr;
    if ((st = check_device(&dev)) != QSA_OK) return st;
    qsa::PagedArgs a = make_paged(q, kcache, page_table, pt_stride, num_pages, num_reqs, row_req, pos, rows,
                                  page_size, compress_ratio, max_visible, flags);
    HIP_CHECK(qsa::launch_score_paged(a, nullptr, scores, ld_scores, dev->cus, scorer_choice(),
                                      static_cast<hipStream_t>(stream)));
    return QSA_OK;
}

QSA_EXPORT size_t qsa_topk_rows_workspace_size(int32_t rows, int32_t max_visible, int32_t k) {
    (void)rows;
    (void)max_visible;
    (void)k;
    return 0;
}

QSA_EXPORT qsa_status qsa_topk_rows(const float* scores, int64_t ld_scores, const int32_t* visible, int32_t rows,
                                    int32_t max_visible, int32_t k, int32_t* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    REQUIRE(rows >= 0, QSA_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %d)", rows);
    REQUIRE(max_visible >= 0, QSA_ERR_INVALID_ARGUMENT, "max_visible must be >= 0 (got %d)", max_visible);
    REQUIRE(k >= 1, QSA_ERR_INVALID_ARGUMENT, "k must be >= 1 (got %d)", k);
    REQUIRE(k <= QSA_MAX_SELECT, QSA_ERR_UNSUPPORTED, "k (%d) exceeds the selector limit %d", k,
            QSA_MAX_SELECT);
    REQUIRE(ld_scores >= max_visible && ld_scores >= 1, QSA_ERR_INVALID_ARGUMENT,
            "ld_scores (%lld) must be >= max_visible (%d)", (long long)ld_scores, max_visible);
    const size_t need = qsa_topk_rows_workspace_size(rows, max_visible, k);
    REQUIRE(workspace_bytes >= need, QSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < required %zu",
            workspace_bytes, need);
    (void)workspace;
    if (rows == 0) return QSA_OK;
    REQUIRE(out != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: out");
    REQUIRE(scores != nullptr || max_visible == 0, QSA_ERR_INVALID_ARGUMENT, "null pointer: scores");
    const DeviceInfo* dev = nullptr;
    qsa_status st = check_device(&dev);
    if (st != QSA_OK) return st;
    qsa::VisibleSource vs;
    vs.visible = visible;
    vs.pos = nullptr;
    vs.row_req = nullptr;
    vs.num_reqs = 1;
    vs.cr = 1;
    vs.max_visible = max_visible;
    HIP_CHECK(qsa::launch_topk_rows(scores, ld_scores, vs, rows, k, 1, k, out,
                                    static_cast<hipStream_t>(stream)));
    return QSA_OK;
}

QSA_EXPORT size_t qsa_sparse_attention_workspace_size(int32_t rows, int32_t q_heads, int32_t kv_heads,
                                                     int32_t head_dim, int32_t k) {
    if (head_dim != 256 || kv_heads < 1 || q_heads < kv_heads) return 0;
    return qsa::attend_workspace_bytes(rows, kv_heads, k);
}

QSA_EXPORT qsa_status qsa_sparse_attention(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* page_table, int64_t pt_stride, int32_t num_pages,
                                           int32_t num_reqs, const int32_t* row_req, const int32_t* tokens,
                                           int32_t k, int32_t rows, int32_t q_heads, int32_t kv_heads,
                                           int32_t head_dim, int32_t page_size, float scale, float* out,
                                           void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    REQUIRE(rows >= 0, QSA_ERR_INVALID_ARGUMENT, "rows must be >= 0 (got %d)", rows);
    REQUIRE(k >= 1, QSA_ERR_INVALID_ARGUMENT, "k must be >= 1 (got %d)", k);
    REQUIRE(head_dim == 256, QSA_ERR_UNSUPPORTED, "head_dim must be 256 (got %d)", head_dim);
    REQUIRE(kv_heads >= 1 && q_heads >= kv_heads && q_heads % kv_heads == 0, QSA_ERR_INVALID_ARGUMENT,
            "q_heads (%d) must be a positive multiple of kv_heads (%d)", q_heads, kv_heads);
    REQUIRE(q_heads / kv_heads <= 16, QSA_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)",
            q_heads / kv_heads);
    REQUIRE(page_size >= 1, QSA_ERR_INVALID_ARGUMENT, "page_size must be >= 1 (got %d)", page_size);
    REQUIRE(num_pages >= 1, QSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", num_pages);
    REQUIRE(num_reqs >= 1, QSA_ERR_INVALID_ARGUMENT, "num_reqs must be >= 1 (got %d)", num_reqs);
    REQUIRE(pt_stride >= 1, QSA_ERR_INVALID_ARGUMENT, "pt_stride must be >= 1 (got %lld)", (long long)pt_stride);
    REQUIRE((uint64_t)num_pages * (uint64_t)page_size * (uint64_t)kv_heads < (1ull << 32), QSA_ERR_UNSUPPORTED,
            "num_pages * page_size * kv_heads must be < 2^32");
    REQUIRE(std::isfinite(scale), QSA_ERR_INVALID_ARGUMENT, "scale must be finite");
    const size_t need = qsa::attend_workspace_bytes(rows, kv_heads, k);
    REQUIRE(workspace_bytes >= need, QSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < required %zu",
            workspace_bytes, need);
    if (rows == 0) return QSA_OK;
    REQUIRE(need == 0 || workspace != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: workspace");
    REQUIRE(need == 0 || aligned16(workspace), QSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    REQUIRE(q && k_cache && v_cache && page_table && tokens && out, QSA_ERR_INVALID_ARGUMENT,
            "null pointer among q, k_cache, v_cache, page_table, tokens, out");
    REQUIRE(aligned16(q) && aligned16(k_cache) && aligned16(v_cache), QSA_ERR_INVALID_ARGUMENT,
            "q, k_cache and v_cache must be 16-byte aligned");
    const DeviceInfo* dev = nullptr;
    qsa_status st = check_device(&dev);
    if (st != QSA_OK) return st;
    HIP_CHECK(qsa::launch_attend(static_cast<const _Float16*>(q), static_cast<const _Float16*>(k_cache),
                                 static_cast<const _Float16*>(v_cache), page_table, pt_stride, num_pages, num_reqs,
                                 row_req, tokens, k, rows, q_heads, kv_heads, page_size, scale, out,
                                 need > 0 ? workspace : nullptr, static_cast<hipStream_t>(stream)));
    return QSA_OK;
}

QSA_EXPORT qsa_status qsa_compress_keys(const void* k_tok, const int32_t* tok_req, const int32_t* tok_pos,
                                        int32_t tokens, int32_t head_dim, const float* norm_w, float eps,
                                        int32_t rope_dim, double rope_base, uint32_t flags, void* state,
                                        void* kcache, const int32_t* page_table, int64_t pt_stride,
                                        int32_t num_pages, int32_t num_reqs, int32_t page_size,
                                        int32_t compress_ratio, void* stream) {
    g_err[0] = 0;
    g_recorded = 0;
    REQUIRE(tokens >= 0, QSA_ERR_INVALID_ARGUMENT, "tokens must be >= 0 (got %d)", tokens);
    REQUIRE(head_dim == 128, QSA_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
    REQUIRE(compress_ratio >= 1, QSA_ERR_INVALID_ARGUMENT, "compress_ratio must be >= 1 (got %d)",
            compress_ratio);
    REQUIRE(compress_ratio <= 64, QSA_ERR_UNSUPPORTED, "compress_ratio must be <= 64 (got %d)", compress_ratio);
    REQUIRE(page_size >= compress_ratio && page_size % compress_ratio == 0, QSA_ERR_INVALID_ARGUMENT,
            "page_size (%d) must be a positive multiple of compress_ratio (%d)", page_size, compress_ratio);
    REQUIRE(rope_dim >= 0 && rope_dim <= head_dim, QSA_ERR_INVALID_ARGUMENT, "rope_dim must be in [0, %d] (got %d)",
            head_dim, rope_dim);
    REQUIRE(rope_dim % 16 == 0, QSA_ERR_UNSUPPORTED, "rope_dim must be a multiple of 16 (got %d)", rope_dim);
    REQUIRE(rope_dim == 0 || (std::isfinite(rope_base) && rope_base > 0.0), QSA_ERR_INVALID_ARGUMENT,
            "rope_base must be finite and > 0");
    REQUIRE(std::isfinite(eps) && eps >= 0.0f, QSA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    REQUIRE((flags & ~QSA_ROPE_INTERLEAVED) == 0, QSA_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", flags);
    REQUIRE(num_pages >= 1, QSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1 (got %d)", num_pages);
    REQUIRE(num_reqs >= 1, QSA_ERR_INVALID_ARGUMENT, "num_reqs must be >= 1 (got %d)", num_reqs);
    REQUIRE(pt_stride >= 1, QSA_ERR_INVALID_ARGUMENT, "pt_stride must be >= 1 (got %lld)", (long long)pt_stride);
    if (tokens == 0) return QSA_OK;
    REQUIRE(k_tok && tok_pos && kcache && page_table, QSA_ERR_INVALID_ARGUMENT,
            "null pointer among k_tok, tok_pos, kcache, page_table");
    REQUIRE(state || compress_ratio == 1, QSA_ERR_INVALID_ARGUMENT, "null pointer: state");
    REQUIRE(aligned16(k_tok) && aligned16(kcache) && (state == nullptr || aligned16(state)),
            QSA_ERR_INVALID_ARGUMENT, "k_tok, kcache and state must be 16-byte aligned");
    const DeviceInfo* dev = nullptr;
    qsa_status st = check_device(&dev);
    if (st != QSA_OK) return st;
    HIP_CHECK(qsa::launch_compress(static_cast<const _Float16*>(k_tok), tok_req, tok_pos, tokens, norm_w, eps,
                                   rope_dim, rope_base, (flags & QSA_ROPE_INTERLEAVED) != 0,
                                   static_cast<_Float16*>(state), static_cast<_Float16*>(kcache), page_table,
                                   pt_stride, num_pages, num_reqs, page_size, compress_ratio, dev->cus,
                                   static_cast<hipStream_t>(stream), mark));
    g_events = nullptr;
    return QSA_OK;
}

QSA_EXPORT size_t qsa_select_paged_tokens_workspace_size(int32_t rows, int32_t num_reqs, int32_t max_visible,
                                                         int32_t compress_ratio, int32_t k, uint32_t flags) {
    if (rows <= 0 || max_visible <= 0 || k < 1 || compress_ratio < 1) return 0;
    const int32_t kb = (flags & QSA_OUT_KEYS) ? k : k / compress_ratio;
    if (kb < 1) return 0;
    const Path p = choose_path(rows, num_reqs, max_visible, flags);
    if (p == Path::Stream) return qsa::stream_bytes(rows, max_visible, kb);
    if (p == Path::Fused) return fused_layout(rows, max_visible, kb).total;
    return two_pass_bytes(rows, max_visible);
}

// Scratch of qsa_select_paged_tokens_noalloc: one array per device, held
// from the library's load on that device until the process ends.  Host code
// never uses the array's name as an address (it names a host-side stand-in);
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {

// Everything qsa_select_paged_tokens receives except its workspace.
struct SelectCall {
    const void* q;
    const void* kcache;
    const int32_t* page_table;
    int64_t pt_stride;
    int32_t num_pages, num_reqs;
    const int32_t* row_req;
    const int32_t* pos;
    int32_t rows, heads, head_dim, page_size, compress_ratio, max_visible, k;
    uint32_t flags;
    int32_t* out;
};

// Host checks of a select call (all but the workspace); *need receives the
// workspace bytes the call takes.
qsa_status check_select(const SelectCall& c, size_t* need) {
    qsa_status st = check_paged(c.q, c.kcache, c.page_table, c.pt_stride, c.num_pages, c.num_reqs, c.pos, c.rows,
                                c.heads, c.head_dim, c.page_size, c.compress_ratio, c.max_visible);
    if (st != QSA_OK) return st;
    REQUIRE((c.flags & ~(QSA_SCORE_RELU | QSA_OUT_KEYS | QSA_STREAM_SELECT)) == 0, QSA_ERR_INVALID_ARGUMENT,
            "unknown flags 0x%x", c.flags);
    REQUIRE(c.k >= 1, QSA_ERR_INVALID_ARGUMENT, "k must be >= 1 (got %d)", c.k);
    const bool out_keys = (c.flags & QSA_OUT_KEYS) != 0;
    REQUIRE(out_keys || c.k % c.compress_ratio == 0, QSA_ERR_INVALID_ARGUMENT,
            "k (%d) must be a multiple of compress_ratio (%d) unless QSA_OUT_KEYS is set", c.k, c.compress_ratio);
    const int32_t kb = out_keys ? c.k : c.k / c.compress_ratio;
    REQUIRE(kb <= QSA_MAX_SELECT, QSA_ERR_UNSUPPORTED, "%d selected entries per row exceed the limit %d", kb,
            QSA_MAX_SELECT);
    *need = qsa_select_paged_tokens_workspace_size(c.rows, c.num_reqs, c.max_visible, c.compress_ratio, c.k,
                                                   c.flags);
    return QSA_OK;
}

// The launches of a checked select call with rows > 0 on `workspace` (at
// least the bytes check_select asked for).
qsa_status run_select(const SelectCall& c, void* workspace, const DeviceInfo* dev, hipStream_t s) {
    const bool out_keys = (c.flags & QSA_OUT_KEYS) != 0;
    const int32_t kb = out_keys ? c.k : c.k / c.compress_ratio;
    qsa::PagedArgs a = make_paged(c.q, c.kcache, c.page_table, c.pt_stride, c.num_pages, c.num_reqs, c.row_req,
                                  c.pos, c.rows, c.page_size, c.compress_ratio, c.max_visible, c.flags);
    qsa::VisibleSource vs;
    vs.visible = nullptr;
    vs.pos = c.pos;
    vs.row_req = c.row_req;
    vs.num_reqs = c.num_reqs;
    vs.cr = c.compress_ratio;
    vs.max_visible = c.max_visible;
    const int32_t expand = out_keys ? 1 : c.compress_ratio;
    const Path path = choose_path(c.rows, c.num_reqs, c.max_visible, c.flags);
    if (path == Path::Stream) {
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_stream_select(a, kb, expand, c.k, c.out, workspace, s, mark));
        HIP_CHECK(mark(s));
        g_events = nullptr;
        g_path = "stream";
        return QSA_OK;
    }
    if (path == Path::Fused) {
        const FusedLayout L = fused_layout(c.rows, c.max_visible, kb);
        unsigned char* w = static_cast<unsigned char*>(workspace);
        float* samp = reinterpret_cast<float*>(w + L.off_samp);
        uint64_t* thresh = reinterpret_cast<uint64_t*>(w + L.off_thresh);
        int32_t* count = reinterpret_cast<int32_t*>(w + L.off_count);
        int32_t* redo = reinterpret_cast<int32_t*>(w + L.off_redo);
        uint64_t* cand = reinterpret_cast<uint64_t*>(w + L.off_cand);
        // (the relu form uses the head-sum buffer for its tile counts only)
        _Float16* qsum = reinterpret_cast<_Float16*>(w + L.off_qsum);
        const int cus = dev->cus;
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_qsum_prep(a, qsum, s));
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_score_store(a, qsum, L.plan.stride, false, samp, L.plan.ld_s, cus, s));
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_sample_threshold(samp, L.plan.ld_s, vs, L.plan, force_fallback(), thresh, count, redo,
                                               c.rows, s));
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_score_filter(a, qsum, thresh, cand, count, L.plan.cand_cap, cus, s));
        HIP_CHECK(mark(s));
        HIP_CHECK(qsa::launch_fused_final(a, vs, L.plan, thresh, cand, count, redo, force_redo(), kb, expand, c.k,
                                          c.out, s));
        HIP_CHECK(mark(s));
        g_events = nullptr;
        g_path = "fused";
        return QSA_OK;
    }
    float* scores = static_cast<float*>(workspace);
    const int64_t ld = two_pass_ld(c.max_visible);
    HIP_CHECK(mark(s));
    // (head sums in the default form, tile counts in the relu form)
    _Float16* qsum = reinterpret_cast<_Float16*>(static_cast<unsigned char*>(workspace) +
                                                 two_pass_scores_bytes(c.rows, c.max_visible));
    if (c.max_visible > 0) HIP_CHECK(qsa::launch_score_paged(a, qsum, scores, ld, dev->cus, scorer_choice(), s));
    HIP_CHECK(mark(s));
    HIP_CHECK(qsa::launch_topk_rows(scores, ld, vs, c.rows, kb, expand, c.k, c.out, s));
    HIP_CHECK(mark(s));
    g_events = nullptr;
    g_path = "two_pass";
    return QSA_OK;
}

struct ScratchSlot {
    std::atomic<void*> ptr{nullptr};
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on its first use
// there, with that device current).
qsa_status device_scratch(void** out) {
    int dev = -1;
    HIP_CHECK(hipGetDevice(&dev));
    REQUIRE(dev >= 0 && dev < kMaxDevices, QSA_ERR_UNSUPPORTED, "device index %d out of range", dev);
    void* p = g_scratch[dev].ptr.load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].ptr.load(std::memory_order_relaxed);
        if (p == nullptr) {
            void* found = nullptr;
            HIP_CHECK(hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)));
            REQUIRE(found != nullptr, QSA_ERR_DEVICE, "hipGetSymbolAddress returned no address for the scratch");
            g_scratch[dev].ptr.store(found, std::memory_order_release);
            p = found;
        }
    }
    *out = p;
    return QSA_OK;
}

}  // namespace

QSA_EXPORT qsa_status qsa_select_paged_tokens(const void* q, const void* kcache, const int32_t* page_table,
                                              int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                                              const int32_t* row_req, const int32_t* pos, int32_t rows,
                                              int32_t heads, int32_t head_dim, int32_t page_size,
                                              int32_t compress_ratio, int32_t max_visible, int32_t k,
                                              uint32_t flags, int32_t* out, void* workspace,
                                              size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    g_recorded = 0;
    const SelectCall c{q, kcache, page_table, pt_stride, num_pages, num_reqs, row_req, pos, rows, heads, head_dim,
                       page_size, compress_ratio, max_visible, k, flags, out};
    size_t need = 0;
    qsa_status st = check_select(c, &need);
    if (st != QSA_OK) return st;
    REQUIRE(workspace_bytes >= need, QSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes < required %zu",
            workspace_bytes, need);
    if (rows == 0) return QSA_OK;
    REQUIRE(out != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: out");
    REQUIRE(need == 0 || workspace != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: workspace");
    const DeviceInfo* dev = nullptr;
    if ((st = check_device(&dev)) != QSA_OK) return st;
    return run_select(c, workspace, dev, static_cast<hipStream_t>(stream));
}

QSA_EXPORT qsa_status qsa_select_paged_tokens_noalloc(const void* q, const void* kcache, const int32_t* page_table,
                                                      int64_t pt_stride, int32_t num_pages, int32_t num_reqs,
                                                      const int32_t* row_req, const int32_t* pos, int32_t rows,
                                                      int32_t heads, int32_t head_dim, int32_t page_size,
                                                      int32_t compress_ratio, int32_t max_visible, int32_t k,
                                                      uint32_t flags, int32_t* out, void* stream) {
    g_err[0] = 0;
    g_recorded = 0;
    const SelectCall c{q, kcache, page_table, pt_stride, num_pages, num_reqs, row_req, pos, rows, heads, head_dim,
                       page_size, compress_ratio, max_visible, k, flags, out};
    size_t need = 0;
    qsa_status st = check_select(c, &need);
    if (st != QSA_OK) return st;
    REQUIRE(need <= (size_t)QSA_NOALLOC_SCRATCH_BYTES, QSA_ERR_UNSUPPORTED,
            "this call needs %zu bytes of scratch, more than the %llu the allocation-free entry point holds; "
            "use qsa_select_paged_tokens with a workspace", need, (unsigned long long)QSA_NOALLOC_SCRATCH_BYTES);
    if (rows == 0) return QSA_OK;
    REQUIRE(out != nullptr, QSA_ERR_INVALID_ARGUMENT, "null pointer: out");
    const DeviceInfo* dev = nullptr;
    if ((st = check_device(&dev)) != QSA_OK) return st;
    void* ws = nullptr;
    if ((st = device_scratch(&ws)) != QSA_OK) return st;
    return run_select(c, ws, dev, static_cast<hipStream_t>(stream));
}
