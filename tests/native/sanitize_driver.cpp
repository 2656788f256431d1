// Host-side checks run under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by tests/test_sanitize.py; no GPU is touched).
//
// 1. The CPU oracle on small seeded inputs: the whole indexer equals its
//    score and select steps composed, and every row selects min(kb, V)
//    blocks in rank order (the sanitizers watch every buffer access).
// 2. The library's host validation: each entry point refuses malformed
//    arguments with the documented status and a "file:line: message" error
//    before any device call; workspace queries and zero-row calls need no
//    device.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <random>
#include <vector>

#include "qsa.h"

extern "C" {
void oracle_score_paged(const uint16_t* q, const uint16_t* kcache, const int32_t* page_table, int64_t pt_stride,
                        const int32_t* row_req, const int32_t* pos, int32_t rows, int32_t heads, int32_t head_dim,
                        int32_t page_size, int32_t compress_ratio, uint32_t flags, float* scores, int64_t ld,
                        int32_t nthreads);
void oracle_select_rows(const float* scores, int64_t ld, const int32_t* visible, int32_t rows, int32_t k,
                        int32_t* out, int32_t nthreads);
void oracle_select_paged_tokens(const uint16_t* q, const uint16_t* kcache, const int32_t* page_table,
                                int64_t pt_stride, const int32_t* row_req, const int32_t* pos, int32_t rows,
                                int32_t heads, int32_t head_dim, int32_t page_size, int32_t compress_ratio, int32_t k,
                                uint32_t flags, int32_t* out, int32_t nthreads);
int32_t oracle_visible_keys(int32_t pos, int32_t cr);
}

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            ++failures;                                    \
        }                                                  \
    } while (0)

// small integers -2..2 as fp16 bit patterns (exact)
static uint16_t half_of_int(int v) {
    static const uint16_t bits[5] = {0xC000, 0xBC00, 0x0000, 0x3C00, 0x4000};
    return bits[v + 2];
}

static void oracle_checks() {
    std::mt19937 rng(7);
    const int heads = 4, dim = 128, cr = 4, page_size = 64, kpp = page_size / cr;
    const int ctx[3] = {260, 97, 1030};
    const int rows_per[3] = {5, 3, 7};
    const int reqs = 3;
    int pages = 0, stride = 0;
    for (int i = 0; i < reqs; ++i) {
        const int n = (ctx[i] + page_size - 1) / page_size;
        pages += n;
        stride = n > stride ? n : stride;
    }
    pages += 2;  // unreferenced pages
    std::vector<int32_t> page_table((size_t)reqs * stride, 0), row_req, pos;
    std::vector<int32_t> perm(pages);
    for (int i = 0; i < pages; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), rng);
    int next = 0;
    for (int i = 0; i < reqs; ++i) {
        const int n = (ctx[i] + page_size - 1) / page_size;
        for (int p = 0; p < n; ++p) page_table[(size_t)i * stride + p] = perm[next++];
        for (int r = 0; r < rows_per[i]; ++r) {
            row_req.push_back(i);
            pos.push_back(ctx[i] - rows_per[i] + r);
        }
    }
    const int rows = (int)pos.size();
    std::uniform_int_distribution<int> d5(-2, 2);
    std::vector<uint16_t> q((size_t)rows * heads * dim), kc((size_t)pages * kpp * dim);
    for (auto& x : q) x = half_of_int(d5(rng));
    for (auto& x : kc) x = half_of_int(d5(rng));

    int vmax = 0;
    std::vector<int32_t> vis(rows);
    for (int r = 0; r < rows; ++r) {
        vis[r] = oracle_visible_keys(pos[r], cr);
        vmax = vis[r] > vmax ? vis[r] : vmax;
    }
    for (uint32_t flags : {0u, 1u}) {
        for (int k : {4, 64, 512}) {
            const int kb = k / cr;
            std::vector<float> scores((size_t)rows * vmax, 0.0f);
            oracle_score_paged(q.data(), kc.data(), page_table.data(), stride, row_req.data(), pos.data(), rows,
                               heads, dim, page_size, cr, flags, scores.data(), vmax, 3);
            std::vector<int32_t> blocks((size_t)rows * kb), full((size_t)rows * k);
            oracle_select_rows(scores.data(), vmax, vis.data(), rows, kb, blocks.data(), 3);
            oracle_select_paged_tokens(q.data(), kc.data(), page_table.data(), stride, row_req.data(), pos.data(),
                                       rows, heads, dim, page_size, cr, k, flags, full.data(), 2);
            for (int r = 0; r < rows; ++r) {
                const int want = vis[r] < kb ? vis[r] : kb;
                for (int i = 0; i < kb; ++i) {
                    const int32_t b = blocks[(size_t)r * kb + i];
                    CHECK((i < want) == (b >= 0), "row %d rank %d block %d (V=%d)", r, i, b, vis[r]);
                    if (i > 0 && b >= 0) {
                        const int32_t a = blocks[(size_t)r * kb + i - 1];
                        const float sa = scores[(size_t)r * vmax + a], sb = scores[(size_t)r * vmax + b];
                        CHECK(sa > sb || (sa == sb && a < b), "row %d rank order broken at %d", r, i);
                    }
                    for (int t = 0; t < cr; ++t)
                        CHECK(full[(size_t)r * k + i * cr + t] == (b >= 0 ? b * cr + t : -1),
                              "row %d: whole indexer differs from score + select at %d", r, i);
                }
            }
        }
    }
}

static const uintptr_t FAKE = 0x10000;  // aligned, never dereferenced
static const void* fp(uintptr_t off = 0) { return reinterpret_cast<const void*>(FAKE + off); }

struct Sel {
    const void* q = fp();
    const void* kc = fp();
    const int32_t* pt = static_cast<const int32_t*>(fp());
    int64_t pt_stride = 16;
    int32_t num_pages = 16, num_reqs = 1;
    const int32_t* row_req = nullptr;
    const int32_t* pos = static_cast<const int32_t*>(fp());
    int32_t rows = 8, heads = 4, head_dim = 128, page_size = 64, cr = 4, max_visible = 256, k = 64;
    uint32_t flags = 0;
    int32_t* out = static_cast<int32_t*>(const_cast<void*>(fp()));
    void* ws = const_cast<void*>(fp());
    size_t ws_bytes = size_t(1) << 30;
    qsa_status run() const {
        return qsa_select_paged_tokens(q, kc, pt, pt_stride, num_pages, num_reqs, row_req, pos, rows, heads, head_dim,
                                       page_size, cr, max_visible, k, flags, out, ws, ws_bytes, nullptr);
    }
    qsa_status run_noalloc() const {
        return qsa_select_paged_tokens_noalloc(q, kc, pt, pt_stride, num_pages, num_reqs, row_req, pos, rows, heads,
                                               head_dim, page_size, cr, max_visible, k, flags, out, nullptr);
    }
};

static void expect(qsa_status got, qsa_status want, const char* what) {
    CHECK(got == want, "%s: status %d, expected %d (%s)", what, (int)got, (int)want, qsa_last_error());
    if (want != QSA_OK) {
        const char* e = qsa_last_error();
        CHECK(e && std::strstr(e, "qsa_api.hip:") == e, "%s: error text '%s' lacks file:line", what, e ? e : "");
    }
}

static void abi_checks() {
    // workspace queries are pure host arithmetic
    CHECK(qsa_select_paged_tokens_workspace_size(0, 1, 100, 4, 64, 0) == 0, "zero rows needs no workspace");
    CHECK(qsa_select_paged_tokens_workspace_size(1616, 1, 46000, 4, 2048, 0) > 0, "kernel shape workspace");
    CHECK(qsa_select_paged_tokens_workspace_size(256, 256, 46000, 4, 2048, 0) >= (size_t)256 * 46000 * 4,
          "decode workspace holds the score matrix");

    struct Case {
        const char* what;
        void (*mod)(Sel&);
        qsa_status want;
    };
    const Case cases[] = {
        {"heads", [](Sel& s) { s.heads = 8; }, QSA_ERR_UNSUPPORTED},
        {"head_dim", [](Sel& s) { s.head_dim = 64; }, QSA_ERR_UNSUPPORTED},
        {"k not a multiple of cr", [](Sel& s) { s.k = 63; }, QSA_ERR_INVALID_ARGUMENT},
        {"k zero", [](Sel& s) { s.k = 0; }, QSA_ERR_INVALID_ARGUMENT},
        {"k beyond the selector", [](Sel& s) { s.k = 4 * (QSA_MAX_SELECT + 1); }, QSA_ERR_UNSUPPORTED},
        {"null q", [](Sel& s) { s.q = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"null kcache", [](Sel& s) { s.kc = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"null page table", [](Sel& s) { s.pt = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"null pos", [](Sel& s) { s.pos = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"null out", [](Sel& s) { s.out = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"null workspace", [](Sel& s) { s.ws = nullptr; }, QSA_ERR_INVALID_ARGUMENT},
        {"small workspace", [](Sel& s) { s.ws_bytes = 16; }, QSA_ERR_WORKSPACE_TOO_SMALL},
        {"page size", [](Sel& s) { s.page_size = 66; }, QSA_ERR_INVALID_ARGUMENT},
        {"compress ratio", [](Sel& s) { s.cr = 0; }, QSA_ERR_INVALID_ARGUMENT},
        {"pt_stride", [](Sel& s) { s.pt_stride = 15; }, QSA_ERR_INVALID_ARGUMENT},
        {"num_pages", [](Sel& s) { s.num_pages = 0; }, QSA_ERR_INVALID_ARGUMENT},
        {"num_reqs", [](Sel& s) { s.num_reqs = 0; }, QSA_ERR_INVALID_ARGUMENT},
        {"rows", [](Sel& s) { s.rows = -1; }, QSA_ERR_INVALID_ARGUMENT},
        {"max_visible", [](Sel& s) { s.max_visible = -1; }, QSA_ERR_INVALID_ARGUMENT},
        {"flags", [](Sel& s) { s.flags = 0x10; }, QSA_ERR_INVALID_ARGUMENT},
        {"misaligned q", [](Sel& s) { s.q = fp(4); }, QSA_ERR_INVALID_ARGUMENT},
    };
    for (const Case& c : cases) {
        Sel s;
        c.mod(s);
        expect(s.run(), c.want, c.what);
        if (std::strcmp(c.what, "null workspace") && std::strcmp(c.what, "small workspace"))
            expect(s.run_noalloc(), c.want, c.what);
    }
    {
        Sel s;
        s.rows = 0;
        s.q = s.kc = nullptr;
        s.out = nullptr;
        s.ws = nullptr;
        s.ws_bytes = 0;
        expect(s.run(), QSA_OK, "zero rows");
        expect(s.run_noalloc(), QSA_OK, "zero rows, no workspace");
    }
    {
        Sel s;  // larger than the allocation-free entry point's scratch
        s.rows = 4096;
        s.max_visible = 200000;
        s.pt_stride = 12500;
        s.num_pages = 20000;
        s.k = 2048;
        expect(s.run_noalloc(), QSA_ERR_UNSUPPORTED, "noalloc beyond its scratch");
    }
    float* scores = static_cast<float*>(const_cast<void*>(fp()));
    expect(qsa_score_paged(fp(), fp(), static_cast<const int32_t*>(fp()), 16, 16, 1, nullptr,
                           static_cast<const int32_t*>(fp()), 8, 4, 128, 64, 4, 256, 0, scores, 255, nullptr),
           QSA_ERR_INVALID_ARGUMENT, "score ld below max_visible");
    expect(qsa_score_paged(fp(), fp(), static_cast<const int32_t*>(fp()), 16, 16, 1, nullptr,
                           static_cast<const int32_t*>(fp()), 8, 4, 128, 64, 4, 256, QSA_OUT_KEYS, scores, 256,
                           nullptr),
           QSA_ERR_INVALID_ARGUMENT, "score flags");
    int32_t* out = static_cast<int32_t*>(const_cast<void*>(fp()));
    expect(qsa_topk_rows(scores, 100, nullptr, 4, 100, 0, out, nullptr, 0, nullptr), QSA_ERR_INVALID_ARGUMENT,
           "topk k");
    expect(qsa_topk_rows(scores, 99, nullptr, 4, 100, 8, out, nullptr, 0, nullptr), QSA_ERR_INVALID_ARGUMENT,
           "topk ld");
    expect(qsa_topk_rows(scores, 100, nullptr, 0, 100, 8, nullptr, nullptr, 0, nullptr), QSA_OK, "topk zero rows");
    expect(qsa_debug_force(0x80), QSA_ERR_INVALID_ARGUMENT, "unknown debug bits");
    expect(qsa_debug_force(QSA_DEBUG_FORCE_STREAM | QSA_DEBUG_FORCE_TWO_PASS), QSA_ERR_INVALID_ARGUMENT,
           "conflicting arms (streaming)");
    expect(qsa_debug_force(QSA_DEBUG_FORCE_TWO_PASS | QSA_DEBUG_FORCE_FUSED), QSA_ERR_INVALID_ARGUMENT,
           "conflicting arms");
    CHECK(qsa_debug_forced() == 0, "a refused mask changes nothing");
    expect(qsa_compress_keys(fp(), nullptr, static_cast<const int32_t*>(fp()), 4, 64, nullptr, 1e-6f, 128, 1e4, 0,
                             const_cast<void*>(fp()), const_cast<void*>(fp()), static_cast<const int32_t*>(fp()), 4,
                             4, 1, 64, 4, nullptr),
           QSA_ERR_UNSUPPORTED, "producer head_dim");
    expect(qsa_sparse_attention(fp(), fp(), fp(), static_cast<const int32_t*>(fp()), 16, 16, 1, nullptr,
                                static_cast<const int32_t*>(fp()), 2048, 8, 24, 2, 128, 64, 0.0625f, scores,
                                const_cast<void*>(fp()), size_t(1) << 30, nullptr),
           QSA_ERR_UNSUPPORTED, "consumer head_dim");
}

int main() {
    oracle_checks();
    abi_checks();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("sanitized host checks passed\n");
    return 0;
}
