// Host-side checks of the C ABI's argument validation, built with the host
// compilation under AddressSanitizer and UndefinedBehaviorSanitizer (see
// tests/test_sanitized_abi.py).  Every call here must return its error before
// anything is enqueued, so no GPU is needed and no kernel runs; the sanitizers
// watch the validation code itself: dims arithmetic, workspace layout sizes,
// the tree-topology parser, the debug-view pointer arithmetic.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "specverify.h"

namespace {
int g_checks = 0, g_failed = 0;

void expect(bool ok, const char* what, int line) {
    ++g_checks;
    if (!ok) {
        ++g_failed;
        std::fprintf(stderr, "FAILED line %d: %s\n", line, what);
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A non-null, 256-byte-aligned address that is never dereferenced.
void* const F = reinterpret_cast<void*>(uintptr_t(1) << 40);
template <typename T> T* f() { return static_cast<T*>(F); }

sv_dims D(int B, int g, int d, int V, int layout = SV_W_ROWS) { return sv_dims{B, g, d, V, layout}; }

// Reference tree check: parent[t] in [-1, t); depth of the deepest node;
// rows with children.
bool ref_tree(const std::vector<int32_t>& p, int* depth, int* qrows) {
    const int T = (int)p.size();
    if (T < 1 || T > SV_MAX_TREE_NODES) return false;
    std::vector<int> dep(T);
    std::vector<char> has_kid(T + 1, 0);
    *depth = 0;
    for (int t = 0; t < T; ++t) {
        if (p[t] < -1 || p[t] >= t) return false;
        dep[t] = p[t] < 0 ? 1 : dep[p[t]] + 1;
        *depth = dep[t] > *depth ? dep[t] : *depth;
        has_kid[p[t] + 1] = 1;
    }
    *qrows = 0;
    for (char c : has_kid) *qrows += c;
    return true;
}
}  // namespace

int main() {
    const size_t big = (size_t)1 << 50;
    // status strings: every code, and values outside the enum
    for (int s = -3; s < 10; ++s) EXPECT(sv_status_string((sv_status)s) != nullptr);
    EXPECT(sv_abi_version() == SV_ABI_VERSION);

    // dims limits, workspace sizes at the extremes (size arithmetic)
    const sv_dims bad[] = {D(0, 4, 64, 100), D(1, 0, 64, 100), D(1, 33, 64, 100), D(1, 4, 12, 100),
                           D(1, 4, 0, 100), D(1, 4, 64, 0), D(1, 4, 64, (1 << 28) + 1),
                           D((1 << 20) + 1, 1, 8, 1), D(1, 4, 65544, 10), D(-1, 4, 64, 100),
                           D(1 << 20, 32, 8, 1 << 28), D(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX),
                           D(INT32_MIN, 4, 64, 100), D(1, 4, 64, 100, 2), D(1, 4, 64, 100, -1),
                           D(1, 4, 64, 100, INT32_MIN)};
    for (const sv_dims& d : bad) {
        EXPECT(sv_workspace_bytes(d) == 0);
        EXPECT(spec_verify(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(), f<float>(), d,
                           f<int32_t>(), f<int32_t>(), F, big, nullptr) == SV_ERR_DIMS);
        EXPECT(spec_verify_static(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(),
                                  f<float>(), d, f<int32_t>(), f<int32_t>(), nullptr) ==
               SV_ERR_DIMS);
        EXPECT(sv_lmhead(f<uint16_t>(), f<uint16_t>(), d, F, big, nullptr) == SV_ERR_DIMS);
        EXPECT(sv_accept_and_draw(f<int32_t>(), f<float>(), f<float>(), d, f<int32_t>(),
                                  f<int32_t>(), F, big, nullptr) == SV_ERR_DIMS);
        EXPECT(spec_verify_greedy(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), d, f<int32_t>(),
                                  f<int32_t>(), nullptr, F, big, nullptr) == SV_ERR_DIMS);
        EXPECT(spec_verify_sparse_q(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<int32_t>(),
                                    f<float>(), 16, f<float>(), d, f<int32_t>(), f<int32_t>(), F,
                                    big, nullptr) == SV_ERR_DIMS);
    }
    const sv_dims large[] = {D(32767, 32, 65536, 1 << 28), D(1 << 20, 32, 65536, 4096),
                             D(1, 1, 8, 1), D(256, 4, 4096, 128256),
                             D(32767, 32, 65536, 1 << 28, SV_W_TILED)};
    for (const sv_dims& d : large) {
        const size_t w = sv_workspace_bytes(d);
        const size_t R = (size_t)d.B * (d.gamma + 1);
        EXPECT(w >= R * (size_t)d.V * 4 && w % 256 == 0);
        const float *lg = nullptr, *mx = nullptr, *sm = nullptr;
        const int32_t* st = nullptr;
        EXPECT(sv_debug_views(F, d, &lg, &mx, &sm, &st) == SV_OK);
        EXPECT(lg == F && (const char*)st + 4 * (size_t)d.B <= (const char*)F + w);
    }

    // the tiled W form: sizes at the extremes, argument errors
    EXPECT(sv_tiled_w_bytes(1 << 28, 65536) == ((size_t)1 << 24) * 2048 * 1024);
    EXPECT(sv_tiled_w_bytes(1, 8) == 1024 && sv_tiled_w_bytes(17, 40) == 4096);
    EXPECT(sv_tiled_w_bytes(0, 64) == 0 && sv_tiled_w_bytes(10, 12) == 0 &&
           sv_tiled_w_bytes(INT32_MAX, INT32_MAX) == 0 && sv_tiled_w_bytes(INT32_MIN, 64) == 0);
    EXPECT(sv_tile_w(f<uint16_t>(), (1 << 28) + 1, 64, f<uint16_t>(), big, nullptr) == SV_ERR_DIMS);
    EXPECT(sv_tile_w(nullptr, 100, 64, f<uint16_t>(), big, nullptr) == SV_ERR_NULL);
    EXPECT(sv_tile_w(f<uint16_t>(), 100, 64, nullptr, big, nullptr) == SV_ERR_NULL);
    EXPECT(sv_tile_w(f<uint16_t>() + 4, 100, 64, f<uint16_t>(), big, nullptr) == SV_ERR_ALIGN);
    EXPECT(sv_tile_w(f<uint16_t>(), 100, 64, f<uint16_t>(), sv_tiled_w_bytes(100, 64) - 1,
                     nullptr) == SV_ERR_WORKSPACE);

    // every pointer argument NULL in turn, misalignment, short workspace
    const sv_dims ok = D(3, 4, 64, 1000);
    const size_t ws = sv_workspace_bytes(ok);
    for (int i = 0; i < 7; ++i) {
        void* a[7];
        for (void*& x : a) x = F;
        a[i] = nullptr;
        EXPECT(spec_verify((uint16_t*)a[0], (uint16_t*)a[1], (int32_t*)a[2], (float*)a[3],
                           (float*)a[4], ok, (int32_t*)a[5], (int32_t*)a[6], F, ws, nullptr) ==
               SV_ERR_NULL);
        EXPECT(spec_verify_static((uint16_t*)a[0], (uint16_t*)a[1], (int32_t*)a[2], (float*)a[3],
                                  (float*)a[4], ok, (int32_t*)a[5], (int32_t*)a[6], nullptr) ==
               SV_ERR_NULL);
    }
    EXPECT(spec_verify(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(), f<float>(), ok,
                       f<int32_t>(), f<int32_t>(), nullptr, ws, nullptr) == SV_ERR_NULL);
    EXPECT(spec_verify(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(), f<float>(), ok,
                       f<int32_t>(), f<int32_t>(), F, ws - 1, nullptr) == SV_ERR_WORKSPACE);
    EXPECT(spec_verify(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(), f<float>(), ok,
                       f<int32_t>(), f<int32_t>(), (char*)F + 128, ws, nullptr) == SV_ERR_ALIGN);
    EXPECT(spec_verify((uint16_t*)((char*)F + 8), f<uint16_t>(), f<int32_t>(), f<float>(),
                       f<float>(), ok, f<int32_t>(), f<int32_t>(), F, ws, nullptr) ==
           SV_ERR_ALIGN);
    EXPECT(spec_verify_static(f<uint16_t>(), f<uint16_t>(), f<int32_t>(), f<float>(), f<float>(),
                              D(20, 4, 64, 128256), f<int32_t>(), f<int32_t>(), nullptr) ==
           SV_ERR_WORKSPACE);
    EXPECT(sv_accept_greedy(f<int32_t>(), ok, f<int32_t>(), f<int32_t>(), nullptr, F, ws - 1,
                            nullptr) == SV_ERR_WORKSPACE);
    EXPECT(sv_accept_and_draw_sparse_q(f<int32_t>(), f<int32_t>(), f<float>(), 0, f<float>(), ok,
                                       f<int32_t>(), f<int32_t>(), F, ws, nullptr) ==
           SV_ERR_DIMS);
    EXPECT(sv_accept_and_draw_sparse_q(f<int32_t>(), f<int32_t>(), f<float>(), (1 << 24) + 1,
                                       f<float>(), ok, f<int32_t>(), f<int32_t>(), F, ws,
                                       nullptr) == SV_ERR_DIMS);
    EXPECT(sv_debug_views(nullptr, ok, nullptr, nullptr, nullptr, nullptr) == SV_ERR_NULL);
    for (int32_t flags : {4, 8, -1, INT32_MIN})
        EXPECT(sv_lmhead_ex(f<uint16_t>(), f<uint16_t>(), ok, flags, F, ws, nullptr) == SV_ERR_DIMS);
    EXPECT(sv_lmhead_ex(f<uint16_t>(), f<uint16_t>(), ok, SV_LMHEAD_LOGITS, F, ws - 1, nullptr) ==
           SV_ERR_WORKSPACE);

    // the clustered head's dims
    const sv_head_dims hbad[] = {{0, 64, 100, 4, 25, 2}, {4, 12, 100, 4, 25, 2},
                                 {4, 64, 100, 0, 25, 2}, {4, 64, 100, SV_HEAD_MAX_CLUSTERS + 1, 1, 1},
                                 {4, 64, 100, 4, 25, 5}, {4, 64, 100, 4, 0, 2},
                                 {4, 64, 100, 8192, 1 << 20, 8192}};
    for (const sv_head_dims& h : hbad) {
        EXPECT(sv_sparse_head_workspace_bytes(h) == 0);
        EXPECT(sv_sparse_head(f<uint16_t>(), f<uint16_t>(), f<uint16_t>(), f<int32_t>(), h,
                              f<int32_t>(), f<float>(), nullptr, F, big, nullptr) == SV_ERR_DIMS);
    }
    const sv_head_dims hok = {32, 1536, 262144, 2048, 128, 32};
    EXPECT(sv_sparse_head_workspace_bytes(hok) > 0);
    EXPECT(sv_sparse_head(f<uint16_t>(), f<uint16_t>(), f<uint16_t>(), f<int32_t>(), hok,
                          f<int32_t>(), f<float>(), nullptr, F, 0, nullptr) == SV_ERR_WORKSPACE);

    // tree topologies: random valid and invalid parent arrays against a
    // reference parser; then the tree entry point's own checks
    std::mt19937 rng(12345);
    for (int it = 0; it < 20000; ++it) {
        const int T = 1 + (int)(rng() % (SV_MAX_TREE_NODES + 8));
        std::vector<int32_t> p(T);
        for (int t = 0; t < T; ++t) p[t] = (int)(rng() % (t + 1)) - 1;     // valid: -1 .. t-1
        if (rng() % 4 == 0) p[rng() % T] = (int)(rng() % 200) - 100;       // maybe invalid
        int dr = 0, qr = 0, depth = -1, q_rows = -1, rounds = -1;
        const bool want = ref_tree(p, &dr, &qr);
        const sv_status got = sv_tree_shape(p.data(), T, &depth, &q_rows, &rounds);
        EXPECT((got == SV_OK) == want);
        if (want && got == SV_OK) {
            EXPECT(depth == dr && q_rows == qr && rounds >= 1 && rounds <= T);
            const sv_dims td = D(2, T, 64, 1000);
            const size_t tws = sv_tree_workspace_bytes(td);
            EXPECT(tws > 0);
            EXPECT(spec_verify_tree(f<uint16_t>(), f<uint16_t>(), p.data(), f<int32_t>(),
                                    f<float>(), f<float>(), td, f<int32_t>(), f<int32_t>(),
                                    nullptr, F, tws - 1, nullptr) == SV_ERR_WORKSPACE);
        }
    }
    EXPECT(sv_tree_shape(nullptr, 4, nullptr, nullptr, nullptr) == SV_ERR_DIMS);
    std::vector<int32_t> chain(SV_MAX_TREE_NODES);
    for (int t = 0; t < SV_MAX_TREE_NODES; ++t) chain[t] = t - 1;
    EXPECT(sv_tree_shape(chain.data(), 0, nullptr, nullptr, nullptr) == SV_ERR_DIMS);
    EXPECT(spec_verify_tree(f<uint16_t>(), f<uint16_t>(), nullptr, f<int32_t>(), f<float>(),
                            f<float>(), D(2, 4, 64, 1000), f<int32_t>(), f<int32_t>(), nullptr, F,
                            big, nullptr) == SV_ERR_NULL);

    std::printf("sanitized ABI checks: %d run, %d failed\n", g_checks, g_failed);
    return g_failed == 0 ? 0 : 1;
}
