// Host-side argument checks of the C ABI, as a standalone program so that the
// library's host code can run under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by `linear_cross_entropy_cce_amd.build
// --host-check`, run by tests/test_abi_sanitized.py).  The same cases as the
// Python tests of the ABI: every call here must be rejected (or sized) on the
// host before anything is enqueued; the pointers are fake, aligned addresses
// that are never dereferenced.  Out-of-range dtype and status values are the
// ints a C caller may pass.  Exit status 0 when every check holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cce.h"

static int failures = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "abi_check: line %d: %s\n", __LINE__, #cond);    \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

namespace {

char *const FAKE = reinterpret_cast<char *>(0x100000);
const int64_t kVmax = (int64_t(1) << 31) - (int64_t(1) << 16);
const size_t kBig = size_t(1) << 40;

struct Fwd {
    const void *H = FAKE, *E = FAKE;
    const int64_t *labels = reinterpret_cast<const int64_t *>(FAKE);
    int64_t N = 16, D = 64, V = 100;
    int dt = CCE_BF16;
    const int32_t *perm = nullptr;
    float *loss = reinterpret_cast<float *>(FAKE), *lse = reinterpret_cast<float *>(FAKE), *tb = nullptr;
    void *ws = FAKE;
    size_t ws_bytes = kBig;
    cce_status run() const {
        return cce_forward(H, E, labels, N, D, V, (cce_dtype)dt, -100, perm, loss, lse, tb, ws, ws_bytes, nullptr);
    }
};

struct Bwd {
    const void *H = FAKE, *E = FAKE;
    const int64_t *labels = reinterpret_cast<const int64_t *>(FAKE);
    const float *lse = reinterpret_cast<const float *>(FAKE), *dloss = reinterpret_cast<const float *>(FAKE);
    const float *tb = nullptr;
    int64_t N = 16, D = 64, V = 100;
    int dt = CCE_BF16;
    float eps = 0.f;
    const int32_t *perm = nullptr;
    unsigned flags = 0;
    void *dH = FAKE, *dE = FAKE;
    int64_t *stats = nullptr;
    void *ws = FAKE;
    size_t ws_bytes = kBig;
    cce_status run() const {
        return cce_backward(H, E, labels, lse, dloss, tb, N, D, V, (cce_dtype)dt, -100, eps, perm, flags, dH, dE,
                            stats, ws, ws_bytes, nullptr);
    }
};

struct Vord {
    const void *H = FAKE, *E = FAKE;
    const int64_t *labels = reinterpret_cast<const int64_t *>(FAKE);
    int64_t N = 16, D = 64, V = 100;
    int dt = CCE_BF16;
    int32_t *perm = reinterpret_cast<int32_t *>(FAKE);
    void *ws = FAKE;
    size_t ws_bytes = kBig;
    cce_status run() const {
        return cce_vocab_order(H, E, labels, N, D, V, (cce_dtype)dt, -100, perm, nullptr, ws, ws_bytes, nullptr);
    }
};

// The checks every entry point shares (null, shape, dtype, alignment, workspace).
template <class C>
void common_errors() {
    C c;
    { C x = c; x.H = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { C x = c; x.E = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { C x = c; x.labels = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { C x = c; x.ws = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { C x = c; x.N = 0; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.V = 0; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.D = 12; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.D = 0; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.V = int64_t(1) << 31; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.V = kVmax + 1; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.N = kVmax + 1; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.N = -1; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.D = INT64_MAX; CHECK(x.run() == CCE_ERR_SHAPE); }
    { C x = c; x.dt = 5; CHECK(x.run() == CCE_ERR_DTYPE); }
    { C x = c; x.dt = -1; CHECK(x.run() == CCE_ERR_DTYPE); }
    { C x = c; x.H = FAKE + 8; CHECK(x.run() == CCE_ERR_ALIGN); }
    { C x = c; x.E = FAKE + 4; CHECK(x.run() == CCE_ERR_ALIGN); }
    { C x = c; x.ws = FAKE + 2; CHECK(x.run() == CCE_ERR_ALIGN); }
    { C x = c; x.ws_bytes = 16; CHECK(x.run() == CCE_ERR_WORKSPACE); }
    { C x = c; x.ws_bytes = 0; CHECK(x.run() == CCE_ERR_WORKSPACE); }
}

void sizes() {
    for (int dt = 0; dt < 2; ++dt) {
        const cce_dtype t = (cce_dtype)dt;
        const int64_t cases[][3] = {{0, 64, 10},    {10, 0, 10},         {10, 12, 10},   {10, 64, 0},
                                    {10, 64, 1},    {10, 64, int64_t(1) << 31}, {10, 64, 10}, {10, 64, kVmax},
                                    {10, 64, kVmax + 1}, {kVmax, 64, 10}, {kVmax + 1, 64, 10}, {-5, 64, 10},
                                    {10, -64, 10},  {10, 64, -10},       {10, INT64_MAX - 7, 10}, {10, 65536, 10},
                                    {10, 65544, 10}};
        for (const auto &c : cases) {
            const int64_t n = c[0], d = c[1], v = c[2];
            const bool ok = n >= 1 && n <= kVmax && v >= 1 && v <= kVmax && d >= 8 && d % 8 == 0 && d <= 65536;
            const size_t f = cce_forward_workspace_bytes(n, d, v, t);
            const size_t b = cce_backward_workspace_bytes(n, d, v, t);
            const size_t s = cce_vocab_order_workspace_bytes(n, d, v, t);
            CHECK((f == 0) == !ok);
            CHECK((b == 0) == !ok);
            CHECK((s == 0) == !ok);
        }
        // no N x V term: doubling both at most roughly doubles the workspace
        const size_t a = cce_backward_workspace_bytes(8192, 2048, 256000, t);
        const size_t a2 = cce_backward_workspace_bytes(16384, 2048, 512000, t);
        CHECK(a > 0 && a2 < 2.2 * a);
        const size_t f1 = cce_forward_workspace_bytes(8192, 2048, 256000, t);
        CHECK(cce_forward_workspace_bytes(16384, 2048, 512000, t) < 2.2 * f1);
    }
    CHECK(cce_forward_workspace_bytes(10, 64, 10, (cce_dtype)7) == 0);
    CHECK(cce_block_max_elems(1, 1) == 4 + 1);
    CHECK(cce_block_max_elems(257, 256) == 8 + 257);
    CHECK(cce_block_max_elems(8192, 256000) == size_t(64) * 2000 + 8192);
    CHECK(cce_block_max_elems(0, 10) == 0);
    CHECK(cce_block_max_elems(10, 0) == 0);
    CHECK(cce_block_max_elems(-1, 10) == 0);
    CHECK(cce_block_max_elems(kVmax + 1, 10) == 0);
}

void forward_errors() {
    Fwd c;
    { Fwd x = c; x.loss = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Fwd x = c; x.lse = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Fwd x = c; x.lse = reinterpret_cast<float *>(FAKE + 2); CHECK(x.run() == CCE_ERR_ALIGN); }
    { Fwd x = c; x.tb = reinterpret_cast<float *>(FAKE + 2); CHECK(x.run() == CCE_ERR_ALIGN); }
    { Fwd x = c; x.perm = reinterpret_cast<const int32_t *>(FAKE + 2); CHECK(x.run() == CCE_ERR_ALIGN); }
    const size_t need = cce_forward_workspace_bytes(16, 64, 100, CCE_BF16);
    { Fwd x = c; x.ws_bytes = need - 1; CHECK(x.run() == CCE_ERR_WORKSPACE); }
}

void backward_errors() {
    Bwd c;
    { Bwd x = c; x.dH = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Bwd x = c; x.dE = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Bwd x = c; x.lse = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Bwd x = c; x.dloss = nullptr; CHECK(x.run() == CCE_ERR_NULL); }
    { Bwd x = c; x.eps = -1.f; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.eps = NAN; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.eps = INFINITY; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.flags = 16; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.flags = 0x80000000u; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.flags = CCE_BWD_FINE_FILTER | CCE_BWD_FULL_DE; CHECK(x.run() == CCE_ERR_ARG); }
    { Bwd x = c; x.dE = FAKE + 8; CHECK(x.run() == CCE_ERR_ALIGN); }
    { Bwd x = c; x.perm = reinterpret_cast<const int32_t *>(FAKE + 2); CHECK(x.run() == CCE_ERR_ALIGN); }
    { Bwd x = c; x.stats = reinterpret_cast<int64_t *>(FAKE + 4); CHECK(x.run() == CCE_ERR_ALIGN); }
    { Bwd x = c; x.tb = reinterpret_cast<const float *>(FAKE + 2); CHECK(x.run() == CCE_ERR_ALIGN); }
    const size_t need = cce_backward_workspace_bytes(16, 64, 100, CCE_BF16);
    { Bwd x = c; x.ws_bytes = need - 1; CHECK(x.run() == CCE_ERR_WORKSPACE); }
}

void composite_errors() {
    const int64_t *y = reinterpret_cast<const int64_t *>(FAKE);
    float *f = reinterpret_cast<float *>(FAKE);
    auto fwd = [&](const void *E1, int64_t V0, int64_t V1, int64_t off1, int dt, size_t ws_bytes) {
        return cce_forward_composite(FAKE, FAKE, V0, E1, V1, off1, y, 16, 64, (cce_dtype)dt, -100, nullptr, f, f,
                                     nullptr, FAKE, ws_bytes, nullptr);
    };
    auto bwd = [&](const void *E1, int64_t V0, int64_t V1, int64_t off1, int dt, size_t ws_bytes, void *dE1,
                   float eps) {
        return cce_backward_composite(FAKE, FAKE, V0, E1, V1, off1, y, f, f, nullptr, 16, 64, (cce_dtype)dt, -100,
                                      eps, nullptr, 0, FAKE, FAKE, dE1, nullptr, FAKE, ws_bytes, nullptr);
    };
    char *E1 = FAKE + 4096, *dE1 = FAKE + 8192;
    const int64_t big = int64_t(1) << 30;
    CHECK(fwd(nullptr, 60, 40, 70, CCE_BF16, kBig) == CCE_ERR_NULL);
    CHECK(fwd(E1, 0, 40, 70, CCE_BF16, kBig) == CCE_ERR_SHAPE);
    CHECK(fwd(E1, 60, 0, 70, CCE_BF16, kBig) == CCE_ERR_SHAPE);
    CHECK(fwd(E1, 60, 40, 59, CCE_BF16, kBig) == CCE_ERR_SHAPE);
    CHECK(fwd(E1, big, big, big, CCE_BF16, kBig) == CCE_ERR_SHAPE);
    CHECK(fwd(E1, 60, 40, INT64_MAX, CCE_BF16, kBig) == CCE_ERR_SHAPE);
    CHECK(fwd(E1 + 8, 60, 40, 70, CCE_BF16, kBig) == CCE_ERR_ALIGN);
    CHECK(fwd(E1, 60, 40, 70, 5, kBig) == CCE_ERR_DTYPE);
    CHECK(fwd(E1, 60, 40, 70, CCE_BF16, cce_forward_workspace_bytes(16, 64, 100, CCE_BF16) - 1) ==
          CCE_ERR_WORKSPACE);
    CHECK(bwd(nullptr, 60, 40, 70, CCE_BF16, kBig, dE1, 0.f) == CCE_ERR_NULL);
    CHECK(bwd(E1, 60, 40, 59, CCE_BF16, kBig, dE1, 0.f) == CCE_ERR_SHAPE);
    CHECK(bwd(E1, big, big, big, CCE_BF16, kBig, dE1, 0.f) == CCE_ERR_SHAPE);
    CHECK(bwd(E1, 60, 40, 70, CCE_BF16, kBig, nullptr, 0.f) == CCE_ERR_NULL);
    CHECK(bwd(E1, 60, 40, 70, CCE_BF16, kBig, dE1 + 8, 0.f) == CCE_ERR_ALIGN);
    CHECK(bwd(E1, 60, 40, 70, CCE_BF16, kBig, dE1, -1.f) == CCE_ERR_ARG);
    CHECK(bwd(E1, 60, 40, 70, CCE_BF16, cce_backward_workspace_bytes(16, 64, 100, CCE_BF16) - 1, dE1, 0.f) ==
          CCE_ERR_WORKSPACE);
    int32_t *perm = reinterpret_cast<int32_t *>(FAKE);
    CHECK(cce_vocab_order_composite(FAKE, FAKE, 60, nullptr, 40, y, 16, 64, CCE_BF16, -100, perm, nullptr, FAKE, kBig,
                                    nullptr) == CCE_ERR_NULL);
    CHECK(cce_vocab_order_composite(FAKE, FAKE, 0, E1, 40, y, 16, 64, CCE_BF16, -100, perm, nullptr, FAKE, kBig,
                                    nullptr) == CCE_ERR_SHAPE);
}

void other_entry_points() {
    int64_t *nb = reinterpret_cast<int64_t *>(FAKE);
    const int64_t *y = reinterpret_cast<const int64_t *>(FAKE);
    CHECK(cce_check_labels(nullptr, 10, 10, -100, nb, nullptr) == CCE_ERR_NULL);
    CHECK(cce_check_labels(y, 10, 10, -100, nullptr, nullptr) == CCE_ERR_NULL);
    CHECK(cce_check_labels(y, 0, 10, -100, nb, nullptr) == CCE_ERR_SHAPE);
    CHECK(cce_check_labels(reinterpret_cast<const int64_t *>(FAKE + 4), 10, 10, -100, nb, nullptr) == CCE_ERR_ALIGN);
    float *f = reinterpret_cast<float *>(FAKE);
    auto na = [&](const void *H, const void *E, int64_t N, int64_t D, int64_t V, int dt, float *loss) {
        return cce_forward_noalloc(H, E, y, N, D, V, (cce_dtype)dt, -100, nullptr, loss, f, nullptr, nullptr);
    };
    CHECK(na(nullptr, FAKE, 16, 64, 100, CCE_BF16, f) == CCE_ERR_NULL);
    CHECK(na(FAKE, FAKE, 16, 64, 100, CCE_BF16, nullptr) == CCE_ERR_NULL);
    CHECK(na(FAKE, FAKE, 16, 64, 100, 9, f) == CCE_ERR_DTYPE);
    CHECK(na(FAKE, FAKE, 16, 12, 100, CCE_BF16, f) == CCE_ERR_SHAPE);
    CHECK(na(FAKE, FAKE + 8, 16, 64, 100, CCE_BF16, f) == CCE_ERR_ALIGN);
    CHECK(na(FAKE, FAKE, int64_t(1) << 20, 64, 100, CCE_BF16, f) == CCE_ERR_WORKSPACE);
    CHECK(na(FAKE, FAKE, 16, 64, int64_t(1) << 22, CCE_BF16, f) == CCE_ERR_WORKSPACE);
    for (int s = 0; s < 8; ++s) CHECK(strlen(cce_status_string((cce_status)s)) > 0);
    CHECK(strcmp(cce_status_string((cce_status)99), "unknown status") == 0);
    CHECK(strcmp(cce_status_string((cce_status)-3), "unknown status") == 0);
    CHECK(cce_version() >= 10000);
    int r = 0, v = 0;
    cce_filter_block(&r, &v);
    CHECK(r > 0 && v > 0 && r % 32 == 0 && v % 32 == 0);
    cce_filter_block(nullptr, nullptr);
}

}  // namespace

int main() {
    sizes();
    common_errors<Fwd>();
    common_errors<Bwd>();
    common_errors<Vord>();
    forward_errors();
    backward_errors();
    composite_errors();
    other_entry_points();
    if (failures) {
        fprintf(stderr, "abi_check: %d failed\n", failures);
        return 1;
    }
    printf("abi_check: all host-side checks hold\n");
    return 0;
}
