// The C ABI of libcce (declared in include/cce.h): argument checks, which run
// before anything is enqueued, workspace sizing, and the calls into the
// launchers.  No allocation, no host synchronisation, no global state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "cce.h"
#include "cce_internal.hpp"

using namespace cce;

namespace {

constexpr int kVersion = 10200;  // 1.2.0

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Row and vocabulary positions are 32-bit in the kernels, and a tile's last
// position (its start + up to 255) must stay below 2^31: N, V <= kMaxRows.
constexpr int64_t kMaxRows = (int64_t(1) << 31) - (int64_t(1) << 16);

bool shape_ok(int64_t N, int64_t D, int64_t V) {
    if (N < 1 || N > kMaxRows) return false;
    if (V < 1 || V > kMaxRows) return false;
    if (D < 8 || D > 65536 || D % 8 != 0) return false;
    // grid sizes stay below 2^31 workgroups, and logit tiles are indexed with 32 bits
    if (ceil_div(N, kBlockRows) * ceil_div(D, 128) >= (int64_t(1) << 31)) return false;
    if (ceil_div(N, kTileRows) * ceil_div(V, kTileVocab) >= (int64_t(1) << 31)) return false;
    return true;
}

// An enum argument as the int its caller passed.  A C caller may pass any int
// (the value is then rejected); in C++ reading such a value as the enum type
// is undefined, so its bytes are read as an int before anything else.
template <typename Enum>
int enum_int(const Enum &e) {
    static_assert(sizeof(Enum) == sizeof(int), "enums of the C ABI are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

bool dtype_ok(int dt) { return dt == CCE_F32 || dt == CCE_BF16; }
size_t elem_size(int dt) { return dt == CCE_BF16 ? 2 : 4; }

cce_status hip_status(hipError_t e) { return e == hipSuccess ? CCE_OK : CCE_ERR_HIP; }

// Every workspace also holds the labels mapped into the processing space of
// a composite head (N int64), after the part the kernels carve.
size_t label_bytes(int64_t N) { return align256((size_t)N * sizeof(int64_t)); }

// Composite head: two non-empty blocks, the second at or after the end of
// the first; ids stay far from int64 overflow.
bool blocks_ok(int64_t V0, int64_t V1, int64_t off1) {
    return V0 >= 1 && V1 >= 1 && off1 >= V0 && off1 < (int64_t(1) << 62) && V1 < (int64_t(1) << 31);
}

// Labels as the kernels read them: the caller's, or (composite head) mapped
// into [0, V0 + V1) in the workspace's label region.
hipError_t map_labels(const int64_t *labels, int64_t N, int64_t ignore_index, const VocabRows &E, int64_t off1,
                      int64_t V, void *label_ws, const int64_t **out, hipStream_t st) {
    *out = labels;
    if (E.v0 >= V) return hipSuccess;
    int64_t *mapped = static_cast<int64_t *>(label_ws);
    *out = mapped;
    return launch_seg_labels(labels, N, ignore_index, E.v0, off1, V - E.v0, mapped, st);
}

// The forward's argument checks other than the workspace's.
cce_status forward_check(const void *H, const VocabRows &E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                         int dtype, const int32_t *perm, float *loss, float *lse, float *block_max) {
    if (!H || !E.e0 || !E.e1 || !labels || !loss || !lse) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!aligned(H, 16) || !aligned(E.e0, 16) || !aligned(E.e1, 16) || !aligned(labels, 8) || !aligned(loss, 4) ||
        !aligned(lse, 4) || !aligned(block_max, 4) || !aligned(perm, 4))
        return CCE_ERR_ALIGN;
    return CCE_OK;
}

cce_status forward_impl(const void *H, const VocabRows &E, int64_t off1, const int64_t *labels, int64_t N, int64_t D,
                        int64_t V, int dtype, int64_t ignore_index, const int32_t *perm, float *loss,
                        float *lse, float *block_max, void *ws, size_t ws_bytes, void *stream) {
    const cce_status c = forward_check(H, E, labels, N, D, V, dtype, perm, loss, lse, block_max);
    if (c != CCE_OK) return c;
    if (!ws) return CCE_ERR_NULL;
    if (!aligned(ws, 16)) return CCE_ERR_ALIGN;
    const FwdShape s = fwd_shape(N, D, V);
    size_t need = 0;
    const FwdWs w = fwd_ws(ws, s, &need);
    if (ws_bytes < align256(need) + label_bytes(N)) return CCE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t *y = nullptr;
    hipError_t e = map_labels(labels, N, ignore_index, E, off1, V, static_cast<char *>(ws) + align256(need), &y, st);
    if (e != hipSuccess) return CCE_ERR_HIP;
    return hip_status(launch_forward(static_cast<cce_dtype>(dtype), H, E, y, s, ignore_index, perm, w, loss, lse,
                                     block_max, st));
}

cce_status vocab_order_impl(const void *H, const VocabRows &E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                            int dtype, int64_t ignore_index, int32_t *perm, float *keys, void *ws,
                            size_t ws_bytes, void *stream) {
    if (!H || !E.e0 || !E.e1 || !labels || !perm || !ws) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!aligned(H, 16) || !aligned(E.e0, 16) || !aligned(E.e1, 16) || !aligned(ws, 16) || !aligned(labels, 8) ||
        !aligned(perm, 4) || !aligned(keys, 4))
        return CCE_ERR_ALIGN;
    size_t need = 0;
    const SortWs w = sort_ws(ws, N, D, V, &need);
    if (ws_bytes < align256(need) + label_bytes(N)) return CCE_ERR_WORKSPACE;
    // (only ignore_index matters to the sort: no label mapping needed)
    return hip_status(launch_vocab_order(static_cast<cce_dtype>(dtype), H, E, labels, N, D, V, ignore_index, perm,
                                         keys, w, static_cast<hipStream_t>(stream)));
}

cce_status backward_impl(const void *H, const VocabRows &E, int64_t off1, const int64_t *labels, const float *lse,
                         const float *dloss, const float *block_max, int64_t N, int64_t D, int64_t V, int dtype,
                         int64_t ignore_index, float filter_eps, const int32_t *perm, unsigned flags, void *dH,
                         const VocabGrads &dE, int64_t *stats, void *ws, size_t ws_bytes, void *stream) {
    if (!H || !E.e0 || !E.e1 || !labels || !lse || !dloss || !dH || !dE.d0 || !dE.d1 || !ws) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!(filter_eps >= 0.f) || isinf(filter_eps)) return CCE_ERR_ARG;  // rejects NaN and negatives
    if (flags & ~(CCE_BWD_NO_KAHAN | CCE_BWD_FULL_DE | CCE_BWD_FINE_FILTER | CCE_BWD_DEBUG_STORE_LIMIT))
        return CCE_ERR_ARG;
    if ((flags & CCE_BWD_FINE_FILTER) && (flags & CCE_BWD_FULL_DE)) return CCE_ERR_ARG;
    if (!aligned(H, 16) || !aligned(E.e0, 16) || !aligned(E.e1, 16) || !aligned(dH, 16) || !aligned(dE.d0, 16) ||
        !aligned(dE.d1, 16) || !aligned(ws, 16) || !aligned(labels, 8) || !aligned(lse, 4) || !aligned(dloss, 4) ||
        !aligned(perm, 4) || !aligned(stats, 8) || !aligned(block_max, 4))
        return CCE_ERR_ALIGN;
    const BwdShape s = bwd_shape(N, D, V);
    size_t need = 0;
    const BwdWs w = bwd_ws(ws, s, elem_size(dtype), &need);
    if (ws_bytes < align256(need) + label_bytes(N)) return CCE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t *y = nullptr;
    hipError_t e = map_labels(labels, N, ignore_index, E, off1, V, static_cast<char *>(ws) + align256(need), &y, st);
    if (e != hipSuccess) return CCE_ERR_HIP;
    return hip_status(launch_backward(static_cast<cce_dtype>(dtype), H, E, y, lse, dloss, block_max, s, ignore_index,
                                      filter_eps, perm, flags, dH, dE, stats, w, st));
}

}  // namespace

extern "C" {

const char *cce_status_string(cce_status status) {
    switch (enum_int(status)) {
        case CCE_OK: return "ok";
        case CCE_ERR_NULL: return "a required pointer is NULL";
        case CCE_ERR_SHAPE:
            return "N, D or V outside the supported range (D % 8 == 0, 8 <= D <= 65536, 1 <= N, V <= 2^31 - 2^16)";
        case CCE_ERR_DTYPE: return "unknown dtype";
        case CCE_ERR_ALIGN: return "a pointer is not aligned (16 bytes for H, E, dH, dE, workspace)";
        case CCE_ERR_WORKSPACE: return "workspace too small";
        case CCE_ERR_HIP: return "a HIP launch failed";
        case CCE_ERR_ARG: return "invalid argument";
    }
    return "unknown status";
}

int cce_version(void) { return kVersion; }

void cce_filter_block(int *block_rows, int *block_vocab) {
    if (block_rows) *block_rows = kBlockRows;
    if (block_vocab) *block_vocab = kBlockVocab;
}

size_t cce_forward_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype) {
    if (!shape_ok(N, D, V) || !dtype_ok(enum_int(dtype))) return 0;
    size_t b = 0;
    fwd_ws(nullptr, fwd_shape(N, D, V), &b);
    return align256(b) + label_bytes(N);
}

size_t cce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype) {
    if (!shape_ok(N, D, V) || !dtype_ok(enum_int(dtype))) return 0;
    size_t b = 0;
    bwd_ws(nullptr, bwd_shape(N, D, V), elem_size(enum_int(dtype)), &b);
    return align256(b) + label_bytes(N);
}

size_t cce_block_max_elems(int64_t N, int64_t V) {
    if (!shape_ok(N, 8, V)) return 0;
    return (size_t)block_max_elems(N, V);
}

size_t cce_vocab_order_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype) {
    if (!shape_ok(N, D, V) || !dtype_ok(enum_int(dtype))) return 0;
    size_t b = 0;
    sort_ws(nullptr, N, D, V, &b);
    return align256(b) + label_bytes(N);
}

cce_status cce_forward(const void *H, const void *E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                       cce_dtype dtype, int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                       float *block_max, void *ws, size_t ws_bytes, void *stream) {
    return forward_impl(H, VocabRows{E, E, kOneBlock}, 0, labels, N, D, V, enum_int(dtype), ignore_index, perm, loss,
                        lse, block_max, ws, ws_bytes, stream);
}

static_assert(kNoAllocScratchBytes == CCE_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

cce_status cce_forward_noalloc(const void *H, const void *E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                               cce_dtype dtype, int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                               float *block_max, void *stream) {
    const VocabRows rows{E, E, kOneBlock};
    const int dt = enum_int(dtype);
    const cce_status c = forward_check(H, rows, labels, N, D, V, dt, perm, loss, lse, block_max);
    if (c != CCE_OK) return c;
    if (cce_forward_workspace_bytes(N, D, V, static_cast<cce_dtype>(dt)) > kNoAllocScratchBytes)
        return CCE_ERR_WORKSPACE;
    void *ws = nullptr;
    if (noalloc_scratch(&ws) != hipSuccess) return CCE_ERR_HIP;
    return forward_impl(H, rows, 0, labels, N, D, V, dt, ignore_index, perm, loss, lse, block_max, ws,
                        kNoAllocScratchBytes, stream);
}

cce_status cce_forward_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1, int64_t off1,
                                 const int64_t *labels, int64_t N, int64_t D, cce_dtype dtype, int64_t ignore_index,
                                 const int32_t *perm, float *loss, float *lse, float *block_max, void *ws,
                                 size_t ws_bytes, void *stream) {
    if (!blocks_ok(V0, V1, off1)) return CCE_ERR_SHAPE;
    return forward_impl(H, VocabRows{E0, E1, V0}, off1, labels, N, D, V0 + V1, enum_int(dtype), ignore_index, perm,
                        loss, lse, block_max, ws, ws_bytes, stream);
}

cce_status cce_vocab_order(const void *H, const void *E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                           cce_dtype dtype, int64_t ignore_index, int32_t *perm, float *keys, void *ws,
                           size_t ws_bytes, void *stream) {
    return vocab_order_impl(H, VocabRows{E, E, kOneBlock}, labels, N, D, V, enum_int(dtype), ignore_index, perm,
                            keys, ws, ws_bytes, stream);
}

cce_status cce_vocab_order_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1,
                                     const int64_t *labels, int64_t N, int64_t D, cce_dtype dtype,
                                     int64_t ignore_index, int32_t *perm, float *keys, void *ws, size_t ws_bytes,
                                     void *stream) {
    if (!blocks_ok(V0, V1, V0)) return CCE_ERR_SHAPE;
    return vocab_order_impl(H, VocabRows{E0, E1, V0}, labels, N, D, V0 + V1, enum_int(dtype), ignore_index, perm,
                            keys, ws, ws_bytes, stream);
}

cce_status cce_backward(const void *H, const void *E, const int64_t *labels, const float *lse, const float *dloss,
                        const float *block_max, int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                        int64_t ignore_index, float filter_eps, const int32_t *perm, unsigned flags, void *dH,
                        void *dE, int64_t *stats, void *ws, size_t ws_bytes, void *stream) {
    return backward_impl(H, VocabRows{E, E, kOneBlock}, 0, labels, lse, dloss, block_max, N, D, V, enum_int(dtype),
                         ignore_index, filter_eps, perm, flags, dH, VocabGrads{dE, dE, kOneBlock}, stats, ws,
                         ws_bytes, stream);
}

cce_status cce_backward_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1,
                                  int64_t off1, const int64_t *labels, const float *lse, const float *dloss,
                                  const float *block_max, int64_t N, int64_t D, cce_dtype dtype,
                                  int64_t ignore_index, float filter_eps, const int32_t *perm, unsigned flags,
                                  void *dH, void *dE0, void *dE1, int64_t *stats, void *ws, size_t ws_bytes,
                                  void *stream) {
    if (!blocks_ok(V0, V1, off1)) return CCE_ERR_SHAPE;
    return backward_impl(H, VocabRows{E0, E1, V0}, off1, labels, lse, dloss, block_max, N, D, V0 + V1,
                         enum_int(dtype), ignore_index, filter_eps, perm, flags, dH, VocabGrads{dE0, dE1, V0}, stats,
                         ws, ws_bytes, stream);
}

cce_status cce_check_labels(const int64_t *labels, int64_t N, int64_t V, int64_t ignore_index, int64_t *n_bad,
                            void *stream) {
    if (!labels || !n_bad) return CCE_ERR_NULL;
    if (N < 1 || N > kMaxRows || V < 1 || V > kMaxRows) return CCE_ERR_SHAPE;
    if (!aligned(labels, 8) || !aligned(n_bad, 8)) return CCE_ERR_ALIGN;
    return hip_status(launch_check_labels(labels, N, V, ignore_index, n_bad, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
