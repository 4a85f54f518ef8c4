// The C ABI of libcce (declared in include/cce.h): argument checks, which run
// before anything is enqueued, workspace sizing, and the calls into the
// launchers.  No allocation, no host synchronisation, no global state.
#include <math.h>
#include <stdint.h>

#include "cce.h"
#include "cce_internal.hpp"

using namespace cce;

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool shape_ok(int64_t N, int64_t D, int64_t V) {
    if (N < 1 || N >= (int64_t(1) << 31)) return false;
    if (V < 1 || V >= (int64_t(1) << 31)) return false;
    if (D < 8 || D > 65536 || D % 8 != 0) return false;
    // grid sizes stay below 2^31 workgroups, and logit tiles are indexed with 32 bits
    if (ceil_div(N, kBlockRows) * ceil_div(D, 128) >= (int64_t(1) << 31)) return false;
    if (ceil_div(N, kTileRows) * ceil_div(V, kTileVocab) >= (int64_t(1) << 31)) return false;
    return true;
}

bool dtype_ok(cce_dtype dt) { return dt == CCE_F32 || dt == CCE_BF16; }
size_t elem_size(cce_dtype dt) { return dt == CCE_BF16 ? 2 : 4; }

cce_status hip_status(hipError_t e) { return e == hipSuccess ? CCE_OK : CCE_ERR_HIP; }

}  // namespace

extern "C" {

const char *cce_status_string(cce_status s) {
    switch (s) {
        case CCE_OK: return "ok";
        case CCE_ERR_NULL: return "a required pointer is NULL";
        case CCE_ERR_SHAPE: return "N, D or V outside the supported range (D % 8 == 0, 8 <= D <= 65536, 1 <= N, V < 2^31)";
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
    if (!shape_ok(N, D, V) || !dtype_ok(dtype)) return 0;
    size_t b = 0;
    fwd_ws(nullptr, fwd_shape(N, D, V), &b);
    return b;
}

size_t cce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype) {
    if (!shape_ok(N, D, V) || !dtype_ok(dtype)) return 0;
    size_t b = 0;
    bwd_ws(nullptr, bwd_shape(N, D, V), elem_size(dtype), &b);
    return b;
}

size_t cce_block_max_elems(int64_t N, int64_t V) {
    if (!shape_ok(N, 8, V)) return 0;
    return (size_t)block_max_elems(N, V);
}

size_t cce_vocab_order_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype) {
    if (!shape_ok(N, D, V) || !dtype_ok(dtype)) return 0;
    size_t b = 0;
    sort_ws(nullptr, N, D, V, &b);
    return b;
}

cce_status cce_forward(const void *H, const void *E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                       cce_dtype dtype, int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                       float *block_max, void *ws, size_t ws_bytes, void *stream) {
    if (!H || !E || !labels || !loss || !lse || !ws) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!aligned(H, 16) || !aligned(E, 16) || !aligned(ws, 16) || !aligned(labels, 8) || !aligned(loss, 4) ||
        !aligned(lse, 4) || !aligned(block_max, 4) || !aligned(perm, 4))
        return CCE_ERR_ALIGN;
    const FwdShape s = fwd_shape(N, D, V);
    size_t need = 0;
    const FwdWs w = fwd_ws(ws, s, &need);
    if (ws_bytes < need) return CCE_ERR_WORKSPACE;
    return hip_status(launch_forward(dtype, H, E, labels, s, ignore_index, perm, w, loss, lse, block_max,
                                     static_cast<hipStream_t>(stream)));
}

cce_status cce_vocab_order(const void *H, const void *E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                           cce_dtype dtype, int64_t ignore_index, int32_t *perm, float *keys, void *ws,
                           size_t ws_bytes, void *stream) {
    if (!H || !E || !labels || !perm || !ws) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!aligned(H, 16) || !aligned(E, 16) || !aligned(ws, 16) || !aligned(labels, 8) || !aligned(perm, 4) ||
        !aligned(keys, 4))
        return CCE_ERR_ALIGN;
    size_t need = 0;
    const SortWs w = sort_ws(ws, N, D, V, &need);
    if (ws_bytes < need) return CCE_ERR_WORKSPACE;
    return hip_status(launch_vocab_order(dtype, H, E, labels, N, D, V, ignore_index, perm, keys, w,
                                         static_cast<hipStream_t>(stream)));
}

cce_status cce_backward(const void *H, const void *E, const int64_t *labels, const float *lse, const float *dloss,
                        const float *block_max, int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                        int64_t ignore_index, float filter_eps, const int32_t *perm, unsigned flags, void *dH,
                        void *dE, int64_t *stats, void *ws, size_t ws_bytes, void *stream) {
    if (!H || !E || !labels || !lse || !dloss || !dH || !dE || !ws) return CCE_ERR_NULL;
    if (!dtype_ok(dtype)) return CCE_ERR_DTYPE;
    if (!shape_ok(N, D, V)) return CCE_ERR_SHAPE;
    if (!(filter_eps >= 0.f) || isinf(filter_eps)) return CCE_ERR_ARG;  // rejects NaN and negatives
    if (flags & ~(CCE_BWD_NO_KAHAN | CCE_BWD_FULL_DE)) return CCE_ERR_ARG;
    if (!aligned(H, 16) || !aligned(E, 16) || !aligned(dH, 16) || !aligned(dE, 16) || !aligned(ws, 16) ||
        !aligned(labels, 8) || !aligned(lse, 4) || !aligned(dloss, 4) || !aligned(perm, 4) || !aligned(stats, 8) ||
        !aligned(block_max, 4))
        return CCE_ERR_ALIGN;
    const BwdShape s = bwd_shape(N, D, V);
    size_t need = 0;
    const BwdWs w = bwd_ws(ws, s, elem_size(dtype), &need);
    if (ws_bytes < need) return CCE_ERR_WORKSPACE;
    return hip_status(launch_backward(dtype, H, E, labels, lse, dloss, block_max, s, ignore_index, filter_eps, perm,
                                      flags, dH, dE, stats, w, static_cast<hipStream_t>(stream)));
}

cce_status cce_check_labels(const int64_t *labels, int64_t N, int64_t V, int64_t ignore_index, int64_t *n_bad,
                            void *stream) {
    if (!labels || !n_bad) return CCE_ERR_NULL;
    if (N < 1 || N >= (int64_t(1) << 31) || V < 1 || V >= (int64_t(1) << 31)) return CCE_ERR_SHAPE;
    if (!aligned(labels, 8) || !aligned(n_bad, 8)) return CCE_ERR_ALIGN;
    return hip_status(launch_check_labels(labels, N, V, ignore_index, n_bad, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
