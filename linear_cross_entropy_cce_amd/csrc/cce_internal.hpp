// Host-side plumbing shared by the launch code and the C ABI of libcce.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cce.h"

namespace cce {

// Logit tile of the forward and of the backward recompute: kTileVocab
// vocabulary entries (MFMA M side) x kTileRows valid tokens (MFMA N side).
constexpr int kTileVocab = 256;
constexpr int kTileRows = 256;
// K pipeline of the logit kernels: LDS stages of kLogitRowBytes per row,
// kLogitStages of them (kLogitStages - 1 in flight).
constexpr int kLogitRowBytes = 128;
constexpr int kLogitStages = 2;
// Gradient-filter block: a quarter of the logit tile.
constexpr int kBlockVocab = 128;
constexpr int kBlockRows = 128;
// The backward's store of kept gradient blocks holds as many blocks as a
// dense [rows x kStoreVocab] slice would (a multiple of 2 kBlockVocab): 32
// KB of store per row at bf16, both layouts; the worst-case pass count, and
// with it the launches a peaked head spends on empty passes, is about
// V / kStoreVocab.
constexpr int kStoreVocab = 16384;
// ... and at least this many blocks (64 MB at bf16, both layouts).
constexpr int64_t kMinStoreBlocks = 1024;
// Workgroups of the persistent backward kernels.
constexpr int kPassGroups = 256;
// Most workgroups of the forward's persistent grid.
constexpr int kFwdMaxGroups = 1024;
// Most vocabulary ranges per token tile in the forward's work split (its
// partial buffers are sized for this many; at most 64, one per lane of the
// merge).
constexpr int kFwdRanges = 32;
// Device scratch of the allocation-free forward (one copy per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;

// The classifier as the kernels see it: rows 0 .. V-1 of the processing
// space, held by one matrix (e1 == e0, v0 >= V) or by the two row blocks of a
// composite head (row v < v0 in the first block, v - v0 in the second).  The
// gradients dE have the same two-block layout.
struct VocabRows {
    const void *e0, *e1;
    int64_t v0;
};
struct VocabGrads {
    void *d0, *d1;
    int64_t v0;
};
constexpr int64_t kOneBlock = INT64_MAX;  // v0 of a one-matrix classifier

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
// Entries of the block-max table: one per 128 x 128 block of the logit
// matrix of the valid rows, [2 ceil(N / 256), 2 ceil(V / 256)], then the
// label logit of each row [N].
inline int64_t block_max_blocks(int64_t N, int64_t V) { return 4 * ceil_div(N, kTileRows) * ceil_div(V, kTileVocab); }
inline int64_t block_max_elems(int64_t N, int64_t V) { return block_max_blocks(N, V) + N; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Carves a caller workspace into aligned regions (or only sizes it when the
// base is null).
struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(size_t count) {
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off = align256(off + count * sizeof(T));
        return p;
    }
};

struct FwdShape {
    int64_t N, D, V;
    int n_vtiles;  // vocabulary tiles of kTileVocab
    int n_rtiles;  // token tiles of kTileRows (upper bound, from N)
};
FwdShape fwd_shape(int64_t N, int64_t D, int64_t V);

struct FwdWs {
    int32_t *idx;      // [N] compacted valid-row indices
    int32_t *nvalid;   // [1]
    int32_t *inv_perm; // [V] processing position of each vocabulary id (with a permutation and the table)
    float *part_m;     // [n_rtiles kFwdRanges, kTileRows] per segment: running max (log2 units)
    float *part_s;     // [n_rtiles kFwdRanges, kTileRows] per segment: sum of 2^(z log2e - m)
    float *zy;         // [N] label logit of each valid row, by compacted position
    int32_t *grid;     // [4] the forward's work split (a, bb, m), recorded for the merge
};
FwdWs fwd_ws(void *ws, const FwdShape &s, size_t *bytes);

// Backward plan.  Work is organised by 256 x 256 logit tiles (token tile rt
// of the valid rows, vocabulary tile vt of the processing order) and their
// four 128 x 128 filter blocks.  Tiles that may keep a block are listed
// vocabulary-tile-major and cut into passes whose kept blocks fit the block
// store (cap blocks); every pass runs recompute -> dE -> dH on its range.
struct BwdShape {
    int64_t N, D, V;
    int64_t Np;        // N rounded up to kTileRows
    int n_rtiles;      // Np / kTileRows
    int n_vtiles;      // ceil(V / kTileVocab)
    int n_rb;          // Np / kBlockRows
    int cbp;           // 2 n_vtiles: row width of the block maps
    int64_t cap;       // block-store capacity (blocks)
    int64_t cap_eff;   // cap - 2 n_rb: pass packing bound (a vocabulary tile adds at most 2 n_rb blocks)
    int max_passes;
    int plan_ints;     // size of the plan record
};
BwdShape bwd_shape(int64_t N, int64_t D, int64_t V);

struct BwdWs {
    int32_t *idx;      // [N]
    int32_t *nvalid;   // [1]
    int32_t *inv_perm; // [V] processing position of each vocabulary id
    float *lmin;       // [n_rb] smallest lse of each 128-token block (for the block-max bound)
    float *glab;       // [Np] label-entry gradient of rows whose label block is label-only (else 0)
    uint8_t *lab;      // [n_rb, cbp] valid tokens whose label falls in the block
    uint8_t *st;       // [n_rb, cbp] block status: 0 dropped, 1 softmax kept, 2 label only
    int32_t *slot;     // [n_rb, cbp] store slot of a kept block
    uint16_t *smask;   // [n_rb, cbp] 32 x 32 sub-tiles of a kept block whose gradient may be nonzero
    uint8_t *csoft;    // [cbp] 1 where a block of the vocabulary block (column) may keep a softmax part
    int32_t *cnlab;    // [cbp] blocks of the column that hold a label
    int32_t *cent;     // [cbp] valid tokens whose label falls in the column
    int32_t *vneed;    // [n_vtiles] blocks the vocabulary tile's tiles may keep
    int32_t *vact;     // [n_vtiles] its tiles that may keep one
    int32_t *cpre;     // [cbp + 1] static columns (see k_plan) before each column
    int32_t *slist;    // [cbp] static columns, in order
    int32_t *ipre;     // [cbp + 1] work items before each static column (slist order)
    int32_t *citem;    // work items of the static columns: column
    int32_t *cft;      //   and 256-feature tile (-1: every feature; -2 - f: 32-feature tile f of a hot column)
    int32_t *tpos;     // [N] label position of each valid token (-1: none)
    int32_t *hidx;     // [cbp] index of a hot column (-1: not hot)
    int32_t *hcol;     // [hmax] the hot columns
    int32_t *hent;     // [hmax + 1] first entry of each hot column
    int32_t *nhot;     // [1] hot columns
    int32_t *hrlo;     // [hmax, 129] entries before each row of a hot column
    int32_t *hent_t;   // [N] the hot columns' entries (valid-token positions), grouped by row
    int32_t *hcnt;     // [hmax, slices, 128] entries per token slice and row of each hot column
    int32_t *dlist;    // [cbp] the other columns, in order
    uint8_t *tneed;    // [n_vtiles, n_rtiles] blocks the tile may keep (bits 0-2), recompute flag (bit 7)
    int64_t *cum;      // [n_vtiles] plan scratch: cumulative blocks
    int32_t *act;      // [n_vtiles] plan scratch: listed tiles before each vocabulary tile
    int32_t *tlist;    // [n_vtiles * n_rtiles] active tiles, vocabulary-tile-major
    int32_t *plan;     // [plan_ints] passes, active tiles, per-pass ranges and slot counters
    float *dh_acc;     // [Np, D] fp32 running dH across passes (max_passes > 1)
    void *Ht;          // [D, Np] valid rows of H, transposed
    void *Gt;          // [cap, 128, 128] kept gradient blocks, vocabulary-major
    void *Gn;          // [cap, 128, 128] the same blocks, row-major
};
BwdWs bwd_ws(void *ws, const BwdShape &s, size_t elem, size_t *bytes);

struct SortWs {
    float *hsum_part;  // [P, D] partial column sums of valid H rows
    float *hbar;       // [D]
    float *keys;       // [V]
    uint32_t *ukeys[2];
    int32_t *vals[2];
    uint32_t *hist;    // [tiles * 256]
    int32_t *idx;      // [N] compacted valid-row indices
    int32_t *nvalid;   // [1]
};
SortWs sort_ws(void *ws, int64_t N, int64_t D, int64_t V, size_t *bytes);

// Device address of the allocation-free forward's scratch on the current
// device (looked up once per device, then cached).
hipError_t noalloc_scratch(void **ptr);

// ---- launchers (return hipGetLastError() after enqueuing) ----
hipError_t launch_compact(const int64_t *labels, int64_t N, int64_t ignore_index, int32_t *idx,
                          int32_t *nvalid, hipStream_t st);
hipError_t launch_check_labels(const int64_t *labels, int64_t N, int64_t V, int64_t ignore_index,
                               int64_t *n_bad, hipStream_t st);
hipError_t launch_inv_perm(const int32_t *perm, int V, int32_t *inv, hipStream_t st);
hipError_t launch_seg_labels(const int64_t *labels, int64_t N, int64_t ignore_index, int64_t V0, int64_t off1,
                             int64_t V1, int64_t *out, hipStream_t st);
hipError_t launch_forward(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels,
                          const FwdShape &s, int64_t ignore_index, const int32_t *perm, const FwdWs &w,
                          float *loss, float *lse, float *block_max, hipStream_t st);
hipError_t launch_backward(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels,
                           const float *lse, const float *dloss, const float *block_max, const BwdShape &s,
                           int64_t ignore_index, float eps, const int32_t *perm, unsigned flags,
                           void *dH, const VocabGrads &dE, int64_t *stats, const BwdWs &w, hipStream_t st);
hipError_t launch_vocab_order(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels,
                              int64_t N, int64_t D, int64_t V, int64_t ignore_index, int32_t *perm,
                              float *keys_out, const SortWs &w, hipStream_t st);

}  // namespace cce
