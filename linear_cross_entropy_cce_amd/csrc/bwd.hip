// Backward of the fused classifier-head + cross-entropy on gfx950.
//
// The backward recomputes the logits blockwise from H and E (no logits are
// kept from the forward), skips blocks whose softmax entries (other than the
// label entries, whose gradient dloss (p - 1) is always kept) all fall below
// a threshold, and accumulates the classifier gradient with Kahan compensation
// (CCE paper summary "Cut Your Losses in Large-Vocabulary Language Models",
// sections "Approach" and "Limitations"; lit note "The loss and the mask: Cut
// Cross-Entropy + FlexAttention", section "Contribution").
//
// Layout of the work.  D (2048-4096 for the heads of interest) is far wider
// than an attention head, so dH_i and dE_v rows cannot stay on chip while the
// other dimension is swept.  The gradient G = dloss (p - onehot) of every
// kept 128 x 128 filter block is therefore written once, in two layouts, to a
// block store, and the two gradient products read it back:
//
//   plan        which 128 x 128 blocks may be kept: all of them, or, with the
//               forward's block-max table, only blocks whose largest non-label
//               logit comes near the smallest lse of their rows, plus blocks
//               holding a label; the 256 x 256 logit tiles holding such blocks
//               are listed and cut, in vocabulary order, into passes whose
//               blocks fit the store
//   k_g_pass    per listed tile: recompute the logits of the blocks that may
//               keep a softmax part (MFMA, the forward's code and K order),
//               p = exp(z - lse), block filter, and the kept blocks' G into
//               the store; a label-only block (only label entries kept) gets
//               its label entries from the forward's label logits when it was
//               not recomputed, and records each row's label gradient
//   k_grad_pass both products of the pass in one launch:
//               dE_v = sum over kept row blocks of G^T H (MFMA), Kahan-
//               compensated across row blocks, written once;
//               dH_i = sum over blocks with a kept softmax part of G E (MFMA
//               with E read through the LDS transpose loads), the running sum
//               kept in fp32 across passes, plus g_i e_{y_i} for a row whose
//               label block is label-only
//
// When the softmax is peaked almost every tile is dropped before its logits
// are formed and one pass holds every kept block; when it is flat the passes
// stream through the vocabulary like dense chunks.  Extra memory is linear in
// N and V (store, transposed H) plus one byte-sized entry per block.
#include <math.h>

#include <algorithm>

#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {

using TileF = Tile<kTileVocab, kTileRows, 2, 4>;   // logit tile: A = vocabulary, B = tokens; 8 waves
using TileFD = TileF;                             // tile of the DMA recompute
using TileG = Tile<128, 256, 2, 4>;               // dE / dH tile: A = a 128-row gradient block, B = 256 features
static_assert(TileG::BM == kBlockVocab && TileG::BM == kBlockRows, "gradient GEMM rows = one filter block");
static_assert(kTileVocab == 2 * kBlockVocab && kTileRows == 2 * kBlockRows, "a logit tile holds 2 x 2 blocks");

constexpr int kBlockElems = kBlockRows * kBlockVocab;  // elements of one stored block
constexpr int kListCap = 512;
// At most this many label entries go through the label path at once.
constexpr int kLabelEntries = 512;
// dE's compensated (Kahan) sum takes one term per this many kept row blocks
// of a vocabulary block: each term is an fp32 MFMA sum over up to 512 tokens.
constexpr int kKahanBlocks = 4;
// A vocabulary block whose kept blocks are all label-only takes the label
// path (its dE rows from the label entries, one pass over a row of H per
// entry, instead of block products over every token of its kept blocks)
// when it has at most kLabelEntries label entries.
__host__ __device__ __forceinline__ bool label_path_ok(int n_entries) { return n_entries <= kLabelEntries; }
// A static column (see k_plan) with more label entries than this is split
// into one work item per 256-feature tile; the others are one item each.
constexpr int kColSplitEntries = 32;
// Feature tile of a static column item that covers every feature.
constexpr int kAllFeatures = -1;
// 256-feature tiles of a row of D features (the products' tile width), and
// the kHotF-feature tiles of a hot column's items.
constexpr int kHotF = 32;
__host__ __device__ __forceinline__ int n_feature_tiles(int64_t D) { return (int)((D + 255) / 256); }
__host__ __device__ __forceinline__ int n_hot_tiles(int64_t D) { return (int)((D + kHotF - 1) / kHotF); }
static_assert(TileG::BN == 256, "feature tiles of the products");
// Hot columns: at most hot_max of them; their entries are counted and placed
// in hot_slices token slices of hot_slice tokens (a multiple of 1024, at
// most 64 slices).
inline int64_t hot_max(int64_t N, int64_t cbp) { return std::min<int64_t>(cbp, N / (kLabelEntries + 1) + 1); }
inline int hot_slice(int64_t N) { return 1024 * (int)((N + 1024 * 64 - 1) / (1024 * 64)); }
inline int hot_slices(int64_t N) { return (int)((N + hot_slice(N) - 1) / hot_slice(N)); }

// Plan record: P, number of listed tiles, first vocabulary tile of each pass
// [max_passes + 1], first list entry of each pass [max_passes + 1], store
// slot counter of each pass [max_passes].
struct PlanView {
    int32_t *P, *n_active, *vt_begin, *list_begin, *counter;
};
__device__ __forceinline__ PlanView plan_view(int32_t *plan, int max_passes) {
    return {plan, plan + 1, plan + 2, plan + 3 + max_passes, plan + 4 + 2 * max_passes};
}
// After the record, per pass kQueues work-queue counters (8 for the
// recompute phase, one per XCD part of the tile list, and 1 for the gradient
// phase).
constexpr int kQueues = 9;
static int plan_ints(int max_passes) { return 4 + (3 + kQueues) * max_passes; }
__device__ __forceinline__ int32_t *plan_queues(int32_t *plan, int max_passes, int p) {
    return plan + 4 + 3 * max_passes + kQueues * p;
}

// Next item of a work queue for the whole workgroup: thread 0 takes a
// ticket, the others read it from LDS.  Items go to whichever workgroup asks
// first; what an item computes does not depend on which one runs it.
__device__ __forceinline__ int take_ticket(int32_t *counter, int *slot) {
    if (threadIdx.x == 0) *slot = atomicAdd(counter, 1);
    __syncthreads();
    const int t = *slot;
    __syncthreads();  // every thread has read the ticket before the next one overwrites it
    return t;
}

// Everything the pass kernels read or write.
template <typename T>
struct BwdArgs {
    int32_t *plan;
    int max_passes;
    const int32_t *tlist;
    const uint8_t *tneed;
    int n_rt;
    const T *H, *Ht;
    Rows2<const T> E;  // classifier rows in processing space (one matrix or two blocks)
    int64_t ldh;  // Np
    const int32_t *idx, *nvalid, *perm, *inv_perm;
    const int64_t *labels;
    const float *lse, *dloss;
    const float *zlab;  // [N] label logit of each valid row from the forward's tiles (with the table)
    float *glab;        // [N] by valid-row position: gradient of the label entry of a label-only block, else 0
    int D, V, cbp, n_rb;
    float eps;
    int full_de;  // dE from every block (status 3 = kept for dE only), dH filtered
    int fine;     // the filter decides per 32 x 32 sub-tile (CCE_BWD_FINE_FILTER)
    T *Gt, *Gn;
    int64_t cap;
    int64_t cap_take;  // slots the epilogue may take: cap (cap / 2 with CCE_BWD_DEBUG_STORE_LIMIT)
    uint8_t *st;
    int32_t *slot;
    uint16_t *smask;  // bit 4 i + j: sub-tile (vocabulary rows 32 i.., tokens 32 j..) of a kept block may be nonzero
    const int32_t *cpre, *slist, *dlist;  // column lists of k_plan
    const int32_t *ipre, *citem, *cft;    // static column items of k_plan
    const int32_t *hidx, *hent, *hrlo, *hent_t;  // hot columns (k_plan, k_hot_count, k_hot_place)
    const int32_t *cent;                  // label entries per column
    int CB;                               // vocabulary blocks
    int64_t *stats;
    float *dh_acc;
    Rows2<T> dE;  // same layout as E
    T *dH;
};

// ------------------------------------------------------------ small kernels
constexpr int kStatsLen = 7;  // entries of the stats array

__global__ void k_stats_fin(int64_t *stats, const int32_t *__restrict__ nvalid_p, int64_t n_vblocks) {
    if (threadIdx.x == 0) {
        const int64_t nv = *nvalid_p;
        stats[2] = ((nv + kBlockRows - 1) / kBlockRows) * n_vblocks;
        stats[3] = nv;
    }
}

// lmin[rb] = smallest lse over the valid tokens of 128-token block rb (+inf
// if none), for rb = 2 b and 2 b + 1 (one per half of a 256-thread group).
__device__ __forceinline__ void lse_min_pair(const float *__restrict__ lse, const int32_t *__restrict__ idx,
                                             const int32_t *__restrict__ nvalid_p, float *__restrict__ lmin,
                                             int n_rb, int64_t b, float *part) {
    const int half = threadIdx.x >> 7;
    const int64_t rb = 2 * b + half;
    const int64_t tok = rb * kBlockRows + (threadIdx.x & 127);
    float v = tok < *nvalid_p ? lse[idx[tok]] : __builtin_huge_valf();
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if ((threadIdx.x & 127) == 0 && rb < n_rb) lmin[rb] = fminf(part[2 * half], part[2 * half + 1]);
}

// True when every p in block (rb, cb) is provably below eps / 2: the block's
// largest logit T minus the smallest lse L of its tokens is below
// thr = ln(eps / 2), with a relative margin for fp32 rounding of the
// recomputed logits and of T - L.  The filter then keeps nothing of the
// block's softmax part.  NaN never passes.
__device__ __forceinline__ bool block_below(const float *__restrict__ bmax, int64_t ld,
                                            const float *__restrict__ lmin, float thr, int rb, int cb) {
    if (!bmax) return false;
    const float T = bmax[(int64_t)rb * ld + cb];
    const float L = lmin[rb];
    return (T - L) + 0x1p-10f * (fabsf(T) + fabsf(L)) < thr;
}

// dst[c][j] = src[row(j)][c] for c < cols, j < n_out; rows j >= n_rows give 0.
// row(j) = rowmap ? rowmap[row0 + j] : row0 + j.  64 x 64 tiles through LDS.
template <typename T>
__device__ __forceinline__ void transpose_tile(const T *__restrict__ src, int64_t ld_src, int64_t n_src_rows,
                                               const int32_t *__restrict__ rowmap, int64_t row0,
                                               const int32_t *__restrict__ n_rows_dev, int n_rows_host, int cols,
                                               int n_out, T *__restrict__ dst, int64_t ld_dst, int bx, int by,
                                               T (*tile)[64 + 2]) {
    constexpr int CE = ChunkElems<T>::value;
    const int n_rows = n_rows_dev ? *n_rows_dev : n_rows_host;
    const int j0 = bx * 64;
    const int c0 = by * 64;
    for (int q = threadIdx.x; q < 64 * (64 / CE); q += 256) {
        const int jj = q / (64 / CE);
        const int cc = (q % (64 / CE)) * CE;
        const int j = j0 + jj;
        const int c = c0 + cc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < n_rows && c < cols) {
            const int64_t row = rowmap ? rowmap[row0 + j] : row0 + j;
            if (row >= 0 && row < n_src_rows) v = ld16(reinterpret_cast<const char *>(src + row * ld_src + c));
        }
        const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int k = 0; k < CE; ++k) tile[jj][cc + k] = e[k];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * (64 / CE); q += 256) {
        const int cc = q / (64 / CE);
        const int jj = (q % (64 / CE)) * CE;
        const int c = c0 + cc;
        const int j = j0 + jj;
        if (c >= cols || j >= n_out) continue;
        u32x4 v;
        T *e = reinterpret_cast<T *>(&v);
#pragma unroll
        for (int k = 0; k < CE; ++k) e[k] = tile[jj + k][cc];
        *reinterpret_cast<u32x4 *>(dst + (int64_t)c * ld_dst + j) = v;
    }
}

// The backward's clearing, one grid-stride launch: three regions of 32-bit
// words (the label map; the plan's column and tile sums; the label
// gradients), the stats entries if given, and dH = 0 for the rows whose
// label is ignore_index (one wave per row).
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_clear(uint32_t *__restrict__ r0, int64_t n0, uint32_t *__restrict__ r1,
                                                   int64_t n1, uint32_t *__restrict__ r2, int64_t n2,
                                                   int64_t *__restrict__ stats, const int64_t *__restrict__ labels,
                                                   int64_t N, int D, int64_t ignore_index, T *__restrict__ dH) {
    constexpr int CE = ChunkElems<T>::value;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int64_t i = i0; i < n0; i += stride) r0[i] = 0u;
    for (int64_t i = i0; i < n1; i += stride) r1[i] = 0u;
    for (int64_t i = i0; i < n2; i += stride) r2[i] = 0u;
    if (stats && i0 < kStatsLen) stats[i0] = 0;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < N; row += (int64_t)gridDim.x * 4) {
        if (labels[row] != ignore_index) continue;  // (wave-uniform)
        for (int k = lane * CE; k < D; k += 64 * CE) *reinterpret_cast<u32x4 *>(dH + row * D + k) = z;
    }
}

// Compacts the indices i in [0, n) with flag(i) != 0 into list[], in order,
// using every thread of the workgroup (wave ballots + per-wave offsets).
// Returns the count.  Must be called by all threads.
template <int kThreads, class Flag>
__device__ __forceinline__ int build_list(int n, Flag flag, int *list, int *wcnt) {
    constexpr int kW = kThreads / 64;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int total = 0;
    for (int base = 0; base < n; base += kThreads) {
        const int i = base + t;
        const bool f = i < n && flag(i);
        const uint64_t b = __ballot(f);
        if (lane == 0) wcnt[wave] = __popcll(b);
        __syncthreads();
        int off = total;
        for (int w = 0; w < wave; ++w) off += wcnt[w];
        if (f) list[off + __popcll(b & below)] = i;
        int sum = 0;
        for (int w = 0; w < kW; ++w) sum += wcnt[w];
        total += sum;
        __syncthreads();
    }
    return total;
}

// The K stages, among kspb per block, of the listed blocks 0 .. n-1 that
// cover a sub-tile whose gradient may be nonzero: stage k of block i is
// listed iff mask[i] & sel(k).  Entries (i << 4 | k) in block then stage
// order, bit 31 set on each block's last listed stage.  Returns their number.
// Must be called by all threads.
template <int kThreads, class Sel>
__device__ __forceinline__ int build_stages(int n, int kspb, const int *mask, Sel sel, int *stl, int *wtot) {
    constexpr int kW = kThreads / 64;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int total = 0;
    for (int base = 0; base < n; base += kThreads) {
        const int i = base + t;
        int c = 0;
        if (i < n)
            for (int k = 0; k < kspb; ++k) c += (mask[i] & sel(k)) != 0;
        int x = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) wtot[wave] = x;
        __syncthreads();
        int off = total + x - c;
        for (int w = 0; w < wave; ++w) off += wtot[w];
        if (i < n) {
            int last = -1;
            for (int k = 0; k < kspb; ++k)
                if (mask[i] & sel(k)) {
                    stl[off] = (i << 4) | k;
                    last = off++;
                }
            if (last >= 0) stl[last] |= (int)0x80000000u;
        }
        int sum = 0;
        for (int w = 0; w < kW; ++w) sum += wtot[w];
        total += sum;
        __syncthreads();
    }
    return total;
}

// ------------------------------------------------------------------ plan
// lab[rb][cb] = the number of valid tokens of row block rb whose label falls
// in vocabulary block cb (processing order; zeroed before).  A block holds
// at most 128 tokens, so each count fits its byte: the byte is added to
// through its aligned 32-bit word (the map's region is 256-byte aligned and
// padded).  tpos[t] = the label's position in processing order (-1: not a
// valid label).
__device__ __forceinline__ void label_map_block(const int64_t *__restrict__ labels, const int32_t *__restrict__ idx,
                                                const int32_t *__restrict__ nvalid_p,
                                                const int32_t *__restrict__ inv_perm, int64_t V, int cbp,
                                                uint8_t *__restrict__ lab, int32_t *__restrict__ tpos, int64_t b) {
    const int64_t t = b * 256 + threadIdx.x;
    if (t >= *nvalid_p) return;
    const int64_t y = labels[idx[t]];
    if (y < 0 || y >= V) {  // not a valid label: undefined by contract
        tpos[t] = -1;
        return;
    }
    const int64_t pos = inv_perm ? inv_perm[y] : y;
    tpos[t] = (int32_t)pos;
    const int64_t i = (t / kBlockRows) * cbp + pos / kBlockVocab;
    atomicAdd(reinterpret_cast<uint32_t *>(lab + (i & ~int64_t(3))), 1u << (8 * (i & 3)));
}

// Per tile (vocabulary-tile-major index vt * n_rt + rt): the number of its
// blocks that may be kept (bits 0-2), which of its blocks may keep a
// softmax part (bits 3-6, block q = 2 (vocabulary half) + token half) and
// whether any does (bit 7).  A block may keep its softmax part unless the
// bound rules it out, and may keep its label entries if it holds a label;
// only the blocks that may keep a softmax part are recomputed.  Per
// vocabulary block (column, zeroed before): csoft = 1 if one of its blocks
// may keep a softmax part, cnlab = its blocks that hold a label, cent = the
// valid tokens whose label falls in it.  Per vocabulary tile (zeroed
// before): vneed = the blocks its tiles may keep, vact = its tiles that may
// keep one.
__global__ __launch_bounds__(256) void k_tile_class(const int32_t *__restrict__ nvalid_p, int64_t V, int n_rt,
                                                    int n_vt, int cbp, const uint8_t *__restrict__ lab,
                                                    const float *__restrict__ bmax, const float *__restrict__ lmin,
                                                    float thr, uint8_t *__restrict__ tneed,
                                                    uint8_t *__restrict__ csoft, int32_t *__restrict__ cnlab,
                                                    int32_t *__restrict__ cent, int32_t *__restrict__ vneed,
                                                    int32_t *__restrict__ vact) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)n_rt * n_vt) return;
    const int vt = (int)(i / n_rt), rt = (int)(i % n_rt);
    const int nv = *nvalid_p;
    if ((int64_t)rt * kTileRows >= nv) {
        tneed[i] = 0;
        return;
    }
    int mask = 0, need = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rb = 2 * rt + (q & 1), cb = 2 * vt + (q >> 1);
        if ((int64_t)rb * kBlockRows >= nv || (int64_t)cb * kBlockVocab >= V) continue;
        const bool soft = !block_below(bmax, cbp, lmin, thr, rb, cb);
        const int n_lab = lab[(int64_t)rb * cbp + cb];
        const bool has_label = n_lab != 0;
        mask |= soft ? 1 << q : 0;
        need += (soft || has_label) ? 1 : 0;
        if (soft) csoft[cb] = 1;  // (every writer stores 1)
        if (has_label) {
            atomicAdd(&cnlab[cb], 1);
            atomicAdd(&cent[cb], n_lab);
        }
    }
    tneed[i] = (uint8_t)(need | (mask << 3) | (mask ? 0x80 : 0));
    if (need) {
        atomicAdd(&vneed[vt], need);
        atomicAdd(&vact[vt], 1);
    }
}

// Both columns of vocabulary tile vt are static (a column past the
// vocabulary counts as static: it holds no block).
__device__ __forceinline__ bool vt_static(const int32_t *__restrict__ cpre, int vt, int CB) {
    const int c0 = 2 * vt, c1 = 2 * vt + 1;
    return c0 < CB && cpre[c0 + 1] - cpre[c0] == 1 && (c1 >= CB || cpre[c1 + 1] - cpre[c1] == 1);
}

// One workgroup: prefix sums of the blocks each vocabulary tile may keep and
// of its listed tiles (vneed, vact from k_tile_class), the pass of each
// vocabulary tile and the per-pass ranges; tile_list_block then writes the tile
// list (vocabulary-tile-major, token tiles in order).
// Passes: one if every block fits the store, else pass(vt) =
// floor(cum(vt) / cap_eff) with cum the inclusive block count; a vocabulary
// tile adds at most cap - cap_eff blocks, so no pass exceeds cap.
// Columns (vocabulary blocks cb < CB): with static_ok, a column with more
// than kLabelEntries label entries is hot (hidx[cb] = its index h in hcol,
// its entries from hent[h] on in the hot entry list; nhot of them), whatever
// the bound says; and a column none of whose blocks may keep a softmax part
// and whose label entries pass label_path_ok, or that is hot, is static: its
// kept blocks can only be label-only, so its dE rows come from the label
// entries (or are zero), as the per-feature-tile items would write them.
// slist holds the static columns in order, dlist the others, and cpre[cb]
// the static columns before cb (cpre[CB] all of them).  A static column is
// one work item, or n_dt (one per 256-feature tile) when it has more than
// kColSplitEntries label entries, or one per kHotF-feature tile when it is hot:
// citem and cft list the items in column order (column, and the 256-feature
// tile, kAllFeatures for a whole column, or -2 - the kHotF-feature tile of a
// hot column) and ipre[j] the items before static column j (ipre[cpre[CB]]
// all of them).  The
// label-only blocks of static columns (their label blocks) are counted into
// stats[1] here; the tile epilogue counts the others.
__global__ __launch_bounds__(1024) void k_plan(const int32_t *__restrict__ vneed, const int32_t *__restrict__ vact,
                                               int n_vt, int64_t cap, int64_t cap_eff, int max_passes,
                                               int32_t *__restrict__ plan, int64_t *__restrict__ cum,
                                               int32_t *__restrict__ act, int CB, int static_ok,
                                               const uint8_t *__restrict__ csoft, const int32_t *__restrict__ cnlab,
                                               const int32_t *__restrict__ cent, int32_t *__restrict__ cpre,
                                               int32_t *__restrict__ slist, int32_t *__restrict__ dlist, int n_dt,
                                               int n_d64,
                                               int32_t *__restrict__ ipre, int32_t *__restrict__ citem,
                                               int32_t *__restrict__ cft, int32_t *__restrict__ hidx,
                                               int32_t *__restrict__ hcol, int32_t *__restrict__ hent,
                                               int32_t *__restrict__ nhot, int64_t *__restrict__ stats) {
    __shared__ int64_t wsum[16];
    __shared__ int32_t wact[16];
    __shared__ int32_t wcol[16], witem[16], whot[16], went[16];
    __shared__ int64_t carry_n;
    __shared__ int32_t carry_a, carry_c, carry_i, carry_h, carry_e;
    const PlanView pv = plan_view(plan, max_passes);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    if (t == 0) { carry_c = 0; carry_i = 0; carry_h = 0; carry_e = 0; }
    __syncthreads();
    int64_t n_static_lab = 0;
    const bool can_split = n_dt > 1;
    for (int base = 0; base < CB; base += 1024) {
        const int cb = base + t;
        const int ce = cb < CB ? cent[cb] : 0;
        const int hot = (cb < CB && static_ok && !label_path_ok(ce)) ? 1 : 0;
        const int is_s = (cb < CB && static_ok && !csoft[cb] && (label_path_ok(ce) || hot)) ? 1 : 0;
        const int ni = is_s ? (hot ? n_d64 : (can_split && ce > kColSplitEntries ? n_dt : 1)) : 0;
        if (is_s) n_static_lab += cnlab[cb];
        int x = is_s, xi = ni, xh = hot, xe = hot ? ce : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            const int yi = __shfl_up(xi, o, 64);
            const int yh = __shfl_up(xh, o, 64);
            const int ye = __shfl_up(xe, o, 64);
            if (lane >= o) { x += y; xi += yi; xh += yh; xe += ye; }
        }
        if (lane == 63) { wcol[w] = x; witem[w] = xi; whot[w] = xh; went[w] = xe; }
        __syncthreads();
        int off = carry_c, offi = carry_i, offh = carry_h, offe = carry_e;
        for (int k = 0; k < w; ++k) { off += wcol[k]; offi += witem[k]; offh += whot[k]; offe += went[k]; }
        const int excl = off + x - is_s, iexcl = offi + xi - ni;
        const int hexcl = offh + xh - hot, eexcl = offe + xe - (hot ? ce : 0);
        if (cb < CB) {
            cpre[cb] = excl;
            hidx[cb] = hot ? hexcl : -1;
            if (hot) {
                hcol[hexcl] = cb;
                hent[hexcl] = eexcl;
            }
            if (is_s) {
                slist[excl] = cb;
                ipre[excl] = iexcl;
                for (int k = 0; k < ni; ++k) {
                    citem[iexcl + k] = cb;
                    cft[iexcl + k] = hot ? -2 - k : (ni == 1 ? kAllFeatures : k);
                }
            } else {
                dlist[cb - excl] = cb;
            }
        }
        __syncthreads();
        if (t == 1023) { carry_c = off + x; carry_i = offi + xi; carry_h = offh + xh; carry_e = offe + xe; }
        __syncthreads();
    }
    if (t == 0) {
        cpre[CB] = carry_c;
        ipre[carry_c] = carry_i;
        hent[carry_h] = carry_e;
        *nhot = carry_h;
    }
    if (stats) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) n_static_lab += __shfl_xor(n_static_lab, o, 64);
        if (lane == 0 && n_static_lab)
            atomicAdd(reinterpret_cast<unsigned long long *>(stats + 1), (unsigned long long)n_static_lab);
    }
    __syncthreads();  // cpre is read below
    if (t == 0) { carry_n = 0; carry_a = 0; }
    __syncthreads();
    for (int base = 0; base < n_vt; base += 1024) {
        const int vt = base + t;
        int64_t nd = 0;
        int ac = 0;
        if (vt < n_vt) {
            nd = vneed[vt];
            // (a vocabulary tile whose columns are both static lists no tile:
            // label_static_block writes what its tiles would)
            ac = vt_static(cpre, vt, CB) ? 0 : vact[vt];
        }
        int64_t xs = nd;
        int xa = ac;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t ys = __shfl_up(xs, o, 64);
            const int ya = __shfl_up(xa, o, 64);
            if (lane >= o) { xs += ys; xa += ya; }
        }
        if (lane == 63) { wsum[w] = xs; wact[w] = xa; }
        __syncthreads();
        int64_t off = carry_n;
        int offa = carry_a;
        for (int k = 0; k < w; ++k) { off += wsum[k]; offa += wact[k]; }
        if (vt < n_vt) {
            cum[vt] = off + xs;          // inclusive
            act[vt] = offa + xa - ac;    // exclusive
        }
        __syncthreads();
        if (t == 1023) { carry_n = off + xs; carry_a = offa + xa; }
        __syncthreads();
    }
    const int64_t total = carry_n;
    const int n_active = carry_a;
    auto pass_of = [&](int vt) -> int {
        if (total <= cap) return 0;
        const int64_t q = cum[vt] / cap_eff;
        return q < max_passes - 1 ? (int)q : max_passes - 1;
    };
    for (int vt = t; vt < n_vt; vt += 1024) {
        const int p = pass_of(vt);
        const int pp = vt ? pass_of(vt - 1) : -1;
        for (int q = pp + 1; q <= p; ++q) {
            pv.vt_begin[q] = vt;
            pv.list_begin[q] = act[vt];
        }
    }
    if (t == 0) {
        const int P = pass_of(n_vt - 1) + 1;
        *pv.P = P;
        *pv.n_active = n_active;
        for (int q = P; q <= max_passes; ++q) {
            pv.vt_begin[q] = n_vt;
            pv.list_begin[q] = n_active;
        }
    }
    for (int q = t; q < max_passes; q += 1024) pv.counter[q] = 0;
    for (int q = t; q < kQueues * max_passes; q += 1024) plan_queues(plan, max_passes, 0)[q] = 0;

}

// The tile list: the listed tiles (that may keep a block) of vocabulary tile
// vt at act[vt] onwards, token tiles in order.  One wave per vocabulary tile.
// A vocabulary tile whose columns are both static lists nothing (k_plan
// counted none); in the others a tile that recomputes nothing and whose
// label blocks all lie in static columns gets -1 (label_static_block writes what
// it would have).
__device__ __forceinline__ void tile_list_block(const uint8_t *__restrict__ tneed, int n_rt, int n_vt,
                                                const int32_t *__restrict__ act, const uint8_t *__restrict__ lab,
                                                int cbp, const int32_t *__restrict__ cpre, int CB,
                                                int32_t *__restrict__ tlist, int64_t b) {
    const int lane = threadIdx.x & 63;
    const int vt = (int)(b * 4 + (threadIdx.x >> 6));
    if (vt >= n_vt || vt_static(cpre, vt, CB)) return;  // wave-uniform
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const uint8_t *row = tneed + (int64_t)vt * n_rt;
    bool col_static[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int cb = 2 * vt + h;
        col_static[h] = cb < CB && cpre[cb + 1] - cpre[cb] == 1;
    }
    int pos = act[vt];
    for (int r0 = 0; r0 < n_rt; r0 += 64) {
        const int rt = r0 + lane;
        const int tn8 = rt < n_rt ? row[rt] : 0;
        const bool on = (tn8 & 7) != 0;
        bool skip = false;
        if (on && !(tn8 & 0x80)) {  // only label blocks: skip when every one is in a static column
            skip = true;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (lab[(int64_t)(2 * rt + j) * cbp + 2 * vt + h] && !col_static[h]) skip = false;
        }
        const uint64_t bal = __ballot(on);
        if (on) tlist[pos + __popcll(bal & below)] = skip ? -1 : vt * n_rt + rt;
        pos += __popcll(bal);
    }
}

// The label-only blocks of static columns (see k_plan), which no listed
// tile holds unless the tile's other column needs it: per valid token whose
// label falls in a static column, the block's status (2, label only) and the
// label entry's fp32 gradient dloss (p - 1), p from the forward's label logit
// (the values the tile epilogue writes for a block it does not recompute).
__device__ __forceinline__ void label_static_block(const int64_t *__restrict__ labels,
                                                   const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ nvalid_p,
                                                   const int32_t *__restrict__ inv_perm, int64_t V, int cbp,
                                                   const int32_t *__restrict__ cpre, const float *__restrict__ lse,
                                                   const float *__restrict__ dloss, const float *__restrict__ zlab,
                                                   uint8_t *__restrict__ st, float *__restrict__ glab, int64_t b) {
    const int64_t t = b * 256 + threadIdx.x;
    if (t >= *nvalid_p) return;
    const int64_t row = idx[t];
    const int64_t y = labels[row];
    if (y < 0 || y >= V) return;  // not a valid label: undefined by contract
    const int64_t pos = inv_perm ? inv_perm[y] : y;
    const int cb = (int)(pos / kBlockVocab);
    if (cpre[cb + 1] - cpre[cb] != 1) return;  // not a static column
    st[(t / kBlockRows) * cbp + cb] = 2;       // (every token of the block stores 2)
    const float dl = dloss[row];
    if (dl != 0.f) {
        const float pl = __builtin_amdgcn_exp2f((zlab[row] - lse[row]) * kLog2e);
        glab[t] = dl * (pl - 1.f);
    }
}

// The setup work that needs the compacted rows, one launch: workgroups
// [0, n_tr) transpose H's valid rows (64 x 64 tiles, n_tx per row of
// tiles), the next n_lse the smallest lse of two row blocks each (with the
// block-max table), the rest the label map (256 tokens each).
template <typename T>
__global__ __launch_bounds__(256) void k_bwd_prep(const T *__restrict__ H, int D, int64_t N,
                                                  const int32_t *__restrict__ idx, const int32_t *__restrict__ nvalid_p,
                                                  int Np, T *__restrict__ Ht, int n_tx, int64_t n_tr,
                                                  const float *__restrict__ lse, float *__restrict__ lmin, int n_rb,
                                                  int64_t n_lse, const int64_t *__restrict__ labels,
                                                  const int32_t *__restrict__ inv_perm, int64_t V, int cbp,
                                                  uint8_t *__restrict__ lab, int32_t *__restrict__ tpos) {
    __shared__ T tile[64][64 + 2];
    __shared__ float part[4];
    int64_t b = blockIdx.x;
    if (b < n_tr) {  // (uniform)
        transpose_tile<T>(H, D, N, idx, 0, nvalid_p, 0, D, Np, Ht, Np, (int)(b % n_tx), (int)(b / n_tx), tile);
        return;
    }
    b -= n_tr;
    if (b < n_lse) {
        lse_min_pair(lse, idx, nvalid_p, lmin, n_rb, b, part);
        return;
    }
    label_map_block(labels, idx, nvalid_p, inv_perm, V, cbp, lab, tpos, b - n_lse);
}

// The tile list (workgroups [0, n_list), one wave per vocabulary tile) and
// the label-only blocks of static columns (the rest, 256 tokens each), one
// launch after the plan.
__global__ __launch_bounds__(256) void k_bwd_lists(const uint8_t *__restrict__ tneed, int n_rt, int n_vt,
                                                   const int32_t *__restrict__ act, const uint8_t *__restrict__ lab,
                                                   int cbp, const int32_t *__restrict__ cpre, int CB,
                                                   int32_t *__restrict__ tlist, int64_t n_list,
                                                   const int64_t *__restrict__ labels,
                                                   const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ nvalid_p,
                                                   const int32_t *__restrict__ inv_perm, int64_t V,
                                                   const float *__restrict__ lse, const float *__restrict__ dloss,
                                                   const float *__restrict__ zlab, uint8_t *__restrict__ st,
                                                   float *__restrict__ glab) {
    const int64_t b = blockIdx.x;
    if (b < n_list) {  // (uniform)
        tile_list_block(tneed, n_rt, n_vt, act, lab, cbp, cpre, CB, tlist, b);
        return;
    }
    label_static_block(labels, idx, nvalid_p, inv_perm, V, cbp, cpre, lse, dloss, zlab, st, glab, b - n_list);
}

// The label entries of each hot column (see k_plan): the valid tokens t
// whose label falls in column hcol[h], grouped by vocabulary row with a
// stable counting sort (token order within a row): row r's entries are
// hent_t[hent[h] + hrlo[129 h + r] .. hent[h] + hrlo[129 h + r + 1]).  Two
// launches over (token slice, hot column) workgroups: k_hot_count counts
// each slice's entries per row (order-free LDS atomics); k_hot_place sums
// the counts of the earlier slices, and places the slice's entries in token
// order, the positions from wave ballots per chunk of 1024 tokens, the
// earlier waves' counts and a running count per row.
__global__ __launch_bounds__(1024) void k_hot_count(const int32_t *__restrict__ nhot_p,
                                                    const int32_t *__restrict__ hcol,
                                                    const int32_t *__restrict__ nvalid_p,
                                                    const int32_t *__restrict__ tpos, int slice,
                                                    int32_t *__restrict__ hcnt) {
    __shared__ int cnt[kBlockVocab];
    const int s = blockIdx.x, h = blockIdx.y, S = gridDim.x;
    if (h >= *nhot_p) return;  // (uniform)
    const int cb = hcol[h], nv = *nvalid_p;
    const int t = threadIdx.x;
    if (t < kBlockVocab) cnt[t] = 0;
    __syncthreads();
    for (int tok = s * slice + t; tok < min(nv, (s + 1) * slice); tok += 1024) {
        const int pos = tpos[tok];
        if (pos >= 0 && pos / kBlockVocab == cb) atomicAdd(&cnt[pos % kBlockVocab], 1);
    }
    __syncthreads();
    if (t < kBlockVocab) hcnt[((int64_t)h * S + s) * kBlockVocab + t] = cnt[t];
}

__global__ __launch_bounds__(1024) void k_hot_place(const int32_t *__restrict__ nhot_p,
                                                    const int32_t *__restrict__ hcol,
                                                    const int32_t *__restrict__ hent,
                                                    const int32_t *__restrict__ nvalid_p,
                                                    const int32_t *__restrict__ tpos, int slice,
                                                    const int32_t *__restrict__ hcnt, int32_t *__restrict__ hrlo,
                                                    int32_t *__restrict__ hent_t) {
    __shared__ int run[kBlockVocab];        // the next position of each row
    __shared__ int wrow[16][kBlockVocab];   // entries of each row per wave of a chunk
    __shared__ int part[2];
    const int s = blockIdx.x, h = blockIdx.y, S = gridDim.x;
    if (h >= *nhot_p) return;  // (uniform)
    const int cb = hcol[h], nv = *nvalid_p;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int32_t *out = hent_t + hent[h];
    // row starts: an exclusive scan of the rows' totals (two waves); this
    // slice starts each row after the earlier slices' entries of the row
    int tot = 0, before = 0;
    if (t < kBlockVocab) {
        const int32_t *c = hcnt + (int64_t)h * S * kBlockVocab + t;
        for (int q = 0; q < S; ++q) {
            const int v = c[(int64_t)q * kBlockVocab];
            tot += v;
            before += q < s ? v : 0;
        }
        int x = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) part[wave] = x;
        run[t] = x - tot;  // (exclusive within the wave; the first wave's total is added below)
    }
    __syncthreads();
    if (t < kBlockVocab) {
        if (t >= 64) run[t] += part[0];
        if (s == 0) {
            hrlo[129 * h + t] = run[t];
            if (t == kBlockVocab - 1) hrlo[129 * h + kBlockVocab] = part[0] + part[1];
        }
        run[t] += before;
    }
    __syncthreads();
    const int end = min(nv, (s + 1) * slice);
    for (int c0 = s * slice; c0 < end; c0 += 1024) {  // (uniform)
        const int tok = c0 + t;
        const int pos = tok < end ? tpos[tok] : -1;
        const int r = (pos >= 0 && pos / kBlockVocab == cb) ? pos % kBlockVocab : -1;
        // lanes of this wave with the same row: rank among them in token order
        uint64_t same = __ballot(r >= 0);
#pragma unroll
        for (int b = 0; b < 7; ++b) {
            const bool bit = (r >> b) & 1;
            const uint64_t bal = __ballot(bit);
            same &= bit ? bal : ~bal;
        }
        for (int q = t; q < 16 * kBlockVocab; q += 1024) (&wrow[0][0])[q] = 0;
        __syncthreads();
        const int rank = __popcll(same & below);
        if (r >= 0 && rank == 0) wrow[wave][r] = __popcll(same);
        __syncthreads();
        if (r >= 0) {
            int p = run[r] + rank;
            for (int w = 0; w < wave; ++w) p += wrow[w][r];
            out[p] = tok;
        }
        __syncthreads();
        if (t < kBlockVocab) {
            int c = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w) c += wrow[w][t];
            run[t] += c;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------- recompute + G
// Epilogue of a listed tile.  In the blocks of qmask acc holds the
// recomputed logits and p = exp(z - lse) decides each 128 x 128 block's
// status (1 = some p >= eps other than at a label entry, 2 = none but a
// label in it, 0 = dropped); the other blocks (left out by the bound; acc is
// not read) only have labels to decide.  A label entry's p comes from the
// recompute or, in a block not recomputed, from the forward's label logit
// (the same bits).  Kept blocks take a store slot and their gradient
// g = dloss (p [status 1 or label entry] - [v == y]) is written to
// Gt[slot][v][row] (read by dE) and, for status 1, to Gn[slot][row][v] (read
// by dH); a label-only block records its label entries' g (fp32) in glab by
// row instead.  With full_de every real block is kept for dE: Gt holds the
// unfiltered dloss (p - [v == y]) and a block the filter drops gets status 3
// (dE only).
template <typename T, class TL, bool SOFTMAX>
__device__ __forceinline__ void g_epilogue(f32x16 (&acc)[TL::TM][TL::TN], int tok0, int nv, int p0,
                                           int V, int rt, int vt, int cbp, float eps,
                                           const int32_t *__restrict__ idx, const int32_t *__restrict__ inv_perm,
                                           const int64_t *__restrict__ labels, const float *__restrict__ lse,
                                           const float *__restrict__ dloss, const float *__restrict__ zlab,
                                           float *__restrict__ glab, T *__restrict__ Gt, T *__restrict__ Gn,
                                           int64_t cap, int32_t *__restrict__ counter, uint8_t *__restrict__ st,
                                           int32_t *__restrict__ slotm, int64_t *__restrict__ stats, int *qflag,
                                           int *qstat, int *qslot, int full_de, int qmask, int fine,
                                           uint16_t *__restrict__ smask, const int32_t *__restrict__ cpre, int CB) {
    // qflag[0..3]: per block, bit 0 = some non-label p >= eps, bit 1 = a label
    // entry; qflag[4..7]: the 32 x 32 sub-tiles (bit 4 i + j: vocabulary
    // rows 32 i.., tokens 32 j.. of the block) with a non-label p >= eps;
    // qflag[8..11]: the sub-tiles holding a label entry.
    const int tid = opaque_tid();  // fresh per tile: see tile_row
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % TL::WM, wn = wave / TL::WM;
    const int th = (wn * TL::kWaveN) / kBlockRows;  // token half of this wave
    const int quad = wm * 2 + th;                   // this wave's block: vocabulary half wm, token half th
    // Per token column: lse (+inf past the valid tokens, so that p = 0 there),
    // dloss (0 there, so that g = 0), the label's row as acc_row_const in
    // this lane (-1000: none) and the label entry's softmax probability.
    float lse_t[TL::TN], dl_t[TL::TN], pl_t[TL::TN];
    int lab_t[TL::TN], lsub[TL::TN];  // lsub: 32-row group of the label within this wave's rows (-1: none)
    bool any_live = false, any_label = false;
    const int rbase = wm * TL::kWaveM + 4 * (lane >> 5);  // tile_row = rbase + acc_row_const
    const bool wsoft = SOFTMAX && ((qmask >> quad) & 1);  // this wave's block was recomputed (wave-uniform)
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int tok = tok0 + tile_col<TL>(tn, tid);
        lse_t[tn] = __builtin_huge_valf();
        dl_t[tn] = 0.f;
        pl_t[tn] = 0.f;
        lab_t[tn] = -1000;
        lsub[tn] = -1;
        if (tok < nv) {
            const int64_t row = idx[tok];
            lse_t[tn] = lse[row];
            dl_t[tn] = dloss[row];
            const int64_t y = labels[row];
            const bool y_ok = y >= 0 && y < V;  // other labels are undefined by contract
            const int ypos = y_ok ? (inv_perm ? inv_perm[y] : (int)y) : -(1 << 30);
            const int lr = ypos - p0 - wm * TL::kWaveM;  // row within this wave's 128 vocabulary rows
            const bool here = lr >= 0 && lr < TL::kWaveM;
            lab_t[tn] = here ? ypos - p0 - rbase : -1000;
            lsub[tn] = here ? lr / 32 : -1;
            any_label |= here;
            // the label entry's own softmax probability where the block was
            // not recomputed: from the forward's label logit, the same bits
            // as the recompute (same MFMA code and K order) and the same formula
            if (here && !wsoft) pl_t[tn] = __builtin_amdgcn_exp2f((zlab[row] - lse_t[tn]) * kLog2e);
        }
    }
    const int vlim = row_limit<TL>(V - p0, tid);  // entry (tm, r) is a real vocabulary row iff acc_row_const < vlim
    // This wave's sub-tile (tm, tn) is sub-tile 4 tm + jw + tn of its block.
    static_assert(TL::kWaveM == kBlockVocab && TL::TM == 4 && TL::TN == 2 && TL::kWaveN == 64,
                  "a wave holds 4 x 2 sub-tiles of 32 x 32 of one block");
    const int jw = 2 * (wn & 1);
    uint32_t sub_live = 0;  // this wave's sub-tiles with a non-label p >= eps (block bit numbering)
    if (wsoft) {
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            // past the valid tokens p = 0, which eps = 0 would count as kept:
            // a block with no valid token (recomputed by the VGPR-staged path,
            // which computes every block) must stay dropped, since the pass
            // plan only counts blocks that hold one
            const bool tv = lse_t[tn] != __builtin_huge_valf();
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm) {
                bool live = false;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool ok = acc_row_const(tm, r) < vlim;
                    const float p = ok ? __builtin_amdgcn_exp2f((acc[tm][tn][r] - lse_t[tn]) * kLog2e) : 0.f;
                    acc[tm][tn][r] = p;
                    // the filter looks at the entries other than the label one
                    live |= (p >= eps) && ok && tv && acc_row_const(tm, r) != lab_t[tn];
                }
                any_live |= live;
                if (__ballot(live)) sub_live |= 1u << (4 * tm + jw + tn);
            }
        }
    }
    uint32_t sub_lab = 0;  // this wave's sub-tiles holding a label entry
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
            if (__ballot(lsub[tn] == tm)) sub_lab |= 1u << (4 * tm + jw + tn);
    const uint64_t bl = __ballot(any_live), bb = __ballot(any_label);
    if (lane == 0 && (bl | bb)) {
        atomicOr(&qflag[quad], (bl ? 1 : 0) | (bb ? 2 : 0));
        atomicOr(&qflag[4 + quad], (int)sub_live);
        atomicOr(&qflag[8 + quad], (int)sub_lab);
    }
    __syncthreads();
    if (tid < 4) {
        const int f = qflag[tid];
        int sv = (f & 1) ? 1 : ((f & 2) ? 2 : 0);
        const int rb = 2 * rt + (tid & 1), cb = 2 * vt + (tid >> 1);
        // full dE: a real block the filter drops is still kept for dE
        if (full_de && sv == 0 && rb * kBlockRows < nv && (int64_t)cb * kBlockVocab < V) sv = 3;
        int s = -1;
        if (sv) {
            s = atomicAdd(counter, 1);
            if (s >= cap) {
                // the plan sizes every pass to fit the store, so this only
                // happens when it is told to (CCE_BWD_DEBUG_STORE_LIMIT):
                // the block is dropped and counted, never written past the store
                s = -1;
                sv = 0;
                if (stats) atomicAdd(reinterpret_cast<unsigned long long *>(stats + 5), 1ull);
            }
        }
        qstat[tid] = sv;
        qslot[tid] = s;
        st[(int64_t)rb * cbp + cb] = (uint8_t)sv;
        if (sv) {
            slotm[(int64_t)rb * cbp + cb] = s;
            // sub-tiles whose stored gradient may be nonzero: with the fine
            // filter those with a kept softmax part or a label entry; a
            // label-only block only its label sub-tiles; otherwise all
            const int live16 = qflag[4 + tid], lab16 = qflag[8 + tid];
            smask[(int64_t)rb * cbp + cb] =
                (uint16_t)(sv == 1 ? (fine ? (live16 | lab16) : 0xFFFF) : (sv == 2 ? lab16 : 0xFFFF));
        }
        if (stats) {
            // (the label-only blocks of static columns are counted by k_plan)
            const bool col_static = cb < CB && cpre[cb + 1] - cpre[cb] == 1;
            if (sv == 1 || (sv == 2 && !col_static))
                atomicAdd(reinterpret_cast<unsigned long long *>(stats + (sv == 1 ? 0 : 1)), 1ull);
            // 32 x 32 sub-tiles whose softmax part is kept (all 16 of a kept block without the fine filter)
            if (sv == 1)
                atomicAdd(reinterpret_cast<unsigned long long *>(stats + 6),
                          (unsigned long long)(fine ? __popc((unsigned)qflag[4 + tid]) : 16));
            // blocks whose logits were recomputed (real rows and vocabulary entries only)
            if (SOFTMAX && ((qmask >> tid) & 1) && rb * kBlockRows < nv && (int64_t)cb * kBlockVocab < V)
                atomicAdd(reinterpret_cast<unsigned long long *>(stats + 4), 1ull);
        }
    }
    __syncthreads();
    const int status = qstat[quad];
    if (status == 0) return;  // wave-uniform
    const bool glab_only = status == 2;
    // the block's sub-tiles that keep their softmax part (all of a kept
    // block without the fine filter)
    const uint32_t keep16 = fine ? (uint32_t)qflag[4 + quad] : 0xFFFFu;
    T *gt = Gt + (int64_t)qslot[quad] * kBlockElems;
    T *gn = Gn + (int64_t)qslot[quad] * kBlockElems;

#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int tl = tile_col<TL>(tn, tid) - th * kBlockRows;  // token within the block
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                T g4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = r4 * 4 + q;
                    const int rl = tile_row<TL>(tm, r, tid);
                    const bool ok = acc_row_const(tm, r) < vlim && dl_t[tn] != 0.f;
                    const bool il = acc_row_const(tm, r) == lab_t[tn];
                    const float onehot = il ? 1.f : 0.f;
                    // the label entry keeps its exact softmax part; the others only in a kept block
                    // (sub-tile)
                    const bool subk = (keep16 >> (4 * tm + jw + tn)) & 1;
                    const float pk = il ? (wsoft ? acc[tm][tn][r] : pl_t[tn])
                                        : ((wsoft && status == 1 && subk) ? acc[tm][tn][r] : 0.f);
                    const float g = ok ? dl_t[tn] * (pk - onehot) : 0.f;
                    g4[q] = from_f32<T>(g);
                    // full dE: the vocabulary-major copy (read by dE) holds the unfiltered gradient
                    const float gf = (wsoft && full_de && ok) ? dl_t[tn] * (acc[tm][tn][r] - onehot) : g;
                    gt[(rl - wm * kBlockVocab) * kBlockRows + tl] = from_f32<T>(gf);
                    // label-only block: dH takes the label entry's gradient (fp32) from glab
                    if (glab_only && il && ok) glab[tok0 + tile_col<TL>(tn, tid)] = g;
                }
                // rows r4*4 .. r4*4+3 are consecutive vocabulary entries (dH reads these; only for status 1)
                if (status == 1) {
                    T *dst = gn + tl * kBlockVocab + tile_row<TL>(tm, r4 * 4, tid) - wm * kBlockVocab;
#pragma unroll
                    for (int q = 0; q < 4; ++q) dst[q] = g4[q];
                }
            }
    }
}

// Recompute of logit tile (rt, vt) on the DMA pipeline (needs
// D * sizeof(T) % kLogitRowBytes == 0): the forward's engine, tile shape and
// K order.  Rows past the end of an operand are clamped to a valid row: their
// logits are finite and the epilogue masks them.
// Only the blocks in qmask (bit 2 (vocabulary half) + token half) are
// computed: the halves of A and B no such block uses are not loaded and the
// waves of the other blocks skip their MFMAs.
template <typename T, class TL>
__device__ __forceinline__ void recompute_dma(const T *__restrict__ H, Rows2<const T> E,
                                              const int32_t *__restrict__ idx, int nv,
                                              const int32_t *__restrict__ perm, int D, int V, int tok0, int p0,
                                              int qmask, u32x4 *lds, f32x16 (&acc)[TL::TM][TL::TN]) {
    using DE = DmaEngine<T, TL, kLogitRowBytes, kLogitStages>;
    const size_t rowb = (size_t)D * sizeof(T);
    const int ns = D * (int)sizeof(T) / DE::kStageBytes;
    const int tid = opaque_tid();  // per-tile address arithmetic stays in this tile's code
    DE eng(lds);
#pragma unroll
    for (int j = 0; j < DE::NIA; ++j) {
        const int r = DE::row_a(j, tid);
        const int pos = min(p0 + r, V - 1);
        int vid = perm ? perm[pos] : pos;
        vid = (vid >= 0 && vid < V) ? vid : 0;
        eng.pa[j] = reinterpret_cast<const char *>(E.row(vid)) + DE::chunk_off(j, r, tid);
    }
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j, tid);
        const int tok = min(tok0 + r, nv - 1);
        eng.pb[j] = reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb + DE::chunk_off(j, r, tid);
    }
    static_assert(TL::kWaveM == TL::BM / 2 && TL::BN / TL::WN * 2 <= TL::BN, "a wave lies in one block");
    const int halves = ((qmask & 3) ? 1 : 0) | ((qmask & 12) ? 2 : 0)    // vocabulary halves
                       | ((qmask & 5) ? 4 : 0) | ((qmask & 10) ? 8 : 0);  // token halves
    const int wave = tid >> 6;
    const int quad = (wave % TL::WM) * 2 + (wave / TL::WM) * TL::kWaveN / (TL::BN / 2);
    const bool active = (qmask >> quad) & 1;  // wave-uniform
#pragma unroll
    for (int q = 0; q < DE::kDepth; ++q)
        if (q < ns) eng.issue_halves(q, q * DE::kStageBytes, halves);
    for (int s = 0; s < ns; ++s) {
        const int ahead = ns - 1 - s;
        eng.wait_stage(eng.clamp_ahead(ahead));
        // as in the forward: the first K-slice's MFMAs before the next DMA
        if (active) eng.compute(s % DE::kStages, acc, tid, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (s + DE::kDepth < ns)
            eng.issue_halves((s + DE::kDepth) % DE::kStages, (s + DE::kDepth) * DE::kStageBytes, halves);
        __builtin_amdgcn_sched_barrier(0);
        if (active) eng.compute(s % DE::kStages, acc, tid, 1, DE::kCpr / 2);
    }
}

// The same on the VGPR-staged engine (any D % 8 == 0), as the forward's
// fallback kernel computes it.
template <typename T, class TL>
__device__ __forceinline__ void recompute_vgpr(const T *__restrict__ H, Rows2<const T> E,
                                               const int32_t *__restrict__ idx, int nv,
                                               const int32_t *__restrict__ perm, int D, int V, int tok0, int p0,
                                               u32x4 *lds, f32x16 (&acc)[TL::TM][TL::TN]) {
    const size_t rowb = (size_t)D * sizeof(T);
    const int kvalid = D * (int)sizeof(T);
    const int ns = (kvalid + TL::kStageBytes - 1) / TL::kStageBytes;
    Engine<T, TL> eng;
#pragma unroll
    for (int j = 0; j < Engine<T, TL>::NA; ++j) {
        const int pos = p0 + eng.row(j);
        const int vid = pos < V ? (perm ? perm[pos] : pos) : -1;
        eng.pa[j] = (vid >= 0 && vid < V) ? reinterpret_cast<const char *>(E.row(vid)) : nullptr;
    }
#pragma unroll
    for (int j = 0; j < Engine<T, TL>::NB; ++j) {
        const int tok = tok0 + eng.row(j);
        eng.pb[j] = tok < nv ? reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb : nullptr;
    }
    eng.load(0, kvalid);
    eng.store(lds);
    __syncthreads();
    for (int s = 0; s < ns; ++s) {
        const bool more = s + 1 < ns;
        if (more) eng.load((s + 1) * TL::kStageBytes, kvalid);
        eng.compute(lds + (s & 1) * TL::kStage, acc);
        if (more) eng.store(lds + ((s + 1) & 1) * TL::kStage);
        __syncthreads();
    }
}

template <typename T, bool DMA>
struct GPassLds {
    static constexpr int value = DMA ? DmaEngine<T, TileFD, kLogitRowBytes, kLogitStages>::kLdsChunks
                                     : TileF::kLdsChunks;
};

// Recompute phase of pass p on workgroups bid = 0 .. nbid - 1, which take
// the pass's listed tiles from work queues.  Workgroup b runs on XCD b % 8;
// with a grid that is a multiple of 8 the list is cut into 8 contiguous
// parts and workgroup b starts on part b % 8 (tiles that share a vocabulary
// tile are adjacent in the list, so they share that XCD's L2), then helps
// with the other parts.
template <typename T, bool DMA>
__device__ __forceinline__ void g_phase(const BwdArgs<T> &a, int p, int bid, int nbid, u32x4 *lds, int *qflag,
                                        int *qstat, int *qslot, int *ticket) {
    using TL = TileF;
    const PlanView pv = plan_view(a.plan, a.max_passes);
    int32_t *queues = plan_queues(a.plan, a.max_passes, p);
    const int nv = *a.nvalid;
    const int lb = pv.list_begin[p], le = pv.list_begin[p + 1];
    const int nparts = nbid % 8 == 0 ? 8 : 1;
    for (int k = 0; k < nparts; ++k) {
        const int part = (bid + k) % nparts;
        const int pb = lb + (int)((int64_t)(le - lb) * part / nparts);
        const int pe = lb + (int)((int64_t)(le - lb) * (part + 1) / nparts);
        if (pe == pb) continue;  // (uniform) an empty part takes no ticket
        for (;;) {
            const int i = pb + take_ticket(queues + part, ticket);
            if (i >= pe) break;
            const int tile = a.tlist[i];
            if (tile < 0) continue;  // a tile left to label_static_block
            const int vt = tile / a.n_rt, rt = tile % a.n_rt;
            const int tn8 = a.tneed[tile];
            const bool rec = (tn8 & 0x80) != 0;
            const int qmask = DMA ? (tn8 >> 3) & 15 : 15;  // the VGPR-staged recompute computes every block
            const int tok0 = rt * TL::BN, p0 = vt * TL::BM;
            if (threadIdx.x < 12) qflag[threadIdx.x] = 0;
            __syncthreads();
            f32x16 acc[TL::TM][TL::TN];
            if (rec) {
                zero_acc<TL>(acc);
                if constexpr (DMA) recompute_dma<T, TL>(a.H, a.E, a.idx, nv, a.perm, a.D, a.V, tok0, p0, qmask, lds, acc);
                else recompute_vgpr<T, TL>(a.H, a.E, a.idx, nv, a.perm, a.D, a.V, tok0, p0, lds, acc);
                __syncthreads();
                g_epilogue<T, TL, true>(acc, tok0, nv, p0, a.V, rt, vt, a.cbp, a.eps, a.idx, a.inv_perm, a.labels,
                                        a.lse, a.dloss, a.zlab, a.glab, a.Gt, a.Gn, a.cap_take, pv.counter + p, a.st, a.slot, a.stats,
                                        qflag, qstat, qslot, a.full_de, qmask, a.fine, a.smask, a.cpre, a.CB);
            } else {
                g_epilogue<T, TL, false>(acc, tok0, nv, p0, a.V, rt, vt, a.cbp, a.eps, a.idx, a.inv_perm, a.labels,
                                         a.lse, a.dloss, a.zlab, a.glab, a.Gt, a.Gn, a.cap_take, pv.counter + p, a.st, a.slot, a.stats,
                                         qflag, qstat, qslot, a.full_de, 0, a.fine, a.smask, a.cpre, a.CB);
            }
        }
    }
}

// ------------------------------------------------------------------- dH
// dH rows of a 128-token block, 256 features: C[row][d] = sum_v G[row][v]
// E[v][d], K = the vocabulary entries of the kept blocks.  A = the stored
// block Gn[slot] (rows x v, v contiguous) through the usual 64-byte LDS rows.
// B = E rows, v-major with d contiguous, copied as they are into LDS and read
// transposed: bf16 with ds_read_b64_tr_b16, which gives each lane 4
// consecutive rows at one column (two of them make the 8 K values of the
// 32x32x16 MFMA operand); fp32 needs one value per lane per MFMA and reads it
// directly.  B rows are kRowB bytes with chunk c of row r stored at
// c ^ 4 (r & 3), so the 4 rows one transposed read touches are 64 bytes apart
// in the bank space.
template <typename T, bool kWide = false>
struct DhEngine {
    using TL = TileG;
    // vocabulary entries per stage: 64 bytes of a stored block row, or 128
    // bytes (kWide: half the stages, one in flight, in the same LDS)
    static constexpr int kKv = (sizeof(T) == 2 ? 32 : 16) * (kWide ? 2 : 1);
    static constexpr int kSpb = kBlockVocab / kKv;        // stages per block
    static constexpr int kStages = kWide ? 2 : 4, kDepth = kStages - 1;
    static constexpr int kStageBytes = kKv * (int)sizeof(T);  // A row bytes per stage
    static constexpr int kCprA = kStageBytes / 16;            // A chunks per row
    static constexpr int kSlices = kKv / (sizeof(T) == 2 ? 16 : 8);  // MFMA K-slices per stage
    static constexpr int kStageA = TL::BM * kCprA;        // chunks
    static constexpr int kRowB = TL::BN * (int)sizeof(T); // bytes of one B row (256 features)
    static constexpr int kCprB = kRowB / 16;
    static constexpr int kStageB = kKv * kCprB;
    static constexpr int kStage = kStageA + kStageB;
    static constexpr int kLdsChunks = kStages * kStage;
    static constexpr int NIA = kStageA / 64 / TL::kWaves;
    static constexpr int NIB = kStageB / 64 / TL::kWaves;
    static constexpr int NI = NIA + NIB;
    static_assert(NIA * 64 * TL::kWaves == kStageA && NIB * 64 * TL::kWaves == kStageB, "stage split");

    u32x4 *lds;
    uint32_t lds0;      // LDS byte address of the stages (wave-uniform)
    int a_off[NIA];     // this lane's A source offsets within a stored block (row + swizzled chunk)
    int b_row[NIB];     // B row (vocabulary entry within the stage) this lane feeds
    int b_off[NIB];     // byte offset of its chunk within an E row (clamped to the last chunk < D)

    __device__ __forceinline__ DhEngine(u32x4 *l, int d0, int D, int tid) : lds(l), lds0(lds_addr(l)) {
        const int w = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int j = 0; j < NIA; ++j) {
            const int sa = 64 * (j * TL::kWaves + w) + lane;
            const int ra = sa / kCprA;
            a_off[j] = ra * kBlockVocab * (int)sizeof(T) + 16 * ((sa % kCprA) ^ dma_swz<kStageBytes>(ra));
        }
        constexpr int kElemsPerChunk = 16 / (int)sizeof(T);
#pragma unroll
        for (int j = 0; j < NIB; ++j) {
            const int sb = 64 * (j * TL::kWaves + w) + lane;
            const int r = sb / kCprB, cs = sb % kCprB;
            const int lc = cs ^ (4 * (r & 3));
            b_row[j] = r;
            b_off[j] = min(d0 + lc * kElemsPerChunk, D - kElemsPerChunk) * (int)sizeof(T);
        }
    }

    // Stage kq of the block with store slot `slot` and first vocabulary
    // position pos0, into LDS buffer buf.
    // The lanes of B instruction j feed kRowsPerInstr consecutive rows, the
    // first of them wave-uniform; with a permutation their ids are read with
    // scalar loads, so that no vector load has to be waited for while the
    // earlier stages are in flight.
    static constexpr int kRowsPerInstr = 64 / kCprB;
    static_assert(kRowsPerInstr == 1 || kRowsPerInstr == 2, "B rows per instruction");

    __device__ __forceinline__ void issue(int buf, const T *Gn, int64_t slot, const Rows2<const T> &E,
                                          const int32_t *perm, int pos0, int kq, int V) const {
        const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t st = lds0 + (uint32_t)(buf * kStage) * 16u;
#pragma unroll
        for (int j = 0; j < NIA; ++j)
            dma16_at(reinterpret_cast<const char *>(Gn + slot * kBlockElems) + a_off[j] + kq * kStageBytes,
                     st + 1024u * (j * TL::kWaves + w));
        const int base = __builtin_amdgcn_readfirstlane(pos0 + kq * kKv);
#pragma unroll
        for (int j = 0; j < NIB; ++j) {
            int vid;
            if (perm) {
                const int p0 = base + (int)(64 * (j * TL::kWaves + w)) / kCprB;  // uniform
                const int v0 = uniform_load(perm, min(p0, V - 1));
                const int v1 = kRowsPerInstr > 1 ? uniform_load(perm, min(p0 + 1, V - 1)) : v0;
                vid = b_row[j] == p0 - base ? v0 : v1;
            } else {
                const int pos = base + b_row[j];
                vid = pos < V ? pos : V - 1;
            }
            vid = (vid >= 0 && vid < V) ? vid : 0;
            dma16_at(reinterpret_cast<const char *>(E.row(vid)) + b_off[j],
                     st + 16u * kStageA + 1024u * (j * TL::kWaves + w));
        }
    }

    __device__ __forceinline__ void wait_stage(int ahead) const {
        if constexpr (kDepth >= 3) {
            if (ahead >= 2) { wait_vmcnt<2 * NI>(); block_sync(); return; }
        }
        if constexpr (kDepth >= 2) {
            if (ahead >= 1) { wait_vmcnt<NI>(); block_sync(); return; }
        }
        wait_vmcnt<0>();
        block_sync();
    }
    __device__ __forceinline__ int clamp_ahead(int ahead) const { return ahead < kDepth - 1 ? ahead : kDepth - 1; }

    __device__ __forceinline__ void compute(int buf, f32x16 (&acc)[TL::TM][TL::TN], int tid,
                                           uint32_t rows = (1u << TL::TM) - 1) const {
        const int lane = tid & 63, wave = tid >> 6;
        const int ra0 = (wave % TL::WM) * TL::kWaveM + (lane & 31);
        const int nb0 = (wave / TL::WM) * TL::kWaveN;
        const u32x4 *A = lds + buf * kStage;
        const char *Bb = reinterpret_cast<const char *>(A + kStageA);
#pragma unroll
        for (int kk = 0; kk < kSlices; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            u32x4 fa[TL::TM], fb[TL::TN];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
                if ((rows >> tm) & 1) fa[tm] = A[dma_slot<kStageBytes>(ra0 + tm * 32, c)];
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int n0 = nb0 + tn * 32;
                if constexpr (sizeof(T) == 2) {
                    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
                    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
                    bf16x4 h[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int row = 16 * kk + 8 * (lane >> 5) + 4 * t + ((lane & 15) >> 2);
                        const int col = n0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
                        const char *a = Bb + row * kRowB + (((col >> 3) ^ (4 * (row & 3))) << 4) + (col & 7) * 2;
                        h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(a));
                    }
                    const u32x2 lo = __builtin_bit_cast(u32x2, h[0]), hi = __builtin_bit_cast(u32x2, h[1]);
                    fb[tn] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    const int col = n0 + (lane & 31);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = 8 * kk + 4 * (lane >> 5) + j;
                        fb[tn][j] = *reinterpret_cast<const uint32_t *>(
                            Bb + row * kRowB + (((col >> 2) ^ (4 * (row & 3))) << 4) + (col & 3) * 4);
                    }
                }
            }
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
                if ((rows >> tm) & 1)
#pragma unroll
                    for (int tn = 0; tn < TL::TN; ++tn) Mfma<T>::step(fa[tm], fb[tn], acc[tm][tn]);
        }
    }
};

// ------------------------------------------------------------- dE (Kahan)
// Shared memory of the gradient-product kernel: the K pipeline's stages,
// reused after the K loop for the output tile, and the block lists.
template <typename T>
struct GradLds {
    static constexpr int kStageChunks = DmaEngine<T, TileG>::kLdsChunks > DhEngine<T>::kLdsChunks
                                            ? DmaEngine<T, TileG>::kLdsChunks
                                            : DhEngine<T>::kLdsChunks;
    static_assert(DhEngine<T, true>::kLdsChunks <= kStageChunks, "wide dH stages fit the stage buffer");
    u32x4 stages[kStageChunks];
    int list[kListCap];
    int lslot[kListCap];
    int wcnt[TileG::kWaves];
    int soft;  // the vocabulary block has a block with a kept softmax part (status 1 or 3)
    // with the fine filter: sub-tile masks of the listed blocks and their listed K stages
    int lmask[kListCap];
    int stl[kListCap * 8];
    // label entries of a vocabulary block (label path), grouped by vocabulary
    // row, in token order within a row
    int ent_h[kLabelEntries];                           // row of H
    float ent_g[kLabelEntries];                         // gradient of the label entry (fp32)
    int tmp_r[kLabelEntries], tmp_h[kLabelEntries];     // the entries in token order, before grouping
    float tmp_g[kLabelEntries];
    int rlo[kBlockVocab + 1];                           // entries of row r: [rlo[r], rlo[r + 1])
    int wrow[TileG::kWaves][kBlockVocab];               // entries of each row per wave
};

// What the label path reads (null labels: no label path).
template <typename T>
struct LabelCols {
    const int64_t *labels;
    const int32_t *idx;
    const int32_t *inv_perm;
    const float *glab;
    const T *H;
    int nv;
    const int32_t *cent;  // label entries per vocabulary block
    // hot columns (k_plan, k_hot_count, k_hot_place): index per column (-1: not hot),
    // first entry, row ranges and the entries (valid-token positions)
    const int32_t *hidx, *hent, *hrlo, *hent_t;
};

// The label entries of vocabulary block cb when every kept block of cb is
// label-only: the valid tokens i of the n kept row blocks sh.list[0 .. n)
// whose label falls in cb (at most kLabelEntries of them), grouped by
// vocabulary row: row r's entries are [sh.rlo[r], sh.rlo[r + 1]) in token
// order, with the row of H (sh.ent_h) and the entry's fp32 gradient g_i
// (sh.ent_g).  The candidates are read 512 at a time and compacted in token
// order; the compacted entries (one per thread) are then grouped with a
// stable counting sort (ranks from wave ballots, as in a radix sort's
// scatter).
template <typename T>
__device__ __forceinline__ void label_group(GradLds<T> &sh, int n, int cb, const LabelCols<T> &lc, int V) {
    constexpr int kThreads = TileG::kThreads;
    static_assert(kThreads == kLabelEntries, "one compacted entry per thread");
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int m = 0;  // entries compacted so far (uniform)
    for (int c0 = 0; c0 < n * kBlockRows; c0 += kThreads) {
        // candidate c: token (sh.list[c / 128] * 128 + c % 128) of a label block
        const int c = c0 + t;
        int row = -1, hrow = 0;
        float g = 0.f;
        if (c < n * kBlockRows) {
            const int tok = sh.list[c / kBlockRows] * kBlockRows + (c % kBlockRows);
            if (tok < lc.nv) {
                const int r = lc.idx[tok];
                const int64_t y = lc.labels[r];
                if (y >= 0 && y < V) {
                    const int pos = lc.inv_perm ? lc.inv_perm[y] : (int)y;
                    if (pos / kBlockVocab == cb) {
                        row = pos % kBlockVocab;
                        hrow = r;
                        g = lc.glab[tok];
                    }
                }
            }
        }
        const uint64_t bal = __ballot(row >= 0);
        if (lane == 0) sh.wcnt[wave] = __popcll(bal);
        __syncthreads();
        int base = m, total = 0;
#pragma unroll
        for (int w = 0; w < TileG::kWaves; ++w) {
            base += w < wave ? sh.wcnt[w] : 0;
            total += sh.wcnt[w];
        }
        if (row >= 0) {
            const int q = base + __popcll(bal & below);
            if (q < kLabelEntries) {  // (callers keep the entries within kLabelEntries)
                sh.tmp_r[q] = row;
                sh.tmp_h[q] = hrow;
                sh.tmp_g[q] = g;
            }
        }
        m += total;
        __syncthreads();  // wcnt is rewritten by the next chunk; tmp_* are read below
    }
    m = min(m, kLabelEntries);
    int row = -1, hrow = 0;
    float g = 0.f;
    if (t < m) {
        row = sh.tmp_r[t];
        hrow = sh.tmp_h[t];
        g = sh.tmp_g[t];
    }
    // lanes of this wave with the same row: their rank among them is the rank in token order
    uint64_t same = __ballot(row >= 0);
#pragma unroll
    for (int b = 0; b < 7; ++b) {
        const bool bit = (row >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & below);
    for (int q = t; q < TileG::kWaves * kBlockVocab; q += kThreads) (&sh.wrow[0][0])[q] = 0;
    __syncthreads();
    if (row >= 0 && rank == 0) sh.wrow[wave][row] = __popcll(same);
    __syncthreads();
    if (t < kBlockVocab) {  // two waves: exclusive scan of the row counts
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < TileG::kWaves; ++w) cnt += sh.wrow[w][t];
        int x = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        sh.rlo[t + 1] = x;  // inclusive within the wave
    }
    __syncthreads();
    if (t >= 64 && t < kBlockVocab) sh.rlo[t + 1] += sh.rlo[64];  // second wave: add the first wave's total
    if (t == 0) sh.rlo[0] = 0;
    __syncthreads();
    if (row >= 0) {
        int p = sh.rlo[row] + rank;
        for (int w = 0; w < wave; ++w) p += sh.wrow[w][row];
        sh.ent_h[p] = hrow;
        sh.ent_g[p] = g;
    }
    __syncthreads();
}

// dE rows of vocabulary block cb, features [d_lo, d_hi) (multiples of the
// 16-byte segment), from the grouped label entries: dE_v = sum of g_i h_i
// over row v's entries, summed in fp32 in token order, zero for a row no
// label falls in.
template <typename T>
__device__ __forceinline__ void label_rows(const GradLds<T> &sh, int cb, int d_lo, int d_hi, const LabelCols<T> &lc,
                                           const int32_t *__restrict__ perm, int D, int V, Rows2<T> dE) {
    constexpr int CE = ChunkElems<T>::value;
    const int segs = (min(d_hi, D) - d_lo + CE - 1) / CE;  // 16-byte segments per row
    if (segs <= 0) return;
    for (int q = threadIdx.x; q < kBlockVocab * segs; q += TileG::kThreads) {
        const int r = q / segs, d = d_lo + (q % segs) * CE;
        const int pos = cb * kBlockVocab + r;
        const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
        if (v < 0 || v >= V) continue;
        float acc[CE];
#pragma unroll
        for (int k = 0; k < CE; ++k) acc[k] = 0.f;
        const int e1 = sh.rlo[r + 1];
        int e = sh.rlo[r];
        for (; e + 4 <= e1; e += 4) {  // four loads in flight, added in entry order
            u32x4 hv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                hv[u] = ld16(reinterpret_cast<const char *>(lc.H + (int64_t)sh.ent_h[e + u] * D + d));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const T *hp = reinterpret_cast<const T *>(&hv[u]);
                const float ge = sh.ent_g[e + u];
#pragma unroll
                for (int k = 0; k < CE; ++k) acc[k] += ge * to_f32(hp[k]);
            }
        }
        for (; e < e1; ++e) {
            const u32x4 hv = ld16(reinterpret_cast<const char *>(lc.H + (int64_t)sh.ent_h[e] * D + d));
            const T *hp = reinterpret_cast<const T *>(&hv);
            const float ge = sh.ent_g[e];
#pragma unroll
            for (int k = 0; k < CE; ++k) acc[k] += ge * to_f32(hp[k]);
        }
        u32x4 out;
        T *op = reinterpret_cast<T *>(&out);
#pragma unroll
        for (int k = 0; k < CE; ++k) op[k] = from_f32<T>(acc[k]);
        *reinterpret_cast<u32x4 *>(dE.row(v) + d) = out;
    }
}

// dE rows of hot column cb (index h), features [kHotF f, kHotF (f + 1))
// (capped at D), from its label entries (k_hot_place: grouped by row,
// token order within a row).  A row's entries are cut into pieces of at most
// kHotPiece; a batch of kPB pieces is summed with one thread per (piece,
// 16-byte segment), each piece in token order in fp32, and each row's
// running sum then adds the batch's pieces of that row in order.  So a
// frequent label's entries are summed by many threads at once, in a fixed
// order.
constexpr int kHotPiece = 32;
template <typename T>
__device__ __forceinline__ void hot_item(GradLds<T> &sh, int h, int cb, int f, const LabelCols<T> &lc,
                                         const int32_t *__restrict__ perm, int D, int V, Rows2<T> dE) {
    constexpr int kThreads = TileG::kThreads;
    constexpr int CE = ChunkElems<T>::value;
    constexpr int kSeg = kHotF / CE;        // 16-byte segments of the item's features
    constexpr int kPB = kThreads / kSeg;    // pieces per batch
    constexpr int kBE = kPB * kHotPiece;    // entries of a batch at most
    constexpr int kCF = kHotF / 4;          // features per thread when rows add their pieces (4 threads a row)
    static_assert(kBE % kThreads == 0 && kBE / kThreads <= 8, "one round of staging loads per batch");
    static_assert(sizeof(sh.stages) >= sizeof(float) * (kBlockVocab * kHotF + kPB * kHotF + 2 * kBE + kBlockVocab + 1),
                  "the hot item's buffers fit the stage buffer");
    float *run = reinterpret_cast<float *>(sh.stages);   // [128][kHotF] running row sums
    float *part = run + kBlockVocab * kHotF;              // [kPB][kHotF] the batch's piece sums
    int *eh = reinterpret_cast<int *>(part + kPB * kHotF);  // [kBE] row of H of each entry of the batch
    float *eg = reinterpret_cast<float *>(eh + kBE);      // [kBE] its gradient
    int *ppre = reinterpret_cast<int *>(eg + kBE);        // [129] pieces before each row
    int *rlo = sh.rlo;                                    // [129] entries before each row
    const int t = threadIdx.x, lane = t & 63;
    const int d0 = kHotF * f;
    const int32_t *ent = lc.hent_t + lc.hent[h];
    if (t <= kBlockVocab) rlo[t] = lc.hrlo[129 * h + t];
    for (int q = t; q < kBlockVocab * kHotF; q += kThreads) run[q] = 0.f;
    __syncthreads();
    if (t < kBlockVocab) {  // pieces per row: exclusive scan over two waves
        const int c = (rlo[t + 1] - rlo[t] + kHotPiece - 1) / kHotPiece;
        int x = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        ppre[t + 1] = x;  // inclusive within the wave
    }
    __syncthreads();
    if (t >= 64 && t < kBlockVocab) ppre[t + 1] += ppre[64];
    if (t == 0) ppre[0] = 0;
    __syncthreads();
    const int np = ppre[kBlockVocab];
    // the row of piece p: the last r with ppre[r] <= p (rows without pieces
    // have ppre[r] == ppre[r + 1])
    auto row_of = [&](int p) {
        int lo = 0, hi = kBlockVocab;  // ppre[lo] <= p < ppre[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (ppre[mid] <= p) lo = mid;
            else hi = mid;
        }
        return lo;
    };
    auto piece_begin = [&](int p, int r) { return rlo[r] + (p - ppre[r]) * kHotPiece; };
    for (int b0 = 0; b0 < np; b0 += kPB) {
        const int b1 = min(np, b0 + kPB);
        const int rb0 = row_of(b0), rb1 = row_of(b1 - 1);
        const int e_lo = piece_begin(b0, rb0);
        const int n_be = min(piece_begin(b1 - 1, rb1) + kHotPiece, rlo[rb1 + 1]) - e_lo;
        {  // stage the batch's entries: every load of a thread in flight at once
            constexpr int kU = kBE / kThreads;
            int tok[kU], hr[kU];
            float gg[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int k = u * kThreads + t;
                tok[u] = k < n_be ? ent[e_lo + k] : -1;
            }
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (tok[u] >= 0) {
                    hr[u] = lc.idx[tok[u]];
                    gg[u] = lc.glab[tok[u]];
                }
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (tok[u] >= 0) {
                    eh[u * kThreads + t] = hr[u];
                    eg[u * kThreads + t] = gg[u];
                }
        }
        __syncthreads();
        {
            const int ps = t / kSeg, sg = t % kSeg, p = b0 + ps;
            const int d = d0 + sg * CE;
            float acc[CE];
#pragma unroll
            for (int c = 0; c < CE; ++c) acc[c] = 0.f;
            if (p < b1 && d < D) {
                const int r = row_of(p);
                const int e_begin = piece_begin(p, r) - e_lo;
                const int e_end = min(piece_begin(p, r) + kHotPiece, rlo[r + 1]) - e_lo;
                for (int e = e_begin; e < e_end; e += 16) {  // sixteen loads in flight, added in entry order
                    u32x4 hv[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        if (e + u < e_end)
                            hv[u] = ld16(reinterpret_cast<const char *>(lc.H + (int64_t)eh[e + u] * D + d));
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        if (e + u < e_end) {
                            const T *hp = reinterpret_cast<const T *>(&hv[u]);
                            const float ge = eg[e + u];
#pragma unroll
                            for (int c = 0; c < CE; ++c) acc[c] += ge * to_f32(hp[c]);
                        }
                }
            }
            if (p < b1) {
#pragma unroll
                for (int c = 0; c < CE; ++c) part[ps * kHotF + sg * CE + c] = acc[c];
            }
        }
        __syncthreads();
        {  // each row adds its pieces of the batch in order (four threads per row)
            const int r = t >> 2, c0 = kCF * (t & 3);
            const int p_lo = max(ppre[r], b0), p_hi = min(ppre[r + 1], b1);
            for (int p = p_lo; p < p_hi; ++p)
#pragma unroll
                for (int c = 0; c < kCF; ++c) run[r * kHotF + c0 + c] += part[(p - b0) * kHotF + c0 + c];
        }
        __syncthreads();
    }
    for (int q = t; q < kBlockVocab * kSeg; q += kThreads) {
        const int r = q / kSeg, d = d0 + (q % kSeg) * CE;
        const int pos = cb * kBlockVocab + r;
        const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
        if (v < 0 || v >= V || d >= D) continue;
        u32x4 out;
        T *op = reinterpret_cast<T *>(&out);
#pragma unroll
        for (int c = 0; c < CE; ++c) op[c] = from_f32<T>(run[r * kHotF + (d - d0) + c]);
        *reinterpret_cast<u32x4 *>(dE.row(v) + d) = out;
    }
    __syncthreads();  // (the stage buffer and rlo are reused by the next item)
}

// The label path for dE item (cb, d0), if it applies: every kept block of
// vocabulary block cb is label-only (status 2) and the block is hot or
// passes label_path_ok.
// Returns -1 when the item's rows were written, else the number of kept row
// blocks, listed in sh.list (for de_item), or -2 when the column's row
// blocks do not fit one list.
template <typename T>
__device__ __forceinline__ int de_try_label(GradLds<T> &sh, int cb, int d0, int n_rb, const uint8_t *__restrict__ st,
                                            int cbp, const LabelCols<T> &lc, const int32_t *__restrict__ perm, int D,
                                            int V, Rows2<T> dE) {
    if (n_rb > kListCap) return -2;  // uniform
    if (threadIdx.x == 0) sh.soft = 0;
    __syncthreads();
    const int n = build_list<TileG::kThreads>(
        n_rb,
        [&](int i) {
            const int s = st[(int64_t)i * cbp + cb];
            if (s == 1 || s == 3) atomicOr(&sh.soft, 1);
            return s != 0;
        },
        sh.list, sh.wcnt);
    // (build_list ends with a barrier: sh.soft is final)
    if (!lc.labels || n == 0 || sh.soft) return n;
    const int h = lc.hidx[cb];
    if (h >= 0) {  // a hot column: its kHotF-feature tiles of this item
        for (int d = d0; d < d0 + TileG::BN && d < D; d += kHotF) hot_item<T>(sh, h, cb, d / kHotF, lc, perm, D, V, dE);
        return -1;
    }
    if (!label_path_ok(lc.cent[cb])) return n;
    label_group<T>(sh, n, cb, lc, V);
    label_rows<T>(sh, cb, d0, d0 + TileG::BN, lc, perm, D, V, dE);
    return -1;
}

// dE rows of a static vocabulary block cb (see k_plan), features
// [d_lo, d_hi): its kept blocks are all label-only and pass label_path_ok, so
// its rows are the label entries' sums in token order (zero rows when
// nothing is kept).
template <typename T>
__device__ __forceinline__ void de_column_item(GradLds<T> &sh, int cb, int d_lo, int d_hi, int n_rb,
                                               const uint8_t *__restrict__ st, int cbp, const LabelCols<T> &lc,
                                               const int32_t *__restrict__ perm, int D, int V, Rows2<T> dE) {
    const int n = build_list<TileG::kThreads>(
        n_rb, [&](int i) { return st[(int64_t)i * cbp + cb] != 0; }, sh.list, sh.wcnt);
    if (n > 0) {
        label_group<T>(sh, n, cb, lc, V);
    } else {
        for (int r = threadIdx.x; r <= kBlockVocab; r += TileG::kThreads) sh.rlo[r] = 0;
        __syncthreads();
    }
    label_rows<T>(sh, cb, d_lo, d_hi, lc, perm, D, V, dE);
}

// dE for one (vocabulary block cb, 256-feature tile d0) item of a pass.  K
// runs over the valid tokens of the row blocks kept for cb, in order (DMA
// pipeline, 64 K-bytes per stage): A = the stored block Gt[slot] (128
// vocabulary rows x 128 tokens), B = H^T.  The product of each group of
// kKahanBlocks kept row blocks (the last group may hold fewer) is formed in a
// fresh fp32 accumulator and then added into (sum, compensation) with
// Kahan's rule; the result is written once, through LDS as 16-byte row
// segments (bf16).  A vocabulary block with nothing kept gets dE = 0.
// pre_n >= 0: the kept row blocks (all of them: n_rb <= kListCap) are
// already listed in sh.list.
template <typename T, bool KAHAN, bool FINE>
__device__ __forceinline__ void de_item(GradLds<T> &sh, int cb, int d0, int n_rb, const uint8_t *__restrict__ st,
                                        const int32_t *__restrict__ slotm, int cbp, const T *__restrict__ Gt,
                                        const T *__restrict__ Ht, int64_t ldh, const int32_t *__restrict__ perm,
                                        int D, int V, Rows2<T> dE, int pre_n, const uint16_t *__restrict__ smask) {
    using TL = TileG;
    // 128-byte stages (two per row block of bf16), one in flight: half the
    // loop iterations and list lookups of 64-byte stages in the same LDS; the
    // fine filter keeps 64-byte stages (32 tokens, one sub-tile column, per
    // stage half)
    constexpr bool kWide = !FINE;
    using DE = DmaEngine<T, TL, kWide ? 128 : 64, kWide ? 2 : 4>;
    static_assert(DE::kLdsChunks <= GradLds<T>::kStageChunks, "stages fit the shared stage buffer");
    constexpr int kBlockBytes = kBlockRows * (int)sizeof(T);  // K bytes of one row block
    constexpr int kSpb = kBlockBytes / DE::kStageBytes;       // stages per row block
    constexpr int64_t kStoreBytes = (int64_t)kBlockElems * sizeof(T);
    constexpr int CE = ChunkElems<T>::value;
    const int tid = opaque_tid();  // per-item lane arithmetic is redone per item, not held in registers
    DE eng(sh.stages);
#pragma unroll
    for (int j = 0; j < DE::NIA; ++j) {
        const int r = DE::row_a(j, tid);
        eng.pa[j] = reinterpret_cast<const char *>(Gt + (int64_t)r * kBlockRows) + DE::chunk_off(j, r, tid);
    }
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j, tid);
        const int d = min(d0 + r, D - 1);
        eng.pb[j] = reinterpret_cast<const char *>(Ht + (int64_t)d * ldh) + DE::chunk_off(j, r, tid);
    }
    f32x16 acc[TL::TM][TL::TN], sum[TL::TM][TL::TN], comp[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    zero_acc<TL>(sum);
    zero_acc<TL>(comp);

    bool any = false;
    for (int base = 0; base < n_rb; base += kListCap) {
        const int cnt = n_rb - base < kListCap ? n_rb - base : kListCap;
        const int n = pre_n >= 0 ? pre_n
                                 : build_list<TL::kThreads>(
                                       cnt, [&](int i) { return st[(int64_t)(base + i) * cbp + cb] != 0; }, sh.list,
                                       sh.wcnt);
        for (int i = threadIdx.x; i < n; i += TL::kThreads) {
            sh.lslot[i] = slotm[(int64_t)(base + sh.list[i]) * cbp + cb];
            if (FINE) sh.lmask[i] = smask[(int64_t)(base + sh.list[i]) * cbp + cb];
        }
        __syncthreads();
        any |= n > 0;
        // Fine filter: stage k covers the tokens of sub-tile column jk(k) of
        // the block; only stages with a possibly nonzero sub-tile are listed,
        // and a wave multiplies only its vocabulary sub-rows whose sub-tile
        // may be nonzero.  (All-zero sub-tiles add exact zeros, so skipping
        // them changes nothing but the work.)
        constexpr int kTokPerStage = DE::kStageBytes / (int)sizeof(T);
        auto jk = [](int k) { return k * kTokPerStage / 32; };
        int total = n * kSpb;
        if constexpr (FINE)
            total = build_stages<TL::kThreads>(
                n, kSpb, sh.lmask, [&](int k) { return 0x1111 << jk(k); }, sh.stl, sh.wcnt);
        auto issue = [&](int buf, int q) {
            int b = q / kSpb, k = q % kSpb;
            if constexpr (FINE) {
                b = (sh.stl[q] >> 4) & 0x7FF;
                k = sh.stl[q] & 15;
            }
            const int kb = k * DE::kStageBytes;
            eng.issue2(buf, sh.lslot[b] * kStoreBytes + kb, (int64_t)(base + sh.list[b]) * kBlockBytes + kb);
        };
#pragma unroll
        for (int q = 0; q < DE::kDepth; ++q)
            if (q < total) issue(q, q);
        for (int s = 0; s < total; ++s) {
            const int ahead = total - 1 - s;
            eng.wait_stage(eng.clamp_ahead(ahead));
            if (s + DE::kDepth < total) issue((s + DE::kDepth) % DE::kStages, s + DE::kDepth);
            bool flush = (s % (kSpb * kKahanBlocks)) == kSpb * kKahanBlocks - 1 || s == total - 1;
            if constexpr (FINE) {
                const int e = sh.stl[s];
                const uint32_t m = (uint32_t)sh.lmask[(e >> 4) & 0x7FF];
                const int j = jk(e & 15), i0 = 2 * ((tid >> 6) % TL::WM);  // the wave's first vocabulary sub-row
                static_assert(TL::TM == 2 && TL::kWaveM == 64, "a wave holds two 32-row sub-rows of the block");
                const uint32_t rows = ((m >> (4 * i0 + j)) & 1) | (((m >> (4 * (i0 + 1) + j)) & 1) << 1);
                compute_rows<T, TL>(eng, s % DE::kStages, acc, tid, rows);
                // (the same terms as without the sub-tile filter: the end of
                // every kKahanBlocks-th listed block, and the last stage)
                // (e is the same in every lane: the flush is uniform)
                flush = __builtin_amdgcn_readfirstlane(
                            e < 0 && ((((e >> 4) & 0x7FF) % kKahanBlocks) == kKahanBlocks - 1 || s == total - 1)) != 0;
            } else {
                eng.compute(s % DE::kStages, acc, tid);
            }
            if (KAHAN && flush) {
#pragma clang fp contract(off)
#pragma unroll
                for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float y = acc[tm][tn][r] - comp[tm][tn][r];
                            const float t = sum[tm][tn][r] + y;
                            comp[tm][tn][r] = (t - sum[tm][tn][r]) - y;
                            sum[tm][tn][r] = t;
                            acc[tm][tn][r] = 0.f;
                        }
            }
        }
        __syncthreads();  // list[], lslot[] and the LDS stages are reused next
    }

    // Output rows: 128 vocabulary entries x 256 features, in 16-byte segments.
    constexpr int kSeg = TL::BN / CE;  // segments per row
    if (!any) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int q = threadIdx.x; q < TL::BM * kSeg; q += TL::kThreads) {
            const int row = q / kSeg, d = d0 + (q % kSeg) * CE;
            const int pos = cb * TL::BM + row;
            const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
            if (v >= 0 && v < V && d < D) *reinterpret_cast<u32x4 *>(dE.row(v) + d) = z;
        }
        return;
    }
    if constexpr (sizeof(T) == 2) {
        // stage the tile in LDS (row stride 256 + 8 elements), then write rows
        constexpr int kLd = TL::BN + 8;
        T *tile = reinterpret_cast<T *>(sh.stages);
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int col = tile_col<TL>(tn, tid);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float val = KAHAN ? sum[tm][tn][r] - comp[tm][tn][r] : acc[tm][tn][r];
                    tile[tile_row<TL>(tm, r, tid) * kLd + col] = from_f32<T>(val);
                }
            }
        __syncthreads();
        for (int q = threadIdx.x; q < TL::BM * kSeg; q += TL::kThreads) {
            const int row = q / kSeg, c = q % kSeg, d = d0 + c * CE;
            const int pos = cb * TL::BM + row;
            const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
            if (v >= 0 && v < V && d < D)
                *reinterpret_cast<u32x4 *>(dE.row(v) + d) =
                    *reinterpret_cast<const u32x4 *>(tile + row * kLd + c * CE);
        }
        __syncthreads();  // the stages are reused by the next item
    } else {
        int vid[TL::TM][16];  // output row of each accumulator row (-1: none), loaded once
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = cb * TL::BM + tile_row<TL>(tm, r, tid);
                const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
                vid[tm][r] = (v >= 0 && v < V) ? v : -1;
            }
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int d = d0 + tile_col<TL>(tn, tid);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float val = KAHAN ? sum[tm][tn][r] - comp[tm][tn][r] : acc[tm][tn][r];
                    if (vid[tm][r] >= 0 && d < D) dE.row(vid[tm][r])[d] = from_f32<T>(val);
                }
            }
    }
}

// dH for one (128-token block rb, 256-feature tile d0) item of a pass.  K
// runs over the kept vocabulary blocks of the pass in order.  Each block's
// product is formed in a fresh accumulator and added to the running sum,
// which starts from the previous passes' fp32 sum, so the result does not
// depend on where the passes are cut.  The last pass writes dH in the output
// dtype.
template <typename T, bool FINE>
__device__ __forceinline__ void dh_item(GradLds<T> &sh, int rb, int d0, bool multi, bool first, bool last, int cb0,
                                        int cb1,
                                        const uint8_t *__restrict__ st, const int32_t *__restrict__ slotm, int cbp,
                                        int nv, const int32_t *__restrict__ idx, const T *__restrict__ Gn,
                                        Rows2<const T> E, const int32_t *__restrict__ perm, int D, int V,
                                        const float *__restrict__ glab,
                                        const int64_t *__restrict__ labels, float *__restrict__ dh_acc,
                                        T *__restrict__ dH, const uint16_t *__restrict__ smask) {
    using TL = TileG;
    using DH = DhEngine<T, !FINE>;  // the fine filter's sub-tile rows need 32-entry stages
    const int tok0 = rb * TL::BM;
    const int tid = opaque_tid();  // per-item lane arithmetic is redone per item, not held in registers

    f32x16 acc[TL::TM][TL::TN], sum[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    if (multi && !first) {  // the running sum of the earlier passes (written for the valid rows)
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int d = min(d0 + tile_col<TL>(tn, tid), D - 1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = tok0 + tile_row<TL>(tm, r, tid);
                    sum[tm][tn][r] = tok < nv ? dh_acc[(int64_t)tok * D + d] : 0.f;
                }
            }
    } else {
        zero_acc<TL>(sum);
    }

    DH eng(sh.stages, d0, D, tid);
    bool any = false;
    for (int base = cb0; base < cb1; base += kListCap) {
        const int cnt = cb1 - base < kListCap ? cb1 - base : kListCap;
        const int n = build_list<TL::kThreads>(
            cnt,
            [&](int i) {
                const int v = st[(int64_t)rb * cbp + base + i];
                return v == 1;  // label-only blocks: the label term below
            },
            sh.list, sh.wcnt);
        for (int i = threadIdx.x; i < n; i += TL::kThreads) {
            sh.lslot[i] = slotm[(int64_t)rb * cbp + base + sh.list[i]];
            if (FINE) sh.lmask[i] = smask[(int64_t)rb * cbp + base + sh.list[i]];
        }
        __syncthreads();
        any |= n > 0;
        // Fine filter: stage k covers the vocabulary entries of sub-tile row
        // ik(k) of the block; as for dE, only stages and wave rows (token
        // sub-columns here) whose sub-tile may be nonzero are multiplied.
        auto ik = [](int k) { return k * DH::kKv / 32; };
        int total = n * DH::kSpb;
        if constexpr (FINE)
            total = build_stages<TL::kThreads>(
                n, DH::kSpb, sh.lmask, [&](int k) { return 0xF << (4 * ik(k)); }, sh.stl, sh.wcnt);
        auto issue = [&](int buf, int q) {
            int b = q / DH::kSpb, k = q % DH::kSpb;
            if constexpr (FINE) {
                b = (sh.stl[q] >> 4) & 0x7FF;
                k = sh.stl[q] & 15;
            }
            eng.issue(buf, Gn, sh.lslot[b], E, perm, (base + sh.list[b]) * kBlockVocab, k, V);
        };
#pragma unroll
        for (int q = 0; q < DH::kDepth; ++q)
            if (q < total) issue(q, q);
        for (int s = 0; s < total; ++s) {
            const int ahead = total - 1 - s;
            eng.wait_stage(eng.clamp_ahead(ahead));
            if (s + DH::kDepth < total) issue((s + DH::kDepth) % DH::kStages, s + DH::kDepth);
            bool flush = (s % DH::kSpb) == DH::kSpb - 1;
            if constexpr (FINE) {
                const int e = sh.stl[s];
                const uint32_t m = (uint32_t)sh.lmask[(e >> 4) & 0x7FF];
                const int i = ik(e & 15), j0 = 2 * ((tid >> 6) % TL::WM);  // the wave's first token sub-column
                static_assert(TL::TM == 2 && TL::kWaveM == 64, "a wave holds two 32-token sub-columns of the block");
                const uint32_t rows = ((m >> (4 * i + j0)) & 1) | (((m >> (4 * i + j0 + 1)) & 1) << 1);
                eng.compute(s % DH::kStages, acc, tid, rows);
                flush = e < 0;
            } else {
                eng.compute(s % DH::kStages, acc, tid);
            }
            if (flush) {
#pragma unroll
                for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            sum[tm][tn][r] += acc[tm][tn][r];
                            acc[tm][tn][r] = 0.f;
                        }
            }
        }
        __syncthreads();  // list[], lslot[] and the LDS stages are reused next
    }
    // nothing added in this pass: the running sum stands (the first pass
    // still writes it, as the later ones read it)
    if (!any && !last && !first) return;

    if (last) {
        int row[TL::TM][16];  // output row of each accumulator row, loaded once
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) row[tm][r] = idx[min(tok0 + tile_row<TL>(tm, r, tid), nv - 1)];
        // The label term of the rows whose label block is label-only (kept out
        // of the block products): dH_i += g_i e_{y_i}, after every block.
        {
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = tok0 + tile_row<TL>(tm, r, tid);
                    const float g = tok < nv ? glab[tok] : 0.f;
                    if (g != 0.f) {
                        const T *e = E.row(labels[row[tm][r]]);
#pragma unroll
                        for (int tn = 0; tn < TL::TN; ++tn) {
                            const int d = d0 + tile_col<TL>(tn, tid);
                            if (d < D) sum[tm][tn][r] += g * to_f32(e[d]);
                        }
                    }
                }
        }
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int d = d0 + tile_col<TL>(tn, tid);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = tok0 + tile_row<TL>(tm, r, tid);
                    if (tok < nv && d < D) dH[(int64_t)row[tm][r] * D + d] = from_f32<T>(sum[tm][tn][r]);
                }
            }
    } else {
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int d = d0 + tile_col<TL>(tn, tid);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = tok0 + tile_row<TL>(tm, r, tid);
                    if (tok < nv && d < D) dh_acc[(int64_t)tok * D + d] = sum[tm][tn][r];
                }
            }
    }
}

// --------------------------------------------------- gradient products
// Gradient phase of pass p: the workgroups take items from a work queue,
// longer items first: the (vocabulary block, feature tile) dE items of the
// vocabulary blocks that are not static (block products over every kept row
// block: the longest), then the (row block, feature tile) dH items, then the
// items of the pass's static vocabulary blocks (all features, or one
// feature tile of a block with many label entries).
template <typename T, bool KAHAN, bool FINE>
__device__ __forceinline__ void grad_phase(const BwdArgs<T> &a, int p, int P, GradLds<T> &sh, int *ticket) {
    using TL = TileG;
    const PlanView pv = plan_view(a.plan, a.max_passes);
    int32_t *queue = plan_queues(a.plan, a.max_passes, p) + 8;
    const int nv = *a.nvalid;
    const int CB = (a.V + kBlockVocab - 1) / kBlockVocab;
    const int cb0 = 2 * pv.vt_begin[p];
    const int cb1 = min(2 * pv.vt_begin[p + 1], CB);
    const int n_dt = (a.D + TL::BN - 1) / TL::BN;
    const int n_rbv = (nv + kBlockRows - 1) / kBlockRows;
    const int64_t n_dh = (int64_t)n_rbv * n_dt;
    // the pass's static columns are slist[s_lo, s_hi) (their items
    // citem[i_lo, i_hi)), the others dlist[c_lo, c_lo + n_dyn)
    const int s_lo = cb1 > cb0 ? a.cpre[cb0] : 0, s_hi = cb1 > cb0 ? a.cpre[cb1] : 0;
    const int i_lo = cb1 > cb0 ? a.ipre[s_lo] : 0, i_hi = cb1 > cb0 ? a.ipre[s_hi] : 0;
    const int c_lo = cb0 - s_lo;
    const int n_dyn = cb1 > cb0 ? (cb1 - cb0) - (s_hi - s_lo) : 0;
    const int64_t n_col = i_hi - i_lo;
    const int64_t n_de = (int64_t)n_dyn * n_dt;
    // (no label path for the full classifier gradient: its label-only blocks
    // store the unfiltered gradient for dE)
    const LabelCols<T> lc{a.full_de ? nullptr : a.labels, a.idx, a.inv_perm, a.glab, a.H, nv, a.cent,
                          a.hidx, a.hent, a.hrlo, a.hent_t};
    // two loops rather than one with a branch: each keeps its own registers
    int64_t it = take_ticket(queue, ticket);
    while (it < n_de) {
        const int cb = a.dlist[c_lo + (int)(it / n_dt)], d0 = (int)(it % n_dt) * TL::BN;
        const int n = de_try_label<T>(sh, cb, d0, n_rbv, a.st, a.cbp, lc, a.perm, a.D, a.V, a.dE);
        if (n != -1)
            de_item<T, KAHAN, FINE>(sh, cb, d0, n_rbv, a.st, a.slot, a.cbp, a.Gt, a.Ht, a.ldh, a.perm, a.D, a.V, a.dE,
                                    n >= 0 ? n : -1, a.smask);
        it = take_ticket(queue, ticket);
    }
    while (it < n_de + n_dh) {
        const int64_t q = it - n_de;
        dh_item<T, FINE>(sh, (int)(q % n_rbv), (int)(q / n_rbv) * TL::BN, P > 1, p == 0, p == P - 1, cb0, cb1, a.st,
                         a.slot, a.cbp, nv, a.idx, a.Gn, a.E, a.perm, a.D, a.V, a.glab, a.labels, a.dh_acc, a.dH,
                         a.smask);
        it = take_ticket(queue, ticket);
    }
    while (it < n_de + n_dh + n_col) {
        const int ci = i_lo + (int)(it - n_de - n_dh);
        const int cb = a.citem[ci], ft = a.cft[ci];
        if (ft <= -2) {
            hot_item<T>(sh, a.hidx[cb], cb, -2 - ft, lc, a.perm, a.D, a.V, a.dE);
        } else {
            const int d_lo = ft == kAllFeatures ? 0 : ft * TL::BN;
            const int d_hi = ft == kAllFeatures ? a.D : min(a.D, d_lo + TL::BN);
            de_column_item<T>(sh, cb, d_lo, d_hi, n_rbv, a.st, a.cbp, lc, a.perm, a.D, a.V, a.dE);
        }
        it = take_ticket(queue, ticket);
    }
}

// One launch per pass and phase.
template <typename T, bool DMA>
__global__ __launch_bounds__(TileF::kThreads) void k_g_pass(BwdArgs<T> a, int p) {
    __shared__ u32x4 lds[GPassLds<T, DMA>::value];
    __shared__ int qflag[12], qstat[4], qslot[4];
    // The work-queue ticket has a word of its own: the epilogue's waves read
    // qslot after its last barrier, while thread 0 may already take the next
    // ticket.
    __shared__ int ticket;
    if (p >= *plan_view(a.plan, a.max_passes).P) return;
    g_phase<T, DMA>(a, p, blockIdx.x, gridDim.x, lds, qflag, qstat, qslot, &ticket);
}

template <typename T, bool KAHAN, bool FINE>
__global__ __launch_bounds__(TileG::kThreads) void k_grad_pass(BwdArgs<T> a, int p) {
    __shared__ GradLds<T> sh;
    __shared__ int ticket;
    const int P = *plan_view(a.plan, a.max_passes).P;
    if (p >= P) return;
    grad_phase<T, KAHAN, FINE>(a, p, P, sh, &ticket);
}

// ---------------------------------------------------------------- launchers
BwdShape bwd_shape(int64_t N, int64_t D, int64_t V) {
    BwdShape s;
    s.N = N;
    s.D = D;
    s.V = V;
    s.Np = round_up(N, kTileRows);
    s.n_rtiles = (int)(s.Np / kTileRows);
    s.n_vtiles = (int)ceil_div(V, kTileVocab);
    s.n_rb = (int)(s.Np / kBlockRows);
    s.cbp = 2 * s.n_vtiles;
    const int64_t total = (int64_t)s.n_rb * s.cbp;
    const int64_t vp = round_up(V, kTileVocab);
    const int64_t slice_cb = (vp < kStoreVocab ? vp : kStoreVocab) / kBlockVocab;
    // (at least kMinStoreBlocks: few rows over a large vocabulary would
    // otherwise take one pass per few vocabulary tiles)
    s.cap = std::max<int64_t>((int64_t)s.n_rb * slice_cb, kMinStoreBlocks);
    if (total <= s.cap) {
        s.cap = total;
        s.cap_eff = total;
        s.max_passes = 1;
    } else {
        s.cap_eff = s.cap - 2 * (int64_t)s.n_rb;
        s.max_passes = (int)(total / s.cap_eff) + 1;
    }
    s.plan_ints = plan_ints(s.max_passes);
    return s;
}

BwdWs bwd_ws(void *ws, const BwdShape &s, size_t elem, size_t *bytes) {
    Carver c(ws);
    BwdWs w;
    const size_t nblk = (size_t)s.n_rb * s.cbp;
    const size_t ntile = (size_t)s.n_rtiles * s.n_vtiles;
    w.idx = c.take<int32_t>(s.N);
    w.nvalid = c.take<int32_t>(1);
    w.inv_perm = c.take<int32_t>(s.V);
    w.lmin = c.take<float>((size_t)s.n_rb);
    w.glab = c.take<float>((size_t)s.Np);
    w.lab = c.take<uint8_t>(nblk);
    w.st = c.take<uint8_t>(nblk);
    w.csoft = c.take<uint8_t>((size_t)s.cbp);  // csoft, cnlab, cent, vneed and vact follow st: one fill clears them
    w.cnlab = c.take<int32_t>((size_t)s.cbp);
    w.cent = c.take<int32_t>((size_t)s.cbp);
    w.vneed = c.take<int32_t>((size_t)s.n_vtiles);
    w.vact = c.take<int32_t>((size_t)s.n_vtiles);
    w.slot = c.take<int32_t>(nblk);
    w.smask = c.take<uint16_t>(nblk);
    w.cpre = c.take<int32_t>((size_t)s.cbp + 1);
    w.slist = c.take<int32_t>((size_t)s.cbp);
    w.ipre = c.take<int32_t>((size_t)s.cbp + 1);
    // (a split column has more than kColSplitEntries of the N label entries)
    // (a hot column has more than kLabelEntries of the N label entries)
    const size_t hmax = (size_t)hot_max(s.N, s.cbp);
    const size_t n_items = (size_t)s.cbp + (size_t)(s.N / (kColSplitEntries + 1) + 1) * (size_t)n_feature_tiles(s.D) +
                           hmax * (size_t)n_hot_tiles(s.D);
    w.citem = c.take<int32_t>(n_items);
    w.cft = c.take<int32_t>(n_items);
    w.tpos = c.take<int32_t>(s.N);
    w.hidx = c.take<int32_t>((size_t)s.cbp);
    w.hcol = c.take<int32_t>(hmax);
    w.hent = c.take<int32_t>(hmax + 1);
    w.nhot = c.take<int32_t>(1);
    w.hrlo = c.take<int32_t>(hmax * 129);
    w.hent_t = c.take<int32_t>(s.N);
    w.hcnt = c.take<int32_t>(hmax * (size_t)hot_slices(s.N) * kBlockVocab);
    w.dlist = c.take<int32_t>((size_t)s.cbp);
    w.tneed = c.take<uint8_t>(ntile);
    w.cum = c.take<int64_t>((size_t)s.n_vtiles);
    w.act = c.take<int32_t>((size_t)s.n_vtiles);
    w.tlist = c.take<int32_t>(ntile);
    w.plan = c.take<int32_t>((size_t)s.plan_ints);

    w.dh_acc = s.max_passes > 1 ? c.take<float>((size_t)s.Np * s.D) : nullptr;
    w.Ht = c.take<char>(elem * (size_t)s.D * s.Np);
    w.Gt = c.take<char>(elem * (size_t)s.cap * kBlockElems);
    w.Gn = c.take<char>(elem * (size_t)s.cap * kBlockElems);
    if (bytes) *bytes = c.off;
    return w;
}

#define CCE_TRY(x)                                  \
    do {                                            \
        hipError_t e_ = (x);                        \
        if (e_ != hipSuccess) return e_;            \
    } while (0)
#define CCE_LAUNCHED() CCE_TRY(hipGetLastError())

template <typename T>
static hipError_t backward_t(const T *H, Rows2<const T> E, const int64_t *labels, const float *lse,
                             const float *dloss, const float *block_max, const BwdShape &s, int64_t ignore_index,
                             float eps, const int32_t *perm, unsigned flags, T *dH, Rows2<T> dE, int64_t *stats,
                             const BwdWs &w, hipStream_t st) {
    const int D = (int)s.D, V = (int)s.V;
    CCE_TRY(launch_compact(labels, s.N, ignore_index, w.idx, w.nvalid, st));
    if (perm) {
        CCE_TRY(launch_inv_perm(perm, V, w.inv_perm, st));
    }
    // Cleared: the label map; st, csoft, cnlab, cent, vneed and vact (one
    // carved run); the label gradients (Np floats); the stats; ignored rows
    // of dH.  (Carved regions are 256-byte aligned: whole 32-bit words.)
    const size_t nblk = (size_t)s.n_rb * s.cbp;
    const size_t run_bytes = (size_t)(reinterpret_cast<char *>(w.vact + s.n_vtiles) - reinterpret_cast<char *>(w.st));
    hipLaunchKernelGGL(k_bwd_clear<T>, dim3(1024), dim3(256), 0, st, reinterpret_cast<uint32_t *>(w.lab),
                       (int64_t)(align256(nblk) / 4), reinterpret_cast<uint32_t *>(w.st), (int64_t)(align256(run_bytes) / 4),
                       reinterpret_cast<uint32_t *>(w.glab), (int64_t)s.Np, stats, labels, s.N, D, ignore_index, dH);
    CCE_LAUNCHED();
    T *Ht = static_cast<T *>(w.Ht);
    T *Gt = static_cast<T *>(w.Gt);
    T *Gn = static_cast<T *>(w.Gn);

    // The block maxima (in the processing order the forward used, which the
    // caller keeps equal to perm) only say something when filtering is on.
    // thr = ln(eps / 2), rounded towards -inf.
    const bool full_de = (flags & CCE_BWD_FULL_DE) != 0;
    const float *tb = (block_max && eps > 0.f && !full_de) ? block_max : nullptr;
    float thr = 0.f;
    if (tb) {
        thr = (float)(log((double)eps) - log(2.0));
        thr = nextafterf(thr, -__builtin_huge_valf());
    }
    const int32_t *invp = perm ? w.inv_perm : nullptr;
    {  // H^T of the valid rows ([D, Np], zero beyond them), lmin (with the table), the label map
        const int n_tx = (int)ceil_div(s.Np, 64);
        const int64_t n_tr = (int64_t)n_tx * ceil_div(D, 64);
        const int64_t n_lse = tb ? ceil_div(s.n_rb, 2) : 0;
        const int64_t n_map = ceil_div(s.N, 256);
        hipLaunchKernelGGL(k_bwd_prep<T>, dim3((unsigned)(n_tr + n_lse + n_map)), dim3(256), 0, st, H, D, s.N, w.idx,
                           w.nvalid, (int)s.Np, Ht, n_tx, n_tr, lse, w.lmin, s.n_rb, n_lse, labels, invp, s.V, s.cbp,
                           w.lab, w.tpos);
        CCE_LAUNCHED();
    }
    const int64_t ntile = (int64_t)s.n_rtiles * s.n_vtiles;
    hipLaunchKernelGGL(k_tile_class, dim3((unsigned)ceil_div(ntile, 256)), dim3(256), 0, st, w.nvalid, s.V,
                       s.n_rtiles, s.n_vtiles, s.cbp, w.lab, tb, w.lmin, thr, w.tneed, w.csoft, w.cnlab, w.cent,
                       w.vneed, w.vact);
    CCE_LAUNCHED();
    // static columns need the label path (off for the full classifier
    // gradient) and a column's row blocks in one list
    const int CB = (int)ceil_div(V, kBlockVocab);
    const int static_ok = (!full_de && s.n_rb <= kListCap) ? 1 : 0;
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, w.vneed, w.vact, s.n_vtiles, s.cap, s.cap_eff,
                       s.max_passes, w.plan, w.cum, w.act, CB, static_ok, w.csoft, w.cnlab, w.cent, w.cpre, w.slist,
                       w.dlist, n_feature_tiles(D), n_hot_tiles(D), w.ipre, w.citem, w.cft, w.hidx, w.hcol, w.hent,
                       w.nhot, stats);
    CCE_LAUNCHED();
    if (static_ok) {  // the hot columns' entries, grouped by row (at most hmax columns)
        const int64_t hmax = hot_max(s.N, s.cbp);
        const int S = hot_slices(s.N), slice = hot_slice(s.N);
        hipLaunchKernelGGL(k_hot_count, dim3((unsigned)S, (unsigned)hmax), dim3(1024), 0, st, w.nhot, w.hcol,
                           w.nvalid, w.tpos, slice, w.hcnt);
        CCE_LAUNCHED();
        hipLaunchKernelGGL(k_hot_place, dim3((unsigned)S, (unsigned)hmax), dim3(1024), 0, st, w.nhot, w.hcol, w.hent,
                           w.nvalid, w.tpos, slice, w.hcnt, w.hrlo, w.hent_t);
        CCE_LAUNCHED();
    }
    {  // the tile list, and the static columns' label-only blocks (without the table no column is static)
        const int64_t n_list = ceil_div(s.n_vtiles, 4);
        const int64_t n_static = (static_ok && tb) ? ceil_div(s.N, 256) : 0;
        hipLaunchKernelGGL(k_bwd_lists, dim3((unsigned)(n_list + n_static)), dim3(256), 0, st, w.tneed, s.n_rtiles,
                           s.n_vtiles, w.act, w.lab, s.cbp, w.cpre, CB, w.tlist, n_list, labels, w.idx, w.nvalid,
                           invp, s.V, lse, dloss, tb ? tb + block_max_blocks(s.N, s.V) : nullptr, w.st, w.glab);
        CCE_LAUNCHED();
    }

    BwdArgs<T> a;
    a.plan = w.plan;
    a.max_passes = s.max_passes;
    a.tlist = w.tlist;
    a.tneed = w.tneed;
    a.n_rt = s.n_rtiles;
    a.H = H;
    a.E = E;
    a.Ht = Ht;
    a.ldh = s.Np;
    a.idx = w.idx;
    a.nvalid = w.nvalid;
    a.perm = perm;
    a.inv_perm = invp;
    a.labels = labels;
    a.lse = lse;
    a.dloss = dloss;
    a.glab = w.glab;
    // the table's second part: the forward's label logits (read for label
    // entries of tiles the bound leaves out)
    a.zlab = tb ? tb + block_max_blocks(s.N, s.V) : nullptr;
    a.D = D;
    a.V = V;
    a.cbp = s.cbp;
    a.n_rb = s.n_rb;
    a.eps = eps;
    a.full_de = full_de ? 1 : 0;
    a.Gt = Gt;
    a.Gn = Gn;
    a.cap = s.cap;
    a.cap_take = (flags & CCE_BWD_DEBUG_STORE_LIMIT) ? s.cap / 2 : s.cap;
    a.st = w.st;
    a.slot = w.slot;
    a.smask = w.smask;
    a.cpre = w.cpre;
    a.slist = w.slist;
    a.ipre = w.ipre;
    a.citem = w.citem;
    a.cft = w.cft;
    a.hidx = w.hidx;
    a.hent = w.hent;
    a.hrlo = w.hrlo;
    a.hent_t = w.hent_t;
    a.dlist = w.dlist;
    a.cent = w.cent;
    a.CB = CB;
    a.fine = (flags & CCE_BWD_FINE_FILTER) ? 1 : 0;
    a.stats = stats;
    a.dh_acc = w.dh_acc;
    a.dE = dE;
    a.dH = dH;

    const bool dma_g = ((int64_t)D * (int64_t)sizeof(T)) % kLogitRowBytes == 0;
    const bool kahan = !(flags & CCE_BWD_NO_KAHAN);
    for (int p = 0; p < s.max_passes; ++p) {
        if (dma_g)
            hipLaunchKernelGGL((k_g_pass<T, true>), dim3(kPassGroups), dim3(TileF::kThreads), 0, st, a, p);
        else
            hipLaunchKernelGGL((k_g_pass<T, false>), dim3(kPassGroups), dim3(TileF::kThreads), 0, st, a, p);
        CCE_LAUNCHED();
        const dim3 gg(2 * kPassGroups), gt(TileG::kThreads);
        if (a.fine) {
            if (kahan) hipLaunchKernelGGL((k_grad_pass<T, true, true>), gg, gt, 0, st, a, p);
            else hipLaunchKernelGGL((k_grad_pass<T, false, true>), gg, gt, 0, st, a, p);
        } else {
            if (kahan) hipLaunchKernelGGL((k_grad_pass<T, true, false>), gg, gt, 0, st, a, p);
            else hipLaunchKernelGGL((k_grad_pass<T, false, false>), gg, gt, 0, st, a, p);
        }
        CCE_LAUNCHED();
    }
    if (stats) {
        hipLaunchKernelGGL(k_stats_fin, dim3(1), dim3(64), 0, st, stats, w.nvalid, (int64_t)ceil_div(V, kBlockVocab));
        CCE_LAUNCHED();
    }
    return hipSuccess;
}

template <typename T>
static Rows2<const T> rows_in(const VocabRows &E, int64_t D) {
    return Rows2<const T>{static_cast<const T *>(E.e0), static_cast<const T *>(E.e1), E.v0, D};
}
template <typename T>
static Rows2<T> rows_out(const VocabGrads &dE, int64_t D) {
    return Rows2<T>{static_cast<T *>(dE.d0), static_cast<T *>(dE.d1), dE.v0, D};
}

hipError_t launch_backward(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels,
                           const float *lse, const float *dloss, const float *block_max, const BwdShape &s,
                           int64_t ignore_index, float eps, const int32_t *perm, unsigned flags,
                           void *dH, const VocabGrads &dE, int64_t *stats, const BwdWs &w, hipStream_t st) {
    if (dt == CCE_BF16)
        return backward_t<bf16_t>(static_cast<const bf16_t *>(H), rows_in<bf16_t>(E, s.D), labels, lse, dloss,
                                  block_max, s, ignore_index, eps, perm, flags, static_cast<bf16_t *>(dH),
                                  rows_out<bf16_t>(dE, s.D), stats, w, st);
    return backward_t<float>(static_cast<const float *>(H), rows_in<float>(E, s.D), labels, lse, dloss, block_max,
                             s, ignore_index, eps, perm, flags, static_cast<float *>(dH), rows_out<float>(dE, s.D),
                             stats, w, st);
}

}  // namespace cce
