// Forward of the fused classifier-head + cross-entropy on gfx950.
//
//  k_compact      valid-row compaction (rows whose label is not ignore_index)
//  k_label_dot    label logit <h_i, e_{y_i}> of each valid row (the indexed matmul);
//                 its last workgroups set the block-max table to -inf
//  k_fwd4         logit tiles Z^T = E_tile * H_tile^T on bf16 MFMA, kept in
//                 registers (4 waves, scheduled K loop); per token and
//                 vocabulary range an online running max / sum-exp (log2
//                 domain); partials written per segment
//  k_fwd_dma      the same on 8 waves (fp32, and a build without k_fwd4)
//  k_fwd          the same with VGPR-staged operands (D * size not a multiple of 128)
//  k_merge        per row: merge of the segment partials in vocabulary order
//                 -> lse; lse - label logit -> loss; its last workgroups
//                 decode the block-max table
//
// The method: cross-entropy needs only the correct-token logit and the
// log-sum-exp over the vocabulary, computed blockwise on chip while streaming
// vocabulary tiles, never writing the [rows x vocabulary] logits to memory
// (lit note "The loss and the mask: Cut Cross-Entropy + FlexAttention",
// section "Contribution"; CCE paper summary "Cut Your Losses in
// Large-Vocabulary Language Models", section "Approach").  The pages' kernel
// merges partial results with a concurrent log-add-exp at block granularity
// (summary, section "Limitations"); here the partials of each vocabulary range
// go to a small buffer and one ordered pass merges them, so the result is
// independent of scheduling.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "cce_device.hpp"
#include "cce_internal.hpp"
#include "k4.hpp"

namespace cce {

using TileF = Tile<kTileVocab, kTileRows, 2, 4>;   // A = vocabulary rows, B = token rows; 8 waves
using TileFD = TileF;                              // tile of the DMA logit kernels

constexpr float kNegInf = -__builtin_huge_valf();


// ------------------------------------------------------------- compaction
// One workgroup of 1024 threads.  Rows are read in batches of kBatch chunks
// of 1024 consecutive rows (one row per thread and chunk, all loads of a
// batch in flight at once); a valid row's position is the count of valid
// rows before it: earlier batches, earlier chunks of the batch, earlier
// waves of its chunk and earlier lanes of its wave (ballots).
__global__ __launch_bounds__(1024) void k_compact(const int64_t *__restrict__ labels, int64_t N,
                                                  int64_t ignore_index, int32_t *__restrict__ idx,
                                                  int32_t *__restrict__ nvalid) {
    constexpr int kBatch = 8;
    constexpr int kCounts = kBatch * 16;
    __shared__ int cnt[kCounts];  // valid rows per (chunk, wave), then their exclusive prefix in that order
    __shared__ int half, btotal;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int base = 0;  // valid rows before the batch (uniform)
    for (int64_t b0 = 0; b0 < N; b0 += (int64_t)kBatch * 1024) {
        bool v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int64_t r = b0 + (int64_t)k * 1024 + t;
            v[k] = r < N && labels[r] != ignore_index;
        }
        uint64_t bal[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            bal[k] = __ballot(v[k]);
            if (lane == 0) cnt[k * 16 + wave] = __popcll(bal[k]);
        }
        __syncthreads();
        int c = 0, x = 0;
        if (t < kCounts) {  // two waves: inclusive scan of the counts within each wave
            c = cnt[t];
            x = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            if (t == 63) half = x;
        }
        __syncthreads();
        if (t < kCounts) {
            const int incl = x + (t >= 64 ? half : 0);
            cnt[t] = incl - c;
            if (t == kCounts - 1) btotal = incl;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (v[k]) idx[base + cnt[k * 16 + wave] + __popcll(bal[k] & below)] = (int32_t)(b0 + (int64_t)k * 1024 + t);
        base += btotal;
        __syncthreads();  // cnt, half and btotal are rewritten by the next batch
    }
    if (t == 0) *nvalid = base;
}

// -------------------------------------------------------------- label check
__global__ __launch_bounds__(1024) void k_check_labels(const int64_t *__restrict__ labels, int64_t N,
                                                       int64_t V, int64_t ignore_index,
                                                       int64_t *__restrict__ n_bad) {
    __shared__ int64_t part[16];
    int64_t c = 0;
    for (int64_t r = threadIdx.x; r < N; r += 1024) {
        const int64_t y = labels[r];
        c += (y != ignore_index) && (y < 0 || y >= V);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t s = 0;
        for (int w = 0; w < 16; ++w) s += part[w];
        *n_bad = s;
    }
}

// ------------------------------------------------------- inverse permutation
__global__ __launch_bounds__(256) void k_inv_perm(const int32_t *__restrict__ perm, int V, int32_t *__restrict__ inv) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k < V) {
        const int v = perm[k];
        if (v >= 0 && v < V) inv[v] = k;
    }
}

// ------------------------------------------------------ composite labels
// Labels of a composite head (ids [0, V0) in the first block, [off1, off1 +
// V1) in the second, nothing in between) -> positions of the concatenated
// processing space [0, V0 + V1).  ignore_index stays; any other id outside
// both blocks becomes V0 + V1, which every kernel treats as out of range.
__global__ __launch_bounds__(256) void k_seg_labels(const int64_t *__restrict__ labels, int64_t N,
                                                    int64_t ignore_index, int64_t V0, int64_t off1, int64_t V1,
                                                    int64_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N) return;
    const int64_t y = labels[i];
    int64_t v = V0 + V1;
    if (y == ignore_index) v = y;
    else if (y >= 0 && y < V0) v = y;
    else if (y >= off1 && y < off1 + V1) v = V0 + (y - off1);
    out[i] = v;
}

// ------------------------------------------------------------ logit + LSE
// Work partition.  The work is the grid of 256 x 256 logit tiles of the valid
// rows: R token tiles x C vocabulary tiles.  Each token tile's vocabulary is
// cut into b ranges (range j: tiles [j C / b, (j + 1) C / b)); a (token tile,
// range) pair is a segment, streamed by one workgroup through one continuous
// K pipeline, and writes one partial (m, s) per token at slot rt b + j.
//
// Placement: hardware workgroup g runs on XCD g % 8, so the grid (persistent:
// as many workgroups as fit on the chip at once) is seen as nx = 8 groups of
// P workgroups (P = 32 on MI355X), one group per XCD.  A block is a x bb
// segments (a token tiles x bb consecutive ranges, a bb = P): the P
// workgroups of one XCD take one block at a time, all in step, so the
// classifier tiles in flight on an XCD are shared by a workgroups and the
// hidden-state tiles by bb in that XCD's L2.  Blocks (ceil(R / a) token
// groups x m range groups, b = bb m) go to the XCDs round-robin.  (a, bb, m)
// are chosen from the shape, the number of valid rows and the grid, so that
// the longest workgroup (steps x the longest range) is shortest; ties prefer
// a = 4 (4 x 8 at the Gemma-2-2B head: one block per XCD, the split that
// measured best there) and then fewer ranges.  An even split of the tile
// list over the workgroups instead cut ranges at vocabulary offsets that
// differ between token tiles when the tile count is not a multiple of the
// grid: on the Llama-3 head (39 token tiles) every workgroup of an XCD then
// streamed its own classifier tile, and the forward fetched 48 times its
// operands from memory.
//
// Within a segment each lane owns TN token columns and keeps, for each, m
// (running max of z log2 e) and l (running sum of 2^(z log2 e - m)) over the
// vocabulary rows it holds.  At the end of a segment the two half-waves and
// the WM waves that hold the same tokens are merged in a fixed order.
struct FwdGrid {
    int R, C;      // token tiles of the valid rows, vocabulary tiles
    int nx, P;     // XCD groups and workgroups per group
    int a, bb, m;  // block shape and range groups
    __device__ __forceinline__ int b() const { return bb * m; }
    __device__ __forceinline__ int blocks() const { return (R + a - 1) / a * m; }
    __device__ __forceinline__ int vt0(int j) const { return (int)((int64_t)j * C / b()); }
};

__device__ __forceinline__ FwdGrid fwd_grid(int nv, int C, int G) {
    FwdGrid g;
    g.R = (nv + kTileRows - 1) / kTileRows;
    g.C = C;
    g.nx = G % 8 == 0 ? 8 : 1;
    g.P = G / g.nx;
    g.a = 1; g.bb = g.P; g.m = 1;
    int64_t best = -1;
    int best_pref = 0;
    const int maxb = C < kFwdRanges ? C : kFwdRanges;
    for (int a = 1; a <= g.P; a *= 2) {
        if (g.P % a) continue;
        const int bb = g.P / a;
        const int pref = a == 4 ? 0 : 1;
        for (int m = 1; bb * m <= maxb; ++m) {
            const int64_t steps = ((g.R + a - 1) / a * (int64_t)m + g.nx - 1) / g.nx;
            const int64_t cost = steps * ((C + bb * m - 1) / (bb * m));
            if (best < 0 || cost < best || (cost == best && pref < best_pref)) {
                best = cost; best_pref = pref; g.a = a; g.bb = bb; g.m = m;
            }
        }
    }
    if (best < 0) { g.a = 1; g.bb = 1; g.m = 1; }  // P > maxb: one range, idle workgroups
    return g;
}

// The forward kernel's workgroup 0 records its choice of (a, bb, m) for the
// merge (one search per launch instead of one per row).
__device__ __forceinline__ FwdGrid fwd_grid_record(int nv, int C, int G, int *__restrict__ rec) {
    const FwdGrid g = fwd_grid(nv, C, G);
    if (blockIdx.x == 0 && threadIdx.x == 0) { rec[0] = g.a; rec[1] = g.bb; rec[2] = g.m; }
    return g;
}
// The same split as recorded.
__device__ __forceinline__ FwdGrid fwd_grid_recorded(int nv, int C, int G, const int *__restrict__ rec) {
    FwdGrid g;
    g.R = (nv + kTileRows - 1) / kTileRows;
    g.C = C;
    g.nx = G % 8 == 0 ? 8 : 1;
    g.P = G / g.nx;
    g.a = rec[0]; g.bb = rec[1]; g.m = rec[2];
    return g;
}

// The segments of hardware workgroup gid, in order: f(rt, t0, ntile, slot).
template <class F>
__device__ __forceinline__ void fwd_segments(const FwdGrid &g, int gid, F &&f) {
    const int x = gid % g.nx, i = gid / g.nx;
    const int ti = i / g.bb, ji = i % g.bb;
    if (ti >= g.a) return;  // (only with the one-range fallback)
    const int nb = g.blocks();
    for (int q = x; q < nb; q += g.nx) {
        const int rt = q / g.m * g.a + ti;
        const int j = q % g.m * g.bb + ji;
        if (rt >= g.R) continue;
        const int t0 = g.vt0(j), t1 = g.vt0(j + 1);
        if (t1 > t0) f(rt, t0, t1 - t0, (int64_t)rt * g.b() + j);
    }
}

// Online max / sum-exp update with the tile's logits.  Returns the largest
// logit this lane holds in the tile (rows past V excluded) other than a label
// entry: with LAB, lpos[tn] is the processing position of token column tn's
// label, that entry is left out of the returned maximum (it still enters the
// sum) and its logit is written to zlab[lrow[tn]] (lrow < 0: no write).
template <class TL, bool LAB>
__device__ __forceinline__ float fwd_tile_update(f32x16 (&acc)[TL::TM][TL::TN], int v0, int V, float (&m)[TL::TN],
                                                 float (&l)[TL::TN], const int (&lpos)[TL::TN],
                                                 const int (&lrow)[TL::TN], float *__restrict__ zlab) {
    const bool full = v0 + TL::BM <= V;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (wave % TL::WM) * TL::kWaveM + 4 * (lane >> 5);  // tile_row = rbase + acc_row_const
    float tmax = kNegInf;
    if (!full) {
        // the last vocabulary tile: rows past V hold copies of row V - 1
        const int lim = row_limit<TL>(V - v0);
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (acc_row_const(tm, r) >= lim) acc[tm][tn][r] = kNegInf;
    }
    // One token column at a time keeps at most TM x 16 values in VGPRs; the
    // scheduling barriers stop the compiler from hoisting every column's
    // accumulator reads to the top (which would spill).
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        __builtin_amdgcn_sched_barrier(0);
        float mx = kNegInf;
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[tm][tn][r]);
        float mxn = mx;
        // The label entry of a token lies in one tile of the vocabulary: only
        // there (and only in the lanes that hold it) is the maximum taken
        // again without it and its logit kept.
        const int lr = LAB ? lpos[tn] - v0 - rbase : -1;  // label row as acc_row_const, if in this lane
        if (LAB && lr >= 0 && lr < TL::TM * 32) {
            mxn = kNegInf;
            float zl = 0.f;
            bool hit = false;
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool il = acc_row_const(tm, r) == lr;
                    mxn = fmaxf(mxn, il ? kNegInf : acc[tm][tn][r]);
                    zl = il ? acc[tm][tn][r] : zl;
                    hit |= il;
                }
            if (hit && lrow[tn] >= 0) zlab[lrow[tn]] = zl;
        }
        tmax = fmaxf(tmax, LAB ? mxn : mx);
        const float mn = fmaxf(m[tn], mx * kLog2e);
        if (mn == kNegInf) continue;
        float sum = 0.f;
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[tm][tn][r], kLog2e, -mn));
        l[tn] = l[tn] * __builtin_amdgcn_exp2f(m[tn] - mn) + sum;
        m[tn] = mn;
    }
    return tmax;
}

// Processing position of the label of each token column this lane holds
// (-2^30 for none: a label out of range), and its row (-1 past the valid
// rows).  Token columns past the valid rows hold a copy of the last valid
// row, and take its label too.
template <class TL>
__device__ __forceinline__ void fwd_label_pos(int (&lpos)[TL::TN], int (&lrow)[TL::TN], int tok0, int nv,
                                              const int32_t *__restrict__ idx, const int64_t *__restrict__ labels,
                                              const int32_t *__restrict__ inv_perm, int V) {
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int t = tok0 + tile_col<TL>(tn);
        const int row = idx[min(t, nv - 1)];
        const int64_t y = labels[row];
        lpos[tn] = (y >= 0 && y < V) ? (inv_perm ? inv_perm[y] : (int)y) : -(1 << 30);
        lrow[tn] = t < nv ? row : -1;
    }
}

// Block-max table: the largest logit other than a label entry of every
// 128 x 128 block of the logit matrix of the valid rows.  A wave of the 256 x 256 tile covers 128
// vocabulary rows x 64 tokens, half of one block; the two waves of a block
// combine with an integer atomic max on the order-preserving encoding.  Lane
// j of each wave keeps the maximum of the j-th tile of a group of 64 and the
// wave writes the group with one vector atomic, so the table costs one memory
// instruction per 64 tiles.
struct BoundSink {
    int *row;   // this wave's block of the table at the segment's first tile (stride 2 per tile); null: no table
    int keep = 0;
    // (Token rows past the valid ones are copies of the last valid row, so a
    // block with some valid rows gets its true maximum; a block with none is
    // left at -inf.)
    template <class TL>
    static __device__ __forceinline__ int *block_of(int *table, int64_t ld, int rt, int t0, int nv) {
        const int wave = threadIdx.x >> 6;
        const int wm = wave % TL::WM, th = (wave / TL::WM) * TL::kWaveN / 128;
        static_assert(TL::kWaveM == 128 && TL::BM == 256 && TL::BN == 256, "a wave covers half of a 128 x 128 block");
        if (!table || (2 * rt + th) * 128 >= nv) return nullptr;
        return table + (int64_t)(2 * rt + th) * ld + 2 * t0 + wm;
    }
    __device__ __forceinline__ void tile(int ct, float lane_max, bool last) {
        if (!row) return;
        const int m = wave_max_i32(bound_enc(lane_max));
        const int lane = threadIdx.x & 63;
        const int j = ct & 63;
        if (lane == j) keep = m;
        if (j == 63 || last) {
            if (lane <= j) atomicMax(row + 2 * (ct - j + lane), keep);
        }
    }
};

// The block-max table's 256-entry chunk c: set to the encoded -inf before
// the logit kernel, decoded to floats after it (workgroups of other kernels'
// launches: no launch of their own).
__device__ __forceinline__ void bound_init_chunk(int *__restrict__ t, int64_t n, int64_t c) {
    const int64_t i = c * 256 + threadIdx.x;
    if (i < n) t[i] = bound_enc(kNegInf);
}
__device__ __forceinline__ void bound_decode_chunk(int *__restrict__ t, int64_t n, int64_t c) {
    const int64_t i = c * 256 + threadIdx.x;
    if (i < n) reinterpret_cast<float *>(t)[i] = bound_dec(t[i]);
}

// Merges (m, l) over the two half-waves and the WM waves that hold the same
// tokens, in a fixed order, and writes the segment's partials for valid
// tokens (slot-major, by token position inside the tile).  Ends with a
// barrier: the LDS is free again when it returns.
template <class TL>
__device__ __forceinline__ void fwd_write_partials(float (&m)[TL::TN], float (&l)[TL::TN], float *red, int tok0,
                                                   int nv, int64_t slot, float *__restrict__ part_m,
                                                   float *__restrict__ part_s) {
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const float mo = __shfl_xor(m[tn], 32, 64);
        const float lo = __shfl_xor(l[tn], 32, 64);
        const float M = fmaxf(m[tn], mo);
        if (M != kNegInf) {
            l[tn] = l[tn] * __builtin_amdgcn_exp2f(m[tn] - M) + lo * __builtin_amdgcn_exp2f(mo - M);
            m[tn] = M;
        }
    }
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % TL::WM;
    if (lane < 32) {
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int c = tile_col<TL>(tn);
            red[(wm * TL::BN + c) * 2 + 0] = m[tn];
            red[(wm * TL::BN + c) * 2 + 1] = l[tn];
        }
    }
    __syncthreads();
    for (int c = tid; c < TL::BN; c += TL::kThreads) {
        const int tok = tok0 + c;
        if (tok >= nv) continue;
        float M = kNegInf;
        for (int w = 0; w < TL::WM; ++w) M = fmaxf(M, red[(w * TL::BN + c) * 2]);
        float L = 0.f;
        if (M != kNegInf)
            for (int w = 0; w < TL::WM; ++w)
                L += red[(w * TL::BN + c) * 2 + 1] * __builtin_amdgcn_exp2f(red[(w * TL::BN + c) * 2] - M);
        part_m[slot * TL::BN + c] = M;
        part_s[slot * TL::BN + c] = L;
    }
    __syncthreads();
}

// One segment on the VGPR-staged pipeline: token tile rt, vocabulary tiles
// [t0, t0 + ntile), partials to slot.
template <typename T, bool LAB>
__device__ __forceinline__ void fwd_segment(const T *__restrict__ H, Rows2<const T> E,
                                            const int32_t *__restrict__ idx, int nv, const int32_t *__restrict__ perm,
                                            const int64_t *__restrict__ labels, const int32_t *__restrict__ inv_perm,
                                            int D, int V, int n_vtiles, int rt, int t0, int ntile, int64_t slot,
                                            u32x4 *lds, float *__restrict__ part_m, float *__restrict__ part_s,
                                            int *__restrict__ tbound, float *__restrict__ zlab) {
    using TL = TileF;
    const int tok0 = rt * TL::BN;
    int lpos[TL::TN], lrow[TL::TN];
    if (LAB) fwd_label_pos<TL>(lpos, lrow, tok0, nv, idx, labels, inv_perm, V);
    const size_t rowb = (size_t)D * sizeof(T);
    const int kvalid = D * (int)sizeof(T);
    const int ns = (kvalid + TL::kStageBytes - 1) / TL::kStageBytes;
    BoundSink bs{BoundSink::block_of<TL>(tbound, 2 * (int64_t)n_vtiles, rt, t0, nv)};

    Engine<T, TL> eng;
#pragma unroll
    for (int j = 0; j < Engine<T, TL>::NB; ++j) {
        const int tok = tok0 + eng.row(j);
        eng.pb[j] = tok < nv ? reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb : nullptr;
    }
    auto set_tile = [&](int vt) {
        const int v0 = vt * TL::BM;
#pragma unroll
        for (int j = 0; j < Engine<T, TL>::NA; ++j) {
            const int pos = v0 + eng.row(j);
            const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
            eng.pa[j] = (v >= 0 && v < V) ? reinterpret_cast<const char *>(E.row(v)) : nullptr;
        }
    };

    float m[TL::TN], l[TL::TN];
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) { m[tn] = kNegInf; l[tn] = 0.f; }
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);

    const int total = ntile * ns;
    if (total > 0) {
        int lt = 0, lk = 0;  // tile / stage of the next load
        set_tile(t0);
        eng.load(0, kvalid);
        eng.store(lds);
        if (++lk == ns) { lk = 0; if (++lt < ntile) set_tile(t0 + lt); }
        __syncthreads();
        int ck = 0, ct = 0;  // stage / tile being computed
        for (int s = 0; s < total; ++s) {
            const bool more = s + 1 < total;
            if (more) eng.load(lk * TL::kStageBytes, kvalid);
            eng.compute(lds + (s & 1) * TL::kStage, acc);
            if (++ck == ns) {
                ck = 0;
                bs.tile(ct, fwd_tile_update<TL, LAB>(acc, (t0 + ct) * TL::BM, V, m, l, lpos, lrow, zlab), ct == ntile - 1);
                ++ct;
                zero_acc<TL>(acc);
            }
            if (more) {
                eng.store(lds + ((s + 1) & 1) * TL::kStage);
                if (++lk == ns) { lk = 0; if (++lt < ntile) set_tile(t0 + lt); }
            }
            __syncthreads();
        }
    }

    fwd_write_partials<TL>(m, l, reinterpret_cast<float *>(lds), tok0, nv, slot, part_m, part_s);
}

// LAB: the block-max table is written (its maxima leave label entries out).
// One kernel per value rather than a branch inside one: with both paths in
// one kernel the scalar registers of the label bookkeeping spilled into the
// tile loop of either path.
template <typename T, bool LAB>
__global__ __launch_bounds__(TileF::kThreads) void k_fwd(
    const T *__restrict__ H, Rows2<const T> E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm, const int64_t *__restrict__ labels,
    const int32_t *__restrict__ inv_perm, int D, int V, int n_vtiles, float *__restrict__ part_m,
    float *__restrict__ part_s, int *__restrict__ tbound, float *__restrict__ zlab, int *__restrict__ grid_rec) {
    __shared__ u32x4 lds[TileF::kLdsChunks];
    const int nv = *nvalid_p;
    if (nv <= 0) return;
    fwd_segments(fwd_grid_record(nv, n_vtiles, gridDim.x, grid_rec), blockIdx.x, [&](int rt, int t0, int ntile, int64_t slot) {
        fwd_segment<T, LAB>(H, E, idx, nv, perm, labels, inv_perm, D, V, n_vtiles, rt, t0, ntile, slot, lds, part_m,
                            part_s, tbound, zlab);
    });
}

// The same computation on the DMA pipeline (DmaEngine): 2 LDS stages of 128
// K-bytes, one in flight while the other is computed.  Rows past the end of
// an operand are clamped to its last row: their logits are finite and masked
// (vocabulary) or never written (tokens).  Needs D * sizeof(T) to be a
// multiple of 128.
template <typename T, class TL, bool LAB>
__device__ __forceinline__ void fwd_segment_dma(const T *__restrict__ H, Rows2<const T> E,
                                                const int32_t *__restrict__ idx, int nv,
                                                const int32_t *__restrict__ perm, const int64_t *__restrict__ labels,
                                                const int32_t *__restrict__ inv_perm, int D, int V, int n_vtiles,
                                                int rt, int t0, int ntile, int64_t slot, u32x4 *lds,
                                                float *__restrict__ part_m, float *__restrict__ part_s,
                                                int *__restrict__ tbound, float *__restrict__ zlab) {
    using DE = DmaEngine<T, TL, kLogitRowBytes, kLogitStages>;
    const int tok0 = rt * TL::BN;
    int lpos[TL::TN], lrow[TL::TN];
    if (LAB) fwd_label_pos<TL>(lpos, lrow, tok0, nv, idx, labels, inv_perm, V);
    const size_t rowb = (size_t)D * sizeof(T);
    const int ns = D * (int)sizeof(T) / DE::kStageBytes;
    BoundSink bs{BoundSink::block_of<TL>(tbound, 2 * (int64_t)n_vtiles, rt, t0, nv)};

    DE eng(lds);
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j);
        const int tok = min(tok0 + r, nv - 1);
        eng.pb[j] = reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb + DE::chunk_off(j, r, threadIdx.x);
    }
    // (Two paths on the uniform perm test: without a permutation no load is
    // issued, so nothing has to wait for the stage in flight.)
    auto set_tile = [&](int vt) {
        if (perm) {
#pragma unroll
            for (int j = 0; j < DE::NIA; ++j) {
                const int r = DE::row_a(j);
                int v = perm[min(vt * TL::BM + r, V - 1)];
                v = (v >= 0 && v < V) ? v : 0;
                eng.pa[j] = reinterpret_cast<const char *>(E.row(v)) + DE::chunk_off(j, r, threadIdx.x);
            }
        } else {
#pragma unroll
            for (int j = 0; j < DE::NIA; ++j) {
                const int r = DE::row_a(j);
                eng.pa[j] = reinterpret_cast<const char *>(E.row(min(vt * TL::BM + r, V - 1))) +
                            DE::chunk_off(j, r, threadIdx.x);
            }
        }
    };

    float m[TL::TN], l[TL::TN];
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) { m[tn] = kNegInf; l[tn] = 0.f; }
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);

    const int total = ntile * ns;
    int lt = 0, lk = 0;  // tile / stage of the next DMA
    if (total > 0) set_tile(t0);
    {
        auto issue_at = [&](int q) {
            eng.issue(q % DE::kStages, lk * DE::kStageBytes);
            if (++lk == ns) { lk = 0; if (++lt < ntile) set_tile(t0 + lt); }
        };
#pragma unroll
        for (int q = 0; q < DE::kDepth; ++q)
            if (q < total) issue_at(q);
        int s = 0;  // global stage counter (the DMA cursor runs kDepth stages ahead, across tiles)
        for (int ct = 0; ct < ntile; ++ct) {
            for (int k = 0; k < ns; ++k, ++s) {
                const int ahead = total - 1 - s;
                eng.wait_stage(eng.clamp_ahead(ahead));
                // The first K-slice's MFMAs go out before the next stage's DMA
                // instructions: every wave reaches this point at once, and
                // issuing the DMA first left the matrix cores idle meanwhile
                // (1-2 % of the kernel).  Same MFMAs in the same order.
                eng.compute(s % DE::kStages, acc, threadIdx.x, 0, 1);
                __builtin_amdgcn_sched_barrier(0);
                if (s + DE::kDepth < total) issue_at(s + DE::kDepth);
                __builtin_amdgcn_sched_barrier(0);
                eng.compute(s % DE::kStages, acc, threadIdx.x, 1, DE::kCpr / 2);
            }
            bs.tile(ct, fwd_tile_update<TL, LAB>(acc, (t0 + ct) * TL::BM, V, m, l, lpos, lrow, zlab), ct == ntile - 1);
            zero_acc<TL>(acc);
        }
    }
    fwd_write_partials<TL>(m, l, reinterpret_cast<float *>(lds), tok0, nv, slot, part_m, part_s);
}

template <typename T, class TL, bool LAB>
__global__ __launch_bounds__(TL::kThreads) void k_fwd_dma(
    const T *__restrict__ H, Rows2<const T> E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm, const int64_t *__restrict__ labels,
    const int32_t *__restrict__ inv_perm, int D, int V, int n_vtiles, float *__restrict__ part_m,
    float *__restrict__ part_s, int *__restrict__ tbound, float *__restrict__ zlab, int *__restrict__ grid_rec) {
    using DE = DmaEngine<T, TL, kLogitRowBytes, kLogitStages>;
    __shared__ u32x4 lds[DE::kLdsChunks];
    const int nv = *nvalid_p;
    if (nv <= 0) return;
    fwd_segments(fwd_grid_record(nv, n_vtiles, gridDim.x, grid_rec), blockIdx.x, [&](int rt, int t0, int ntile, int64_t slot) {
        fwd_segment_dma<T, TL, LAB>(H, E, idx, nv, perm, labels, inv_perm, D, V, n_vtiles, rt, t0, ntile, slot, lds,
                                    part_m, part_s, tbound, zlab);
    });
}

// ------------------------------------- bf16 forward on 4 waves, scheduled K loop
// The same tiles, partition, partials and block-max table as k_fwd_dma, on
// the 4-wave K loop of k4.hpp.

// fwd_tile_update for the 4-wave tile, one token column (64 values) at a
// time; PART: the last vocabulary tile, rows at or past lim (per lane, as
// acc_row_const) count as -inf.  Reads the accumulators only, so at most one
// column's values are live in vector registers.
template <bool LAB, bool PART>
__device__ __forceinline__ float fwd4_columns(const Acc4 &acc, int lim, int v0, float (&m)[4], float (&l)[4],
                                              const int (&lpos)[4], const int (&lrow)[4],
                                              float *__restrict__ zlab) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rbase = (wave & 1) * 128 + 4 * (lane >> 5);
    float tmax = kNegInf;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        __builtin_amdgcn_sched_barrier(0);
        // (lim through an empty asm per column: the compiler would otherwise
        // keep all 64 row masks in scalar registers across the columns.)
        if (PART) asm volatile("" : "+v"(lim));
        float x[4][16];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                x[tm][r] = (PART && acc_row_const(tm, r) >= lim) ? kNegInf : acc_read(acc[tm][tn], r);
        float mx = kNegInf;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[tm][r]);
        float mxn = mx;
        const int lr = LAB ? lpos[tn] - v0 - rbase : -1;
        if (LAB && lr >= 0 && lr < 128) {
            mxn = kNegInf;
            float zl = 0.f;
            bool hit = false;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool il = acc_row_const(tm, r) == lr;
                    mxn = fmaxf(mxn, il ? kNegInf : x[tm][r]);
                    zl = il ? x[tm][r] : zl;
                    hit |= il;
                }
            if (hit && lrow[tn] >= 0) zlab[lrow[tn]] = zl;
        }
        tmax = fmaxf(tmax, LAB ? mxn : mx);
        const float mn = fmaxf(m[tn], mx * kLog2e);
        // Every value at least 64 binary orders below the running maximum:
        // the 64 terms add under 2^-58 of it (and at most 2^-46 of it over a
        // whole vocabulary of 2^18 tiles' worth of rows), below what the fp32
        // sum resolves once it holds the maximum's term; they are left out.
        if (mn == kNegInf || mx * kLog2e < m[tn] - 64.f) continue;
        float sum = 0.f;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(x[tm][r], kLog2e, -mn));
        l[tn] = l[tn] * __builtin_amdgcn_exp2f(m[tn] - mn) + sum;
        m[tn] = mn;
    }
    return tmax;
}

template <bool LAB>
__device__ __forceinline__ void fwd4_segment(const bf16_t *__restrict__ H, Rows2<const bf16_t> E,
                                             const int32_t *__restrict__ idx, int nv,
                                             const int32_t *__restrict__ perm, const int64_t *__restrict__ labels,
                                             const int32_t *__restrict__ inv_perm, int D, int V, int n_vtiles,
                                             int rt, int t0, int ntile, int64_t slot, u32x4 *lds,
                                             float *__restrict__ part_m, float *__restrict__ part_s,
                                             int *__restrict__ tbound, float *__restrict__ zlab,
                                             const float *__restrict__ zy) {
    using TL = Tile4;
    const int tok0 = rt * TL::BN;
    int lpos[TL::TN], lrow[TL::TN];
    if (LAB) fwd_label_pos<TL>(lpos, lrow, tok0, nv, idx, labels, inv_perm, V);
    BoundSink bs{BoundSink::block_of<TL>(tbound, 2 * (int64_t)n_vtiles, rt, t0, nv)};
    // The running maximum of each token starts at its label logit (log2
    // units): a value of the row, so the online sum stays exact, and on a
    // peaked row it lets the tiles far below the label skip their
    // exponentials from the segment's first tile on.
    float m[TL::TN], l[TL::TN];
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const float z = zy[min(tok0 + tile_col<TL>(tn), nv - 1)];
        m[tn] = __builtin_isfinite(z) ? z * kLog2e : kNegInf;
        l[tn] = 0.f;
    }
    k4_run(H, E, idx, nv, perm, D, V, tok0, t0, ntile, lds, [&](int ct, Acc4 &acc) {
        const int v0 = (t0 + ct) * TL::BM;
        const float tmax = v0 + TL::BM <= V
                               ? fwd4_columns<LAB, false>(acc, 0, v0, m, l, lpos, lrow, zlab)
                               : fwd4_columns<LAB, true>(acc, row_limit<TL>(V - v0), v0, m, l, lpos, lrow, zlab);
        bs.tile(ct, tmax, ct == ntile - 1);
    });
    fwd_write_partials<TL>(m, l, reinterpret_cast<float *>(lds), tok0, nv, slot, part_m, part_s);
}

template <bool LAB>
__global__ __launch_bounds__(Tile4::kThreads) void k_fwd4(
    const bf16_t *__restrict__ H, Rows2<const bf16_t> E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm, const int64_t *__restrict__ labels,
    const int32_t *__restrict__ inv_perm, int D, int V, int n_vtiles, float *__restrict__ part_m,
    float *__restrict__ part_s, int *__restrict__ tbound, float *__restrict__ zlab, const float *__restrict__ zy,
    int *__restrict__ grid_rec) {
    __shared__ u32x4 lds[4 * 2 * kTileVocab * 4];  // 4 buffers of 256 A + 256 B rows of 64 bytes
    const int nv = *nvalid_p;
    if (nv <= 0) return;
    fwd_segments(fwd_grid_record(nv, n_vtiles, gridDim.x, grid_rec), blockIdx.x, [&](int rt, int t0, int ntile, int64_t slot) {
        fwd4_segment<LAB>(H, E, idx, nv, perm, labels, inv_perm, D, V, n_vtiles, rt, t0, ntile, slot, lds, part_m,
                          part_s, tbound, zlab, zy);
    });
}

// ------------------------------------------------------------ label gather
// One wave per compacted position w < nv: zy[w] = <h_i, e_{y_i}> for row
// i = idx[w] (fp32 accumulation of exact products; the indexed matmul), or
// -inf where the label is out of range.  The 4-wave forward starts each
// token's running maximum there, and the merge takes the loss from it.
// Workgroups from dot_groups on set the block-max table to -inf instead.
template <typename T>
__global__ __launch_bounds__(256) void k_label_dot(const T *__restrict__ H, Rows2<const T> E,
                                                   const int64_t *__restrict__ labels,
                                                   const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ nvalid_p, int D, int64_t V,
                                                   float *__restrict__ zy, int64_t dot_groups, int *__restrict__ tb,
                                                   int64_t nb) {
    if ((int64_t)blockIdx.x >= dot_groups) {  // (uniform)
        bound_init_chunk(tb, nb, (int64_t)blockIdx.x - dot_groups);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= *nvalid_p) return;
    const int64_t i = idx[w];
    const int64_t y = labels[i];
    if (y < 0 || y >= V) {
        if (lane == 0) zy[w] = kNegInf;
        return;
    }
    constexpr int CE = ChunkElems<T>::value;
    const char *h = reinterpret_cast<const char *>(H + i * (int64_t)D);
    const char *e = reinterpret_cast<const char *>(E.row(y));
    // (the loads of up to kU chunks per lane are issued before the first is
    // used; the products are still added chunk by chunk in feature order)
    constexpr int kU = 8;
    float dot = 0.f;
    for (int k0 = lane * CE; k0 < D; k0 += kU * 64 * CE) {
        u32x4 hv[kU], ev[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int k = k0 + u * 64 * CE;
            if (k < D) {
                hv[u] = ld16(h + k * sizeof(T));
                ev[u] = ld16(e + k * sizeof(T));
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (k0 + u * 64 * CE < D) {
                const T *hp = reinterpret_cast<const T *>(&hv[u]);
                const T *ep = reinterpret_cast<const T *>(&ev[u]);
#pragma unroll
                for (int q = 0; q < CE; ++q) dot += to_f32(hp[q]) * to_f32(ep[q]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
    if (lane == 0) zy[w] = dot;
}

// ------------------------------------------------------------------ merge
// One thread per position w: it zeroes row w if that row is ignored, and if
// w < nv it finishes the valid row at compacted position w.  A workgroup is
// one token tile, so the partial of vocabulary range j is one coalesced
// 1 KB row of the partial buffers for the whole workgroup.  The max and the
// scaled sum run over the ranges in vocabulary order, so the result depends
// only on the partition, never on scheduling.  Workgroups from merge_groups
// on decode the block-max table.
__global__ __launch_bounds__(kTileRows) void k_merge(const int64_t *__restrict__ labels,
                                                     const int32_t *__restrict__ idx,
                                                     const int32_t *__restrict__ nvalid_p,
                                                     const float *__restrict__ part_m,
                                                     const float *__restrict__ part_s, const float *__restrict__ zy,
                                                     const int *__restrict__ grid_rec, int G, int n_vtiles,
                                                     int64_t N, int64_t V, int64_t ignore_index,
                                                     float *__restrict__ loss, float *__restrict__ lse,
                                                     int64_t merge_groups, int *__restrict__ tb, int64_t nb) {
    if ((int64_t)blockIdx.x >= merge_groups) {  // (uniform)
        bound_decode_chunk(tb, nb, (int64_t)blockIdx.x - merge_groups);
        return;
    }
    __shared__ int seg_on[kFwdRanges];  // range j has a segment (is not empty)
    const int rt = blockIdx.x, c = threadIdx.x;
    const int nv = *nvalid_p;
    const FwdGrid g = fwd_grid_recorded(nv, n_vtiles, G, grid_rec);
    const int b = g.b();  // at most kFwdRanges
    if (c < kFwdRanges) seg_on[c] = c < b && g.vt0(c + 1) > g.vt0(c);
    __syncthreads();
    const int64_t w = (int64_t)rt * kTileRows + c;
    if (w >= N) return;
    if (labels[w] == ignore_index) { loss[w] = 0.f; lse[w] = 0.f; }
    if (w >= nv) return;
    const int64_t i = idx[w];
    const int64_t y = labels[i];
    if (y < 0 || y >= V) {  // not a valid label: undefined by contract; flag it, touch nothing
        loss[i] = __builtin_nanf("");
        lse[i] = __builtin_nanf("");
        return;
    }
    const int64_t base = (int64_t)rt * b * kTileRows + c;
    float pm[kFwdRanges], ps[kFwdRanges];
    float M = kNegInf;
#pragma unroll
    for (int j = 0; j < kFwdRanges; ++j) {
        const bool seg = seg_on[j];
        pm[j] = seg ? part_m[base + (int64_t)j * kTileRows] : kNegInf;
        ps[j] = seg ? part_s[base + (int64_t)j * kTileRows] : 0.f;
        M = fmaxf(M, pm[j]);
    }
    float S = 0.f;
#pragma unroll
    for (int j = 0; j < kFwdRanges; ++j)
        if (pm[j] != kNegInf) S += ps[j] * __builtin_amdgcn_exp2f(pm[j] - M);
    const float l = (M + log2f(S)) * kLn2;
    lse[i] = l;
    loss[i] = l - zy[w];  // zy[w] = z_{i, y_i}
}

// ------------------------------------------------- allocation-free forward
// The workspace of cce_forward_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  In host code
// the array's name is only a stand-in symbol, never a device address: the
// first call on a device (with that device current) looks up its address
// with hipGetSymbolAddress, and every later call on that device uses the
// cached address.  The forward needs nothing in it to start at zero (every
// region is written before it is read), and calls that overlap on one GPU
// share it, so they race.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------- launchers
FwdShape fwd_shape(int64_t N, int64_t D, int64_t V) {
    FwdShape s;
    s.N = N;
    s.D = D;
    s.V = V;
    s.n_vtiles = (int)ceil_div(V, kTileVocab);
    s.n_rtiles = (int)ceil_div(N, kTileRows);
    return s;
}

FwdWs fwd_ws(void *ws, const FwdShape &s, size_t *bytes) {
    Carver c(ws);
    FwdWs w;
    w.idx = c.take<int32_t>(s.N);
    w.nvalid = c.take<int32_t>(1);
    w.inv_perm = c.take<int32_t>(s.V);
    // slots rt b + j < n_rtiles kFwdRanges, one partial per token of the tile each
    w.part_m = c.take<float>((size_t)s.n_rtiles * kFwdRanges * kTileRows);
    w.part_s = c.take<float>((size_t)s.n_rtiles * kFwdRanges * kTileRows);
    w.zy = c.take<float>(s.N);
    w.grid = c.take<int32_t>(4);
    if (bytes) *bytes = c.off;
    return w;
}

hipError_t launch_compact(const int64_t *labels, int64_t N, int64_t ignore_index, int32_t *idx,
                          int32_t *nvalid, hipStream_t st) {
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, labels, N, ignore_index, idx, nvalid);
    return hipGetLastError();
}

hipError_t launch_inv_perm(const int32_t *perm, int V, int32_t *inv, hipStream_t st) {
    hipLaunchKernelGGL(k_inv_perm, dim3((unsigned)ceil_div(V, 256)), dim3(256), 0, st, perm, V, inv);
    return hipGetLastError();
}

hipError_t launch_seg_labels(const int64_t *labels, int64_t N, int64_t ignore_index, int64_t V0, int64_t off1,
                             int64_t V1, int64_t *out, hipStream_t st) {
    hipLaunchKernelGGL(k_seg_labels, dim3((unsigned)ceil_div(N, 256)), dim3(256), 0, st, labels, N, ignore_index,
                       V0, off1, V1, out);
    return hipGetLastError();
}

hipError_t launch_check_labels(const int64_t *labels, int64_t N, int64_t V, int64_t ignore_index,
                               int64_t *n_bad, hipStream_t st) {
    hipLaunchKernelGGL(k_check_labels, dim3(1), dim3(1024), 0, st, labels, N, V, ignore_index, n_bad);
    return hipGetLastError();
}

template <typename T>
static hipError_t forward_t(const T *H, Rows2<const T> E, const int64_t *labels, const FwdShape &s,
                            int64_t ignore_index, const int32_t *perm, const FwdWs &w, float *loss, float *lse,
                            float *block_max, hipStream_t st) {
    hipError_t e = launch_compact(labels, s.N, ignore_index, w.idx, w.nvalid, st);
    if (e != hipSuccess) return e;
    int *tb = reinterpret_cast<int *>(block_max);
    const int64_t nb = 4 * (int64_t)s.n_rtiles * s.n_vtiles;
    const int64_t nb_groups = tb ? ceil_div(nb, 256) : 0;  // table chunks (set to -inf, later decoded)
    const int64_t dot_groups = ceil_div(s.N, 4);
    hipLaunchKernelGGL(k_label_dot<T>, dim3((unsigned)(dot_groups + nb_groups)), dim3(256), 0, st, H, E, labels,
                       w.idx, w.nvalid, (int)s.D, s.V, w.zy, dot_groups, tb, nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int32_t *invp = nullptr;  // label positions in the processing order, for the table
    float *zl = tb ? block_max + nb : nullptr;  // the table's second part: label logits by row
    if (tb) {
        if (perm) {
            if ((e = launch_inv_perm(perm, (int)s.V, w.inv_perm, st)) != hipSuccess) return e;
            invp = w.inv_perm;
        }
    }
    // A persistent grid: as many workgroups as are resident at once (every
    // one gets the same share of tiles), at most one per tile.
    const bool dma = (s.D * (int64_t)sizeof(T)) % kLogitRowBytes == 0;
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    constexpr bool bf16 = std::is_same<T, bf16_t>::value;
    const bool four = CCE_K4 && bf16 && dma;
    if constexpr (bf16) {
        if (four)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tb ? k_fwd4<true> : k_fwd4<false>,
                                                             Tile4::kThreads, 0);
    }
    if (four)
        ;
    else if (dma && tb)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fwd_dma<T, TileFD, true>, TileFD::kThreads, 0);
    else if (dma)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fwd_dma<T, TileFD, false>, TileFD::kThreads, 0);
    else if (tb)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fwd<T, true>, TileF::kThreads, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fwd<T, false>, TileF::kThreads, 0);
    if (e != hipSuccess) return e;
    int64_t G = (int64_t)std::max(cus, 1) * std::max(per_cu, 1);
    G = std::min<int64_t>(std::min<int64_t>(G, kFwdMaxGroups), (int64_t)s.n_rtiles * s.n_vtiles);
    if (G >= 8) G &= ~7;  // lets the placement give each XCD a contiguous eighth
    const dim3 grid((unsigned)G);
    if constexpr (bf16) {
        if (four) {
            if (tb)
                hipLaunchKernelGGL(k_fwd4<true>, grid, dim3(Tile4::kThreads), 0, st, H, E, w.idx, w.nvalid, perm,
                                   labels, invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.zy, w.grid);
            else
                hipLaunchKernelGGL(k_fwd4<false>, grid, dim3(Tile4::kThreads), 0, st, H, E, w.idx, w.nvalid, perm,
                                   labels, invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.zy, w.grid);
        }
    }
    if (four)
        ;
    else if (dma && tb)
        hipLaunchKernelGGL((k_fwd_dma<T, TileFD, true>), grid, dim3(TileFD::kThreads), 0, st, H, E, w.idx, w.nvalid,
                           perm, labels, invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.grid);
    else if (dma)
        hipLaunchKernelGGL((k_fwd_dma<T, TileFD, false>), grid, dim3(TileFD::kThreads), 0, st, H, E, w.idx, w.nvalid,
                           perm, labels, invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.grid);
    else if (tb)
        hipLaunchKernelGGL((k_fwd<T, true>), grid, dim3(TileF::kThreads), 0, st, H, E, w.idx, w.nvalid, perm, labels,
                           invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.grid);
    else
        hipLaunchKernelGGL((k_fwd<T, false>), grid, dim3(TileF::kThreads), 0, st, H, E, w.idx, w.nvalid, perm, labels,
                           invp, (int)s.D, (int)s.V, s.n_vtiles, w.part_m, w.part_s, tb, zl, w.grid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t merge_groups = ceil_div(s.N, kTileRows);
    hipLaunchKernelGGL(k_merge, dim3((unsigned)(merge_groups + nb_groups)), dim3(kTileRows), 0, st, labels, w.idx,
                       w.nvalid, w.part_m, w.part_s, w.zy, w.grid, (int)G, s.n_vtiles, s.N, s.V, ignore_index, loss, lse,
                       merge_groups, tb, nb);
    return hipGetLastError();
}

template <typename T>
static Rows2<const T> rows_of(const VocabRows &E, int64_t D) {
    return Rows2<const T>{static_cast<const T *>(E.e0), static_cast<const T *>(E.e1), E.v0, D};
}

hipError_t launch_forward(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels,
                          const FwdShape &s, int64_t ignore_index, const int32_t *perm, const FwdWs &w,
                          float *loss, float *lse, float *block_max, hipStream_t st) {
    if (dt == CCE_BF16)
        return forward_t<bf16_t>(static_cast<const bf16_t *>(H), rows_of<bf16_t>(E, s.D), labels, s, ignore_index,
                                 perm, w, loss, lse, block_max, st);
    return forward_t<float>(static_cast<const float *>(H), rows_of<float>(E, s.D), labels, s, ignore_index, perm, w,
                            loss, lse, block_max, st);
}

}  // namespace cce
