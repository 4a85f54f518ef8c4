// Backward of the fused classifier-head + cross-entropy on gfx950.
//
// The backward recomputes the logits blockwise from H and E (no logits are
// kept from the forward), skips blocks whose softmax entries all fall below a
// threshold, and accumulates the classifier gradient with Kahan compensation
// (CCE paper summary "Cut Your Losses in Large-Vocabulary Language Models",
// sections "Approach" and "Limitations"; lit note "The loss and the mask: Cut
// Cross-Entropy + FlexAttention", section "Contribution").
//
// Layout of the work.  D (2048-4096 for the heads of interest) is far wider
// than an attention head, so dH_i and dE_v rows cannot live on chip while the
// other dimension is swept.  The vocabulary is therefore processed in chunks
// of at most kChunkVocab columns:
//
//   k_bwd_g   recompute the logit tile (MFMA, same code and K order as the
//             forward), p = exp(z - lse), block filter, and for surviving
//             blocks the gradient tile G = dloss (p - onehot) rounded to the
//             input dtype, written into a [rows x chunk] slice in two layouts
//   k_de      dE_v = sum over surviving row blocks of G^T H (MFMA), Kahan-
//             compensated across row blocks, written once in the output dtype
//   k_dh      dH_i += sum over surviving vocabulary blocks of G E (MFMA), fp32
//             accumulators carried across chunks, output dtype on the last
//
// The slice costs 2 bytes per logit to write and 4 to read back, against
// about 8 D flops per logit, and its size is bounded (rows x kChunkVocab), so
// extra memory is linear in N and V and never rows x vocabulary.
#include <math.h>

#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {

using TileF = Tile<kTileVocab, kTileRows, 2, 4>;   // logit tile: A = vocabulary, B = tokens; 8 waves
using TileFD = TileF;                             // tile of the DMA recompute
using TileG = Tile<128, 256, 2, 4>;               // dE / dH tile: A = a 128-row gradient block, B = 256 features
static_assert(TileG::BM == kBlockVocab && TileG::BM == kBlockRows, "gradient GEMM rows = one filter block");

// ------------------------------------------------------------ small kernels
__global__ void k_inv_perm(const int32_t *__restrict__ perm, int V, int32_t *__restrict__ inv) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < V) {
        const int v = perm[k];
        if (v >= 0 && v < V) inv[v] = k;
    }
}

__global__ void k_stats_init(int64_t *stats) {
    if (threadIdx.x < 5) stats[threadIdx.x] = 0;
}

// lmin[rt] = smallest lse over the valid tokens of token tile rt (+inf if none).
__global__ __launch_bounds__(256) void k_lse_min(const float *__restrict__ lse, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ nvalid_p, float *__restrict__ lmin) {
    __shared__ float part[4];
    const int tok = blockIdx.x * kTileRows + threadIdx.x;
    float v = tok < *nvalid_p ? lse[idx[tok]] : __builtin_huge_valf();
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) lmin[blockIdx.x] = fminf(fminf(part[0], part[1]), fminf(part[2], part[3]));
}

// True when every p in logit tile (rt, vocabulary tile vt) is provably below
// eps / 2: the tile's largest logit T minus the smallest lse L of its tokens
// is below thr = ln(eps / 2), with a relative margin for fp32 rounding of the
// recomputed logits and of T - L.  The filter then keeps nothing of the
// tile's softmax part, so its recompute can be left out without changing a
// bit of the result.  NaN never skips.
__device__ __forceinline__ bool tile_below(const float *__restrict__ tbound, int64_t tb_ld, const float *__restrict__ lmin,
                                           float thr, int rt, int vt) {
    if (!tbound) return false;
    const float T = tbound[(int64_t)rt * tb_ld + vt];
    const float L = lmin[rt];
    return (T - L) + 0x1p-10f * (fabsf(T) + fabsf(L)) < thr;
}

__global__ void k_stats_fin(int64_t *stats, const int32_t *__restrict__ nvalid_p, int64_t n_vtiles) {
    if (threadIdx.x == 0) {
        const int64_t nv = *nvalid_p;
        stats[2] = ((nv + kBlockRows - 1) / kBlockRows) * n_vtiles;
        stats[3] = nv;
    }
}

// dst[c][j] = src[row(j)][c] for c < cols, j < n_out; rows j >= n_rows give 0.
// row(j) = rowmap ? rowmap[row0 + j] : row0 + j.  64 x 64 tiles through LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T *__restrict__ src, int64_t ld_src, int64_t n_src_rows,
                                                   const int32_t *__restrict__ rowmap, int64_t row0,
                                                   const int32_t *__restrict__ n_rows_dev, int n_rows_host,
                                                   int cols, int n_out, T *__restrict__ dst, int64_t ld_dst) {
    constexpr int CE = ChunkElems<T>::value;
    __shared__ T tile[64][64 + 2];
    const int n_rows = n_rows_dev ? *n_rows_dev : n_rows_host;
    const int j0 = blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    // load: 64 rows x (64 / CE) chunks
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
    // store: 64 output rows (features c) x (64 / CE) chunks of j
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

// Rows whose label is ignore_index get dH = 0 (one wave per row).
template <typename T>
__global__ __launch_bounds__(256) void k_zero_ignored(const int64_t *__restrict__ labels, int64_t N, int D,
                                                      int64_t ignore_index, T *__restrict__ dH) {
    constexpr int CE = ChunkElems<T>::value;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= N || labels[i] != ignore_index) return;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int k = (threadIdx.x & 63) * CE; k < D; k += 64 * CE)
        *reinterpret_cast<u32x4 *>(dH + i * D + k) = z;
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

// Epilogue of the recompute: p = exp(z - lse) per entry, the status of this
// wave's 128 x 128 filter block (1 = some p >= eps, 2 = only a label in it,
// 0 = skipped), then for kept blocks the gradient entries
// g = dloss (p [status 1] - [v == y]) in both slice layouts.
template <typename T, class TL>
__device__ __forceinline__ void bwd_g_epilogue(f32x16 (&acc)[TL::TM][TL::TN], int tok0, int nv, int p0, int V,
                                               int ct, int rt, int live_ld, float eps,
                                               const int32_t *__restrict__ idx, const int32_t *__restrict__ perm,
                                               const int32_t *__restrict__ inv_perm,
                                               const int64_t *__restrict__ labels, const float *__restrict__ lse,
                                               const float *__restrict__ dloss, T *__restrict__ Gt, int64_t ldt,
                                               T *__restrict__ Gn, int64_t ldn, uint8_t *__restrict__ live,
                                               int64_t *__restrict__ stats, int *qflag, bool no_softmax) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % TL::WM, wn = wave / TL::WM;
    const int quad = wm * 2 + ((wn * TL::kWaveN) >> 7);  // this wave's 128 x 128 filter block
    float lse_t[TL::TN], dl_t[TL::TN];
    int lab_t[TL::TN];
    bool tok_ok[TL::TN];
    bool any_live = false, any_label = false;
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int tok = tok0 + tile_col<TL>(tn);
        tok_ok[tn] = tok < nv;
        lse_t[tn] = 0.f;
        dl_t[tn] = 0.f;
        lab_t[tn] = -1;
        if (tok_ok[tn]) {
            const int64_t row = idx[tok];
            lse_t[tn] = lse[row];
            dl_t[tn] = dloss[row];
            const int64_t y = labels[row];
            const bool y_ok = y >= 0 && y < V;  // other labels are undefined by contract
            const int ypos = y_ok ? (perm ? inv_perm[y] : (int)y) : -(1 << 30);
            const int lr = ypos - p0 - wm * TL::kWaveM;  // row within this wave's 128 vocabulary rows
            lab_t[tn] = (lr >= 0 && lr < TL::kWaveM) ? ypos - p0 : -1;
            any_label |= lab_t[tn] >= 0;
        }
    }
    const int vlim = row_limit<TL>(V - p0);  // entry (tm, r) is a real vocabulary row iff acc_row_const < vlim
    if (!no_softmax) {
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool ok = tok_ok[tn] && (acc_row_const(tm, r) < vlim);
                    const float p = ok ? __builtin_amdgcn_exp2f((acc[tm][tn][r] - lse_t[tn]) * kLog2e) : 0.f;
                    acc[tm][tn][r] = p;
                    any_live |= ok && (p >= eps);
                }
    }
    const uint64_t bl = __ballot(any_live), bb = __ballot(any_label);
    if (lane == 0 && (bl | bb)) atomicOr(&qflag[quad], (bl ? 1 : 0) | (bb ? 2 : 0));
    __syncthreads();
    if (tid < 4) {
        const int f = qflag[tid];
        const int st = (f & 1) ? 1 : ((f & 2) ? 2 : 0);
        const int rb = 2 * rt + (tid & 1), cb = 2 * ct + (tid >> 1);
        live[(int64_t)rb * live_ld + cb] = (uint8_t)st;
        if (stats && st) atomicAdd(reinterpret_cast<unsigned long long *>(stats + (st == 1 ? 0 : 1)), 1ull);
        // filter blocks whose logits were recomputed (real rows and vocabulary entries only)
        if (stats && !no_softmax && rb * kBlockRows < nv && p0 + (tid >> 1) * kBlockVocab < V)
            atomicAdd(reinterpret_cast<unsigned long long *>(stats + 4), 1ull);
    }
    const int qf = qflag[quad];
    const int status = (qf & 1) ? 1 : ((qf & 2) ? 2 : 0);
    if (status == 0) return;  // wave-uniform

#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int64_t tok = tok0 + tile_col<TL>(tn);
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                T g4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = r4 * 4 + q;
                    const int rl = tile_row<TL>(tm, r);
                    const bool ok = tok_ok[tn] && (acc_row_const(tm, r) < vlim);
                    const float pk = status == 1 ? acc[tm][tn][r] : 0.f;
                    const float g = ok ? dl_t[tn] * (pk - (rl == lab_t[tn] ? 1.f : 0.f)) : 0.f;
                    g4[q] = from_f32<T>(g);
                    Gt[(int64_t)(ct * TL::BM + rl) * ldt + tok] = g4[q];
                }
                // rows r4*4 .. r4*4+3 are consecutive vocabulary entries
                T *dst = Gn + tok * ldn + ct * TL::BM + tile_row<TL>(tm, r4 * 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = g4[q];
            }
    }
}

// ------------------------------------------- recompute + filter + G tile
// Workgroup (256-entry vocabulary tile ct of the chunk, 256-token tile rt).
// The logit tile is recomputed with the forward's code and K order, then
// p = exp(z - lse).  Each 128 x 128 quadrant is a filter block with status
// 1 = some p >= eps (softmax part kept), 2 = no p >= eps but a label falls in
// it (only the -dloss one-hot entries are kept), 0 = skipped.
template <typename T>
__global__ __launch_bounds__(TileF::kThreads) void k_bwd_g(
    const T *__restrict__ H, const T *__restrict__ E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ inv_perm, const int64_t *__restrict__ labels,
    const float *__restrict__ lse, const float *__restrict__ dloss, int D, int V, int chunk_v0, int n_ct,
    int live_ld, float eps, T *__restrict__ Gt, int64_t ldt, T *__restrict__ Gn, int64_t ldn,
    uint8_t *__restrict__ live, int64_t *__restrict__ stats, const float *__restrict__ tbound, int64_t tb_ld,
    const float *__restrict__ lmin, float thr) {
    using TL = TileF;
    __shared__ u32x4 lds[TL::kLdsChunks];
    __shared__ int qflag[4];  // bit 0: some p >= eps, bit 1: a label in the block
    const int nv = *nvalid_p;
    const int ct = blockIdx.x % n_ct;
    const int rt = blockIdx.x / n_ct;
    const int tok0 = rt * TL::BN;
    if (tok0 >= nv) return;
    const int p0 = chunk_v0 + ct * TL::BM;  // first vocabulary position (processing order)
    const int tid = threadIdx.x;
    const size_t rowb = (size_t)D * sizeof(T);
    const int kvalid = D * (int)sizeof(T);
    const int ns = (kvalid + TL::kStageBytes - 1) / TL::kStageBytes;
    if (tid < 4) qflag[tid] = 0;
    const bool skip = tile_below(tbound, tb_ld, lmin, thr, rt, p0 / kTileVocab);
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    if (skip) {
        __syncthreads();
        bwd_g_epilogue<T, TL>(acc, tok0, nv, p0, V, ct, rt, live_ld, eps, idx, perm, inv_perm, labels, lse, dloss,
                              Gt, ldt, Gn, ldn, live, stats, qflag, true);
        return;
    }

    Engine<T, TL> eng;
#pragma unroll
    for (int j = 0; j < Engine<T, TL>::NA; ++j) {
        const int pos = p0 + eng.row(j);
        const int vid = pos < V ? (perm ? perm[pos] : pos) : -1;
        eng.pa[j] = (vid >= 0 && vid < V) ? reinterpret_cast<const char *>(E) + (size_t)vid * rowb : nullptr;
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

    bwd_g_epilogue<T, TL>(acc, tok0, nv, p0, V, ct, rt, live_ld, eps, idx, perm, inv_perm, labels, lse, dloss, Gt,
                          ldt, Gn, ldn, live, stats, qflag, false);
}

// The recompute on the DMA pipeline (needs D * sizeof(T) % 64 == 0).  Rows
// past the end of an operand are clamped to a valid row: their logits are
// finite and the epilogue masks them.
template <typename T, class TL>
__global__ __launch_bounds__(TL::kThreads) void k_bwd_g_dma(
    const T *__restrict__ H, const T *__restrict__ E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ inv_perm, const int64_t *__restrict__ labels,
    const float *__restrict__ lse, const float *__restrict__ dloss, int D, int V, int chunk_v0, int n_ct,
    int live_ld, float eps, T *__restrict__ Gt, int64_t ldt, T *__restrict__ Gn, int64_t ldn,
    uint8_t *__restrict__ live, int64_t *__restrict__ stats, const float *__restrict__ tbound, int64_t tb_ld,
    const float *__restrict__ lmin, float thr) {
    using DE = DmaEngine<T, TL, kLogitRowBytes, kLogitStages>;
    __shared__ u32x4 lds[DE::kLdsChunks];
    __shared__ int qflag[4];
    const int nv = *nvalid_p;
    const int ct = blockIdx.x % n_ct;
    const int rt = blockIdx.x / n_ct;
    const int tok0 = rt * TL::BN;
    if (tok0 >= nv) return;
    const int p0 = chunk_v0 + ct * TL::BM;
    const size_t rowb = (size_t)D * sizeof(T);
    const int ns = D * (int)sizeof(T) / DE::kStageBytes;
    if (threadIdx.x < 4) qflag[threadIdx.x] = 0;
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    if (tile_below(tbound, tb_ld, lmin, thr, rt, p0 / kTileVocab)) {
        __syncthreads();
        bwd_g_epilogue<T, TL>(acc, tok0, nv, p0, V, ct, rt, live_ld, eps, idx, perm, inv_perm, labels, lse, dloss,
                              Gt, ldt, Gn, ldn, live, stats, qflag, true);
        return;
    }

    DE eng(lds);
#pragma unroll
    for (int j = 0; j < DE::NIA; ++j) {
        const int r = DE::row_a(j);
        const int pos = min(p0 + r, V - 1);
        int vid = perm ? perm[pos] : pos;
        vid = (vid >= 0 && vid < V) ? vid : 0;
        eng.pa[j] = reinterpret_cast<const char *>(E) + (size_t)vid * rowb + DE::chunk_off(r);
    }
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j);
        const int tok = min(tok0 + r, nv - 1);
        eng.pb[j] = reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb + DE::chunk_off(r);
    }
    {
#pragma unroll
        for (int q = 0; q < DE::kDepth; ++q)
            if (q < ns) eng.issue(q, q * DE::kStageBytes);
        for (int s = 0; s < ns; ++s) {
            const int ahead = ns - 1 - s;
            eng.wait_stage(eng.clamp_ahead(ahead));
            if (s + DE::kDepth < ns) eng.issue((s + DE::kDepth) % DE::kStages, (s + DE::kDepth) * DE::kStageBytes);
            eng.compute(s % DE::kStages, acc);
        }
    }
    __syncthreads();
    bwd_g_epilogue<T, TL>(acc, tok0, nv, p0, V, ct, rt, live_ld, eps, idx, perm, inv_perm, labels, lse, dloss, Gt,
                          ldt, Gn, ldn, live, stats, qflag, false);
}

// ------------------------------------------------------------- dE (Kahan)
// Workgroup (128-entry vocabulary block cb of the chunk, 256-feature tile).
// K runs over the valid tokens of the row blocks kept for this vocabulary
// block (DMA pipeline, 64 K-bytes per stage).  Each row block's product is
// formed in a fresh fp32 MFMA accumulator and then added into
// (sum, compensation) with Kahan's rule; the result is written once.
constexpr int kListCap = 512;

template <typename T, bool KAHAN>
__global__ __launch_bounds__(TileG::kThreads) void k_de(
    const T *__restrict__ Gt, int64_t ldt, const T *__restrict__ Ht, int64_t ldh,
    const uint8_t *__restrict__ live, int live_ld, const int32_t *__restrict__ nvalid_p,
    const int32_t *__restrict__ perm, int n_cb, int D, int V, int chunk_v0, T *__restrict__ dE) {
    using TL = TileG;
    using DE = DmaEngine<T, TL>;
    __shared__ u32x4 lds[DE::kLdsChunks];
    __shared__ int list[kListCap];
    __shared__ int wcnt[TL::kWaves];
    const int nv = *nvalid_p;
    const int n_rb = (nv + kBlockRows - 1) / kBlockRows;
    const int cb = blockIdx.x % n_cb;
    const int d0 = (blockIdx.x / n_cb) * TL::BN;
    constexpr int kBlockBytes = kBlockRows * (int)sizeof(T);
    constexpr int kSpb = kBlockBytes / DE::kStageBytes;  // stages per row block

    DE eng(lds);
#pragma unroll
    for (int j = 0; j < DE::NIA; ++j) {
        const int r = DE::row_a(j);
        eng.pa[j] = reinterpret_cast<const char *>(Gt + (int64_t)(cb * TL::BM + r) * ldt) + DE::chunk_off(r);
    }
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j);
        const int d = min(d0 + r, D - 1);
        eng.pb[j] = reinterpret_cast<const char *>(Ht + (int64_t)d * ldh) + DE::chunk_off(r);
    }

    f32x16 acc[TL::TM][TL::TN], sum[TL::TM][TL::TN], comp[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    zero_acc<TL>(sum);
    zero_acc<TL>(comp);

    for (int base = 0; base < n_rb; base += kListCap) {
        const int cnt = n_rb - base < kListCap ? n_rb - base : kListCap;
        const int n = build_list<TL::kThreads>(
            cnt, [&](int i) { return live[(int64_t)(base + i) * live_ld + cb] != 0; }, list, wcnt);
        const int total = n * kSpb;
        auto kb = [&](int q) { return (base + list[q / kSpb]) * kBlockBytes + (q % kSpb) * DE::kStageBytes; };
#pragma unroll
        for (int q = 0; q < DE::kDepth; ++q)
            if (q < total) eng.issue(q, kb(q));
        for (int s = 0; s < total; ++s) {
            const int ahead = total - 1 - s;
            eng.wait_stage(eng.clamp_ahead(ahead));
            if (s + DE::kDepth < total) eng.issue((s + DE::kDepth) % DE::kStages, kb(s + DE::kDepth));
            eng.compute(s % DE::kStages, acc);
            if (KAHAN && (s % kSpb) == kSpb - 1) {
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
        __syncthreads();  // list[] and the LDS stages are reused by the next batch
    }

    int vid[TL::TM][16];  // output row of each accumulator row (-1: none), loaded once
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int pos = chunk_v0 + cb * TL::BM + tile_row<TL>(tm, r);
            const int v = pos < V ? (perm ? perm[pos] : pos) : -1;
            vid[tm][r] = (v >= 0 && v < V) ? v : -1;
        }
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int d = d0 + tile_col<TL>(tn);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float val = KAHAN ? sum[tm][tn][r] - comp[tm][tn][r] : acc[tm][tn][r];
                if (vid[tm][r] >= 0 && d < D) dE[(int64_t)vid[tm][r] * D + d] = from_f32<T>(val);
            }
        }
}

// ------------------------------------------------------------------- dH
// Workgroup (128-token block rb, 256-feature tile).  K runs over the kept
// vocabulary blocks of the chunk.  With one chunk the result is written to dH
// directly.  Otherwise fp32 partial sums are added into dh_acc (zeroed before
// the first chunk) and a row block with no kept block in this chunk returns
// at once; k_dh_final converts dh_acc after the last chunk.
template <typename T>
__global__ __launch_bounds__(TileG::kThreads) void k_dh(
    const T *__restrict__ Gn, int64_t ldn, const T *__restrict__ Et, int64_t lde,
    const uint8_t *__restrict__ live, int live_ld, const int32_t *__restrict__ nvalid_p,
    const int32_t *__restrict__ idx, int n_cb, int n_rb_grid, int D, float *__restrict__ dh_acc, int direct,
    T *__restrict__ dH) {
    using TL = TileG;
    using DE = DmaEngine<T, TL>;
    __shared__ u32x4 lds[DE::kLdsChunks];
    __shared__ int list[kChunkVocab / kBlockVocab];
    __shared__ int wcnt[TL::kWaves];
    const int nv = *nvalid_p;
    const int rb = blockIdx.x % n_rb_grid;
    const int d0 = (blockIdx.x / n_rb_grid) * TL::BN;
    const int tok0 = rb * TL::BM;
    if (tok0 >= nv) return;
    constexpr int kBlockBytes = kBlockVocab * (int)sizeof(T);
    constexpr int kSpb = kBlockBytes / DE::kStageBytes;

    const int n = build_list<TL::kThreads>(
        n_cb, [&](int i) { return live[(int64_t)rb * live_ld + i] != 0; }, list, wcnt);
    if (n == 0 && !direct) return;  // nothing to add in this chunk
    DE eng(lds);
#pragma unroll
    for (int j = 0; j < DE::NIA; ++j) {
        const int r = DE::row_a(j);
        eng.pa[j] = reinterpret_cast<const char *>(Gn + (int64_t)(tok0 + r) * ldn) + DE::chunk_off(r);
    }
#pragma unroll
    for (int j = 0; j < DE::NIB; ++j) {
        const int r = DE::row_b(j);
        const int d = min(d0 + r, D - 1);
        eng.pb[j] = reinterpret_cast<const char *>(Et + (int64_t)d * lde) + DE::chunk_off(r);
    }
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    const int total = n * kSpb;
    auto kb = [&](int q) { return list[q / kSpb] * kBlockBytes + (q % kSpb) * DE::kStageBytes; };
#pragma unroll
    for (int q = 0; q < DE::kDepth; ++q)
        if (q < total) eng.issue(q, kb(q));
    for (int s = 0; s < total; ++s) {
        const int ahead = total - 1 - s;
        eng.wait_stage(eng.clamp_ahead(ahead));
        if (s + DE::kDepth < total) eng.issue((s + DE::kDepth) % DE::kStages, kb(s + DE::kDepth));
        eng.compute(s % DE::kStages, acc);
    }

    if (direct) {
        int row[TL::TM][16];  // output row of each accumulator row, loaded once
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) row[tm][r] = idx[min(tok0 + tile_row<TL>(tm, r), nv - 1)];
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) {
                const int d = d0 + tile_col<TL>(tn);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = tok0 + tile_row<TL>(tm, r);
                    if (tok < nv && d < D) dH[(int64_t)row[tm][r] * D + d] = from_f32<T>(acc[tm][tn][r]);
                }
            }
        return;
    }
    // Read every partial sum first, then write: the loads overlap instead of
    // each waiting behind the previous store.
    float old[TL::TM][TL::TN][16];
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int d = d0 + tile_col<TL>(tn);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = tok0 + tile_row<TL>(tm, r);
                // unconditional load from a clamped in-bounds address (dh_acc is [Np, D], tok < Np)
                old[tm][tn][r] = __builtin_nontemporal_load(dh_acc + (int64_t)tok * D + min(d, D - 1));
            }
        }
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int d = d0 + tile_col<TL>(tn);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = tok0 + tile_row<TL>(tm, r);
                if (tok < nv && d < D) dh_acc[(int64_t)tok * D + d] = old[tm][tn][r] + acc[tm][tn][r];
            }
        }
}

// dH[idx[t]] = dh_acc[t] in the output dtype, for the valid tokens.
template <typename T>
__global__ __launch_bounds__(256) void k_dh_final(const float *__restrict__ dh_acc, const int32_t *__restrict__ idx,
                                                  const int32_t *__restrict__ nvalid_p, int D, T *__restrict__ dH) {
    const int64_t tok = blockIdx.x;
    if (tok >= *nvalid_p) return;
    const float *src = dh_acc + tok * D;
    T *dst = dH + (int64_t)idx[tok] * D;
    for (int d = threadIdx.x * 4; d < D; d += 256 * 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(src + d);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[d + q] = from_f32<T>(v[q]);
    }
}

__global__ __launch_bounds__(256) void k_fill_zero(float *__restrict__ p, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i < n) *reinterpret_cast<f32x4 *>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------- launchers
BwdShape bwd_shape(int64_t N, int64_t D, int64_t V) {
    BwdShape s;
    s.N = N;
    s.D = D;
    s.V = V;
    s.Np = round_up(N, kTileRows);
    const int64_t Vp = round_up(V, kTileVocab);
    s.Vc = (int)(Vp < kChunkVocab ? Vp : kChunkVocab);
    s.n_chunks = (int)ceil_div(V, s.Vc);
    s.n_rtiles = (int)(s.Np / kTileRows);
    return s;
}

BwdWs bwd_ws(void *ws, const BwdShape &s, size_t elem, size_t *bytes) {
    Carver c(ws);
    BwdWs w;
    w.idx = c.take<int32_t>(s.N);
    w.nvalid = c.take<int32_t>(1);
    w.inv_perm = c.take<int32_t>(s.V);
    w.live = c.take<uint8_t>((size_t)(s.Np / kBlockRows) * (s.Vc / kBlockVocab));
    w.lmin = c.take<float>((size_t)s.n_rtiles);
    w.dh_acc = s.n_chunks > 1 ? c.take<float>((size_t)s.Np * s.D) : nullptr;
    w.Ht = c.take<char>(elem * (size_t)s.D * s.Np);
    w.Gt = c.take<char>(elem * (size_t)s.Vc * s.Np);
    w.Gn = c.take<char>(elem * (size_t)s.Np * s.Vc);
    w.Et = c.take<char>(elem * (size_t)s.D * s.Vc);
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
static hipError_t backward_t(const T *H, const T *E, const int64_t *labels, const float *lse,
                             const float *dloss, const float *tile_bound, const BwdShape &s, int64_t ignore_index,
                             float eps, const int32_t *perm, unsigned flags, T *dH, T *dE, int64_t *stats,
                             const BwdWs &w, hipStream_t st) {
    const int D = (int)s.D, V = (int)s.V;
    CCE_TRY(launch_compact(labels, s.N, ignore_index, w.idx, w.nvalid, st));
    // The tile bound is in the natural vocabulary order and only says something
    // when filtering is on.  thr = ln(eps / 2), rounded towards -inf.
    const float *tb = (tile_bound && !perm && eps > 0.f) ? tile_bound : nullptr;
    float thr = 0.f;
    if (tb) {
        thr = (float)(log((double)eps) - log(2.0));
        thr = nextafterf(thr, -__builtin_huge_valf());
        hipLaunchKernelGGL(k_lse_min, dim3((unsigned)s.n_rtiles), dim3(kTileRows), 0, st, lse, w.idx, w.nvalid,
                           w.lmin);
        CCE_LAUNCHED();
    }
    const int64_t tb_ld = ceil_div(s.V, kTileVocab);
    if (perm) {
        hipLaunchKernelGGL(k_inv_perm, dim3((unsigned)ceil_div(V, 256)), dim3(256), 0, st, perm, V, w.inv_perm);
        CCE_LAUNCHED();
    }
    if (stats) {
        hipLaunchKernelGGL(k_stats_init, dim3(1), dim3(64), 0, st, stats);
        CCE_LAUNCHED();
    }
    T *Ht = static_cast<T *>(w.Ht);
    T *Gt = static_cast<T *>(w.Gt);
    T *Gn = static_cast<T *>(w.Gn);
    T *Et = static_cast<T *>(w.Et);
    // H^T of the valid rows: [D, Np], zero beyond the valid rows.
    hipLaunchKernelGGL(k_transpose<T>, dim3((unsigned)ceil_div(s.Np, 64), (unsigned)ceil_div(D, 64)), dim3(256),
                       0, st, H, (int64_t)D, s.N, w.idx, (int64_t)0, w.nvalid, 0, D, (int)s.Np, Ht, (int64_t)s.Np);
    CCE_LAUNCHED();
    hipLaunchKernelGGL(k_zero_ignored<T>, dim3((unsigned)ceil_div(s.N, 4)), dim3(256), 0, st, labels, s.N, D,
                       ignore_index, dH);
    CCE_LAUNCHED();

    const bool dma_g = ((int64_t)D * (int64_t)sizeof(T)) % kLogitRowBytes == 0;
    if (s.n_chunks > 1) {
        const int64_t n = s.Np * (int64_t)D;  // D % 8 == 0: whole f32x4 groups
        hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)ceil_div(n, 1024)), dim3(256), 0, st, w.dh_acc, n);
        CCE_LAUNCHED();
    }
    const int n_dt = (int)ceil_div(D, TileG::BN);
    const int live_ld = s.Vc / kBlockVocab;
    const int n_rb_grid = (int)(s.Np / kBlockRows);
    for (int c = 0; c < s.n_chunks; ++c) {
        const int cv0 = c * s.Vc;
        const int clen = (int)((V - cv0) < s.Vc ? (V - cv0) : s.Vc);
        const int n_ct = (int)ceil_div(clen, kTileVocab);   // logit tiles in the chunk
        const int n_cb = (int)ceil_div(clen, kBlockVocab);  // filter blocks in the chunk
        // E^T of the chunk (processing order): [D, Vc], zero beyond clen.
        hipLaunchKernelGGL(k_transpose<T>, dim3((unsigned)ceil_div(n_ct * kTileVocab, 64), (unsigned)ceil_div(D, 64)),
                           dim3(256), 0, st, E, (int64_t)D, s.V, perm, (int64_t)cv0, (const int32_t *)nullptr, clen, D,
                           n_ct * kTileVocab, Et, (int64_t)s.Vc);
        CCE_LAUNCHED();
        if (dma_g)
            hipLaunchKernelGGL((k_bwd_g_dma<T, TileFD>), dim3((unsigned)(n_ct * s.n_rtiles)), dim3(TileFD::kThreads), 0, st, H,
                               E, w.idx, w.nvalid, perm, perm ? w.inv_perm : nullptr, labels, lse, dloss, D, V, cv0,
                               n_ct, live_ld, eps, Gt, (int64_t)s.Np, Gn, (int64_t)s.Vc, w.live, stats, tb, tb_ld,
                               w.lmin, thr);
        else
            hipLaunchKernelGGL(k_bwd_g<T>, dim3((unsigned)(n_ct * s.n_rtiles)), dim3(TileF::kThreads), 0, st, H, E,
                               w.idx, w.nvalid, perm, perm ? w.inv_perm : nullptr, labels, lse, dloss, D, V, cv0,
                               n_ct, live_ld, eps, Gt, (int64_t)s.Np, Gn, (int64_t)s.Vc, w.live, stats, tb, tb_ld,
                               w.lmin, thr);
        CCE_LAUNCHED();
        if (flags & CCE_BWD_NO_KAHAN)
            hipLaunchKernelGGL((k_de<T, false>), dim3((unsigned)(n_cb * n_dt)), dim3(TileG::kThreads), 0, st, Gt,
                               (int64_t)s.Np, Ht, (int64_t)s.Np, w.live, live_ld, w.nvalid, perm, n_cb, D, V, cv0, dE);
        else
            hipLaunchKernelGGL((k_de<T, true>), dim3((unsigned)(n_cb * n_dt)), dim3(TileG::kThreads), 0, st, Gt,
                               (int64_t)s.Np, Ht, (int64_t)s.Np, w.live, live_ld, w.nvalid, perm, n_cb, D, V, cv0, dE);
        CCE_LAUNCHED();
        hipLaunchKernelGGL(k_dh<T>, dim3((unsigned)(n_rb_grid * n_dt)), dim3(TileG::kThreads), 0, st, Gn,
                           (int64_t)s.Vc, Et, (int64_t)s.Vc, w.live, live_ld, w.nvalid, w.idx, n_cb, n_rb_grid, D,
                           w.dh_acc, s.n_chunks == 1 ? 1 : 0, dH);
        CCE_LAUNCHED();
    }
    if (s.n_chunks > 1) {
        hipLaunchKernelGGL(k_dh_final<T>, dim3((unsigned)s.N), dim3(256), 0, st, w.dh_acc, w.idx, w.nvalid, D, dH);
        CCE_LAUNCHED();
    }
    if (stats) {
        hipLaunchKernelGGL(k_stats_fin, dim3(1), dim3(64), 0, st, stats, w.nvalid, (int64_t)ceil_div(V, kBlockVocab));
        CCE_LAUNCHED();
    }
    return hipSuccess;
}

hipError_t launch_backward(cce_dtype dt, const void *H, const void *E, const int64_t *labels,
                           const float *lse, const float *dloss, const float *tile_bound, const BwdShape &s,
                           int64_t ignore_index, float eps, const int32_t *perm, unsigned flags,
                           void *dH, void *dE, int64_t *stats, const BwdWs &w, hipStream_t st) {
    if (dt == CCE_BF16)
        return backward_t<bf16_t>(static_cast<const bf16_t *>(H), static_cast<const bf16_t *>(E), labels, lse,
                                  dloss, tile_bound, s, ignore_index, eps, perm, flags, static_cast<bf16_t *>(dH),
                                  static_cast<bf16_t *>(dE), stats, w, st);
    return backward_t<float>(static_cast<const float *>(H), static_cast<const float *>(E), labels, lse, dloss,
                             tile_bound, s, ignore_index, eps, perm, flags, static_cast<float *>(dH),
                             static_cast<float *>(dE), stats, w, st);
}

}  // namespace cce
