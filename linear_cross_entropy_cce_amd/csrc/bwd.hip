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
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {

using TileFR = Tile<kBlockVocab, kBlockRows, 2, 2>;  // logit tile: A = vocabulary, B = tokens
using TileDE = Tile<kBlockVocab, 128, 2, 2>;         // dE tile: A = G^T rows, B = H^T rows (features)
using TileDH = Tile<kBlockRows, 128, 2, 2>;          // dH tile: A = G rows, B = E^T rows (features)

// ------------------------------------------------------------ small kernels
__global__ void k_inv_perm(const int32_t *__restrict__ perm, int V, int32_t *__restrict__ inv) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < V) {
        const int v = perm[k];
        if (v >= 0 && v < V) inv[v] = k;
    }
}

__global__ void k_stats_init(int64_t *stats) {
    if (threadIdx.x < 4) stats[threadIdx.x] = 0;
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

// ------------------------------------------- recompute + filter + G tile
// Workgroup (vocabulary tile ct of the chunk, token tile rt).  Block status:
// 1 = some p >= eps (softmax part kept), 2 = no p >= eps but a label falls in
// the block (only the -dloss one-hot entries are kept), 0 = skipped.
template <typename T>
__global__ __launch_bounds__(TileFR::kThreads) void k_bwd_g(
    const T *__restrict__ H, const T *__restrict__ E, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ inv_perm, const int64_t *__restrict__ labels,
    const float *__restrict__ lse, const float *__restrict__ dloss, int D, int V, int chunk_v0, int n_ct,
    float eps, T *__restrict__ Gt, int64_t ldt, T *__restrict__ Gn, int64_t ldn,
    uint8_t *__restrict__ live, int64_t *__restrict__ stats) {
    using TL = TileFR;
    __shared__ u32x4 lds[TL::kLdsChunks];
    const int nv = *nvalid_p;
    const int ct = blockIdx.x % n_ct;
    const int rt = blockIdx.x / n_ct;
    const int tok0 = rt * TL::BN;
    if (tok0 >= nv) return;
    const int p0 = chunk_v0 + ct * TL::BM;  // first vocabulary position (processing order)
    const int tid = threadIdx.x;
    const size_t rowb = (size_t)D * sizeof(T);
    const int kvalid = D * (int)sizeof(T);
    const int nsteps = (kvalid + TL::kStageBytes - 1) / TL::kStageBytes;

    Stager<TL::kALoads, TL::kBLoads> st;
    stager_slots<TL>(st, tid);
#pragma unroll
    for (int j = 0; j < TL::kALoads; ++j) {
        const int pos = p0 + stage_row_a<TL>(tid, j);
        const int vid = pos < V ? (perm ? perm[pos] : pos) : -1;
        st.a[j] = (vid >= 0 && vid < V) ? reinterpret_cast<const char *>(E) + (size_t)vid * rowb : nullptr;
    }
#pragma unroll
    for (int j = 0; j < TL::kBLoads; ++j) {
        const int tok = tok0 + stage_row_b<TL>(tid, j);
        st.b[j] = tok < nv ? reinterpret_cast<const char *>(H) + (size_t)idx[tok] * rowb : nullptr;
    }
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    mainloop<T, TL>(acc, st, nsteps, [](int s) { return s * TL::kStageBytes; }, kvalid, [](int) {}, lds);

    // Per token column: lse, dloss and the label's local vocabulary row.
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
            lab_t[tn] = ypos - p0;  // may fall outside [0, BM)
            any_label |= (lab_t[tn] >= 0 && lab_t[tn] < TL::BM);
        }
    }
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool ok = tok_ok[tn] && (p0 + tile_row<TL>(tm, r) < V);
                const float p = ok ? __builtin_amdgcn_exp2f((acc[tm][tn][r] - lse_t[tn]) * kLog2e) : 0.f;
                acc[tm][tn][r] = p;
                any_live |= ok && (p >= eps);
            }
    const bool blk_live = __syncthreads_or(any_live);
    const bool blk_label = __syncthreads_or(any_label);
    const int status = blk_live ? 1 : (blk_label ? 2 : 0);
    if (tid == 0) {
        live[rt * n_ct + ct] = (uint8_t)status;
        if (stats && status) atomicAdd(reinterpret_cast<unsigned long long *>(stats + (status == 1 ? 0 : 1)), 1ull);
    }
    if (status == 0) return;

    const int lane = tid & 63;
    (void)lane;
#pragma unroll
    for (int tn = 0; tn < TL::TN; ++tn) {
        const int c = tile_col<TL>(tn);
        const int64_t tok = tok0 + c;
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                T g4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = r4 * 4 + q;
                    const int rl = tile_row<TL>(tm, r);
                    const bool ok = tok_ok[tn] && (p0 + rl < V);
                    const float pk = status == 1 ? acc[tm][tn][r] : 0.f;
                    const float g = ok ? dl_t[tn] * (pk - (rl == lab_t[tn] ? 1.f : 0.f)) : 0.f;
                    g4[q] = from_f32<T>(g);
                    Gt[(int64_t)(ct * TL::BM + rl) * ldt + tok] = g4[q];
                }
                // the four rows r4*4 .. r4*4+3 are consecutive vocabulary entries
                T *dst = Gn + tok * ldn + ct * TL::BM + tile_row<TL>(tm, r4 * 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = g4[q];
            }
    }
}

// ------------------------------------------------------------- dE (Kahan)
// Workgroup (vocabulary tile ct of the chunk, feature tile dt).  K runs over
// the valid tokens of the row blocks that survived for this vocabulary tile.
// Each row block's product is formed in a fresh fp32 MFMA accumulator and then
// added into (sum, compensation) with Kahan's rule.
constexpr int kListCap = 256;

template <typename T, bool KAHAN>
__global__ __launch_bounds__(TileDE::kThreads) void k_de(
    const T *__restrict__ Gt, int64_t ldt, const T *__restrict__ Ht, int64_t ldh,
    const uint8_t *__restrict__ live, const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ perm,
    int n_ct, int D, int V, int chunk_v0, T *__restrict__ dE) {
    using TL = TileDE;
    __shared__ u32x4 lds[TL::kLdsChunks];
    __shared__ int list[kListCap];
    __shared__ int list_n;
    const int nv = *nvalid_p;
    const int n_rt = (nv + kBlockRows - 1) / kBlockRows;
    const int ct = blockIdx.x % n_ct;
    const int d0 = (blockIdx.x / n_ct) * TL::BN;
    const int tid = threadIdx.x;
    constexpr int kBlockBytes = kBlockRows * (int)sizeof(T);
    constexpr int kSpb = kBlockBytes / TL::kStageBytes;  // stages per row block

    Stager<TL::kALoads, TL::kBLoads> st;
    stager_slots<TL>(st, tid);
#pragma unroll
    for (int j = 0; j < TL::kALoads; ++j)
        st.a[j] = reinterpret_cast<const char *>(Gt + (int64_t)(ct * TL::BM + stage_row_a<TL>(tid, j)) * ldt);
#pragma unroll
    for (int j = 0; j < TL::kBLoads; ++j) {
        const int d = d0 + stage_row_b<TL>(tid, j);
        st.b[j] = d < D ? reinterpret_cast<const char *>(Ht + (int64_t)d * ldh) : nullptr;
    }

    f32x16 acc[TL::TM][TL::TN], sum[TL::TM][TL::TN], comp[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    zero_acc<TL>(sum);
    zero_acc<TL>(comp);

    for (int base = 0; base < n_rt; base += kListCap) {
        __syncthreads();
        if (tid == 0) {
            int n = 0;
            const int end = base + kListCap < n_rt ? base + kListCap : n_rt;
            for (int rt = base; rt < end; ++rt)
                if (live[rt * n_ct + ct]) list[n++] = rt;
            list_n = n;
        }
        __syncthreads();
        const int n = list_n;
        if (n == 0) continue;
        mainloop<T, TL>(
            acc, st, n * kSpb,
            [&](int s) { return list[s / kSpb] * kBlockBytes + (s % kSpb) * TL::kStageBytes; }, 0x7fffffff,
            [&](int s) {
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
            },
            lds);
    }

#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int d = d0 + tile_col<TL>(tn);
            if (d >= D) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int pos = chunk_v0 + ct * TL::BM + tile_row<TL>(tm, r);
                if (pos >= V) continue;
                const int64_t vid = perm ? perm[pos] : pos;
                if (vid < 0 || vid >= V) continue;
                const float val = KAHAN ? sum[tm][tn][r] - comp[tm][tn][r] : acc[tm][tn][r];
                dE[vid * D + d] = from_f32<T>(val);
            }
        }
}

// ------------------------------------------------------------------- dH
// Workgroup (token tile rt, feature tile dt).  K runs over the surviving
// vocabulary blocks of the chunk.  fp32 partial sums are carried across
// chunks in dh_acc; the last chunk writes the output row of each token.
template <typename T>
__global__ __launch_bounds__(TileDH::kThreads) void k_dh(
    const T *__restrict__ Gn, int64_t ldn, const T *__restrict__ Et, int64_t lde,
    const uint8_t *__restrict__ live, const int32_t *__restrict__ nvalid_p, const int32_t *__restrict__ idx,
    int n_ct, int n_rt_grid, int D, float *__restrict__ dh_acc, int first, int last, T *__restrict__ dH) {
    using TL = TileDH;
    __shared__ u32x4 lds[TL::kLdsChunks];
    __shared__ int list[kChunkVocab / kBlockVocab];
    __shared__ int list_n;
    const int nv = *nvalid_p;
    const int rt = blockIdx.x % n_rt_grid;
    const int d0 = (blockIdx.x / n_rt_grid) * TL::BN;
    const int tok0 = rt * TL::BM;
    if (tok0 >= nv) return;
    const int tid = threadIdx.x;
    constexpr int kBlockBytes = kBlockVocab * (int)sizeof(T);
    constexpr int kSpb = kBlockBytes / TL::kStageBytes;

    if (tid == 0) {
        int n = 0;
        for (int ct = 0; ct < n_ct; ++ct)
            if (live[rt * n_ct + ct]) list[n++] = ct;
        list_n = n;
    }
    Stager<TL::kALoads, TL::kBLoads> st;
    stager_slots<TL>(st, tid);
#pragma unroll
    for (int j = 0; j < TL::kALoads; ++j) {
        const int tok = tok0 + stage_row_a<TL>(tid, j);
        st.a[j] = tok < nv ? reinterpret_cast<const char *>(Gn + (int64_t)tok * ldn) : nullptr;
    }
#pragma unroll
    for (int j = 0; j < TL::kBLoads; ++j) {
        const int d = d0 + stage_row_b<TL>(tid, j);
        st.b[j] = d < D ? reinterpret_cast<const char *>(Et + (int64_t)d * lde) : nullptr;
    }
    __syncthreads();
    const int n = list_n;
    f32x16 acc[TL::TM][TL::TN];
    zero_acc<TL>(acc);
    mainloop<T, TL>(
        acc, st, n * kSpb, [&](int s) { return list[s / kSpb] * kBlockBytes + (s % kSpb) * TL::kStageBytes; },
        0x7fffffff, [](int) {}, lds);

#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) {
            const int d = d0 + tile_col<TL>(tn);
            if (d >= D) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tok = tok0 + tile_row<TL>(tm, r);
                if (tok >= nv) continue;
                float v = acc[tm][tn][r];
                if (!first) v += dh_acc[(int64_t)tok * D + d];
                if (last)
                    dH[(int64_t)idx[tok] * D + d] = from_f32<T>(v);
                else
                    dh_acc[(int64_t)tok * D + d] = v;
            }
        }
}

// ---------------------------------------------------------------- launchers
BwdShape bwd_shape(int64_t N, int64_t D, int64_t V) {
    BwdShape s;
    s.N = N;
    s.D = D;
    s.V = V;
    s.Np = round_up(N, kBlockRows);
    const int64_t Vp = round_up(V, kBlockVocab);
    s.Vc = (int)(Vp < kChunkVocab ? Vp : kChunkVocab);
    s.n_chunks = (int)ceil_div(V, s.Vc);
    s.n_rtiles = (int)(s.Np / kBlockRows);
    return s;
}

BwdWs bwd_ws(void *ws, const BwdShape &s, size_t elem, size_t *bytes) {
    Carver c(ws);
    BwdWs w;
    w.idx = c.take<int32_t>(s.N);
    w.nvalid = c.take<int32_t>(1);
    w.inv_perm = c.take<int32_t>(s.V);
    w.live = c.take<uint8_t>((size_t)s.n_rtiles * (s.Vc / kBlockVocab));
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
                             const float *dloss, const BwdShape &s, int64_t ignore_index, float eps,
                             const int32_t *perm, unsigned flags, T *dH, T *dE, int64_t *stats,
                             const BwdWs &w, hipStream_t st) {
    const int D = (int)s.D, V = (int)s.V;
    CCE_TRY(launch_compact(labels, s.N, ignore_index, w.idx, w.nvalid, st));
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

    const int n_dt = (int)ceil_div(D, 128);
    for (int c = 0; c < s.n_chunks; ++c) {
        const int cv0 = c * s.Vc;
        const int clen = (int)((V - cv0) < s.Vc ? (V - cv0) : s.Vc);
        const int n_ct = (int)ceil_div(clen, kBlockVocab);
        // E^T of the chunk (processing order): [D, Vc], zero beyond clen.
        hipLaunchKernelGGL(k_transpose<T>, dim3((unsigned)ceil_div(n_ct * kBlockVocab, 64), (unsigned)ceil_div(D, 64)),
                           dim3(256), 0, st, E, (int64_t)D, s.V, perm, (int64_t)cv0, (const int32_t *)nullptr, clen, D,
                           n_ct * kBlockVocab, Et, (int64_t)s.Vc);
        CCE_LAUNCHED();
        hipLaunchKernelGGL(k_bwd_g<T>, dim3((unsigned)(n_ct * s.n_rtiles)), dim3(TileFR::kThreads), 0, st, H, E,
                           w.idx, w.nvalid, perm, perm ? w.inv_perm : nullptr, labels, lse, dloss, D, V, cv0, n_ct,
                           eps, Gt, (int64_t)s.Np, Gn, (int64_t)s.Vc, w.live, stats);
        CCE_LAUNCHED();
        if (flags & CCE_BWD_NO_KAHAN)
            hipLaunchKernelGGL((k_de<T, false>), dim3((unsigned)(n_ct * n_dt)), dim3(TileDE::kThreads), 0, st, Gt,
                               (int64_t)s.Np, Ht, (int64_t)s.Np, w.live, w.nvalid, perm, n_ct, D, V, cv0, dE);
        else
            hipLaunchKernelGGL((k_de<T, true>), dim3((unsigned)(n_ct * n_dt)), dim3(TileDE::kThreads), 0, st, Gt,
                               (int64_t)s.Np, Ht, (int64_t)s.Np, w.live, w.nvalid, perm, n_ct, D, V, cv0, dE);
        CCE_LAUNCHED();
        hipLaunchKernelGGL(k_dh<T>, dim3((unsigned)(s.n_rtiles * n_dt)), dim3(TileDH::kThreads), 0, st, Gn,
                           (int64_t)s.Vc, Et, (int64_t)s.Vc, w.live, w.nvalid, w.idx, n_ct, s.n_rtiles, D, w.dh_acc,
                           c == 0 ? 1 : 0, c == s.n_chunks - 1 ? 1 : 0, dH);
        CCE_LAUNCHED();
    }
    if (stats) {
        hipLaunchKernelGGL(k_stats_fin, dim3(1), dim3(64), 0, st, stats, w.nvalid, (int64_t)ceil_div(V, kBlockVocab));
        CCE_LAUNCHED();
    }
    return hipSuccess;
}

hipError_t launch_backward(cce_dtype dt, const void *H, const void *E, const int64_t *labels,
                           const float *lse, const float *dloss, const BwdShape &s,
                           int64_t ignore_index, float eps, const int32_t *perm, unsigned flags,
                           void *dH, void *dE, int64_t *stats, const BwdWs &w, hipStream_t st) {
    if (dt == CCE_BF16)
        return backward_t<bf16_t>(static_cast<const bf16_t *>(H), static_cast<const bf16_t *>(E), labels, lse,
                                  dloss, s, ignore_index, eps, perm, flags, static_cast<bf16_t *>(dH),
                                  static_cast<bf16_t *>(dE), stats, w, st);
    return backward_t<float>(static_cast<const float *>(H), static_cast<const float *>(E), labels, lse, dloss, s,
                             ignore_index, eps, perm, flags, static_cast<float *>(dH), static_cast<float *>(dE),
                             stats, w, st);
}

}  // namespace cce
