// Optional vocabulary order for the backward: sort the vocabulary by mean
// logit so that the blocks that survive gradient filtering cluster together,
// which makes a block-granular skip pay off (lit note "The loss and the mask:
// Cut Cross-Entropy + FlexAttention", section "Contribution"; CCE paper
// summary "Cut Your Losses in Large-Vocabulary Language Models", section
// "Approach").
//
// The mean logit of entry v over the valid rows is <hbar, e_v> with
// hbar = mean of the valid h_i (linearity), so the keys cost one pass over H
// and one over E:
//   k_hsum / k_hbar   hbar in fp32, fixed summation order
//   k_keys            key_v = <hbar, e_v>, one wave per entry
//   radix sort        stable LSD sort of 32-bit order-preserving key codes,
//                     8-bit digits (histogram / scan / ranked scatter per
//                     pass): descending key, ties by ascending id.
#include "cce_device.hpp"
#include "cce_internal.hpp"

namespace cce {

constexpr int kHsumParts = 64;
constexpr int kSortTile = 2048;  // elements per scatter workgroup (256 threads x 8 rounds)

// Partial column sums: part p sums the valid rows at positions
// [p nv / P, (p + 1) nv / P) of the compacted list, one feature per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_hsum(const T *__restrict__ H, const int32_t *__restrict__ idx,
                                              const int32_t *__restrict__ nvalid_p, int D,
                                              float *__restrict__ part) {
    const int nv = *nvalid_p;
    const int p = blockIdx.x;
    const int d = blockIdx.y * 256 + threadIdx.x;
    if (d >= D) return;
    const int k0 = (int)((int64_t)nv * p / kHsumParts);
    const int k1 = (int)((int64_t)nv * (p + 1) / kHsumParts);
    float s = 0.f;
    for (int k = k0; k < k1; ++k) s += to_f32(H[(int64_t)idx[k] * D + d]);
    part[(int64_t)p * D + d] = s;
}

__global__ __launch_bounds__(256) void k_hbar(const float *__restrict__ part, const int32_t *__restrict__ nvalid_p,
                                              int D, float *__restrict__ hbar) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    if (d >= D) return;
    const int nv = *nvalid_p;
    float s = 0.f;
    for (int p = 0; p < kHsumParts; ++p) s += part[(int64_t)p * D + d];
    hbar[d] = nv > 0 ? s / (float)nv : 0.f;
}

// key_v = <hbar, e_v>; also the order-preserving code of the key (ascending
// code = descending key, -0 == +0) and the initial ids.
template <typename T>
__global__ __launch_bounds__(256) void k_keys(Rows2<const T> E, const float *__restrict__ hbar, int D,
                                              int V, float *__restrict__ keys, uint32_t *__restrict__ code,
                                              int32_t *__restrict__ ids) {
    constexpr int CE = ChunkElems<T>::value;
    const int lane = threadIdx.x & 63;
    const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (v >= V) return;
    const char *e = reinterpret_cast<const char *>(E.row(v));
    float s = 0.f;
    for (int k = lane * CE; k < D; k += 64 * CE) {
        const u32x4 ev = ld16(e + k * sizeof(T));
        const T *ep = reinterpret_cast<const T *>(&ev);
#pragma unroll
        for (int q = 0; q < CE; ++q) s += hbar[k + q] * to_f32(ep[q]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) {
        keys[v] = s;
        const float f = s == 0.f ? 0.f : s;  // -0 -> +0
        const uint32_t u = __float_as_uint(f);
        const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in f
        code[v] = ~asc;                                                    // ascending in -f
        ids[v] = (int32_t)v;
    }
}

// Per tile digit counts, stored digit-major: hist[digit * n_tiles + tile].
__global__ __launch_bounds__(256) void k_radix_hist(const uint32_t *__restrict__ code, int V, int shift,
                                                    int n_tiles, uint32_t *__restrict__ hist) {
    __shared__ uint32_t cnt[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * kSortTile;
    for (int q = threadIdx.x; q < kSortTile; q += 256) {
        const int64_t i = t0 + q;
        if (i < V) atomicAdd(&cnt[(code[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * n_tiles + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of hist (n entries) in place, one workgroup.
__global__ __launch_bounds__(1024) void k_radix_scan(uint32_t *__restrict__ hist, int n) {
    __shared__ uint32_t wtot[16];
    __shared__ uint32_t carry;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    if (t == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int i = base + t;
        const uint32_t x0 = i < n ? hist[i] : 0u;
        uint32_t x = x0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        if (lane == 63) wtot[wave] = x;
        __syncthreads();
        uint32_t wb = 0;
        for (int w = 0; w < wave; ++w) wb += wtot[w];
        const uint32_t c = carry;
        if (i < n) hist[i] = c + wb + x - x0;
        __syncthreads();
        if (t == 1023) carry = c + wb + x;
        __syncthreads();
    }
}

// Stable scatter: elements of the tile in index order; the rank of an element
// among equal digits is (earlier rounds) + (earlier waves of this round) +
// (earlier lanes of its wave), the latter from ballot masks.
__global__ __launch_bounds__(256) void k_radix_scatter(const uint32_t *__restrict__ code_in,
                                                       const int32_t *__restrict__ val_in, int V, int shift,
                                                       int n_tiles, const uint32_t *__restrict__ offs,
                                                       uint32_t *__restrict__ code_out,
                                                       int32_t *__restrict__ val_out) {
    __shared__ uint32_t run[256];
    __shared__ uint32_t wc[4][256];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    run[t] = offs[(int64_t)t * n_tiles + blockIdx.x];
    const int64_t t0 = (int64_t)blockIdx.x * kSortTile;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int round = 0; round < kSortTile / 256; ++round) {
#pragma unroll
        for (int w = 0; w < 4; ++w) wc[w][t] = 0;
        __syncthreads();
        const int64_t i = t0 + round * 256 + t;
        const bool ok = i < V;
        const uint32_t k = ok ? code_in[i] : 0u;
        const int32_t v = ok ? val_in[i] : 0;
        const uint32_t dg = (k >> shift) & 255u;
        uint64_t mask = __ballot(ok);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (dg >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            mask &= bit ? bal : ~bal;
        }
        const int rank = __popcll(mask & below);
        if (ok && rank == 0) wc[wave][dg] = (uint32_t)__popcll(mask);
        __syncthreads();
        if (ok) {
            uint32_t pos = run[dg] + rank;
            for (int w = 0; w < wave; ++w) pos += wc[w][dg];
            if (pos < (uint32_t)V) {  // always true for a consistent histogram; never write outside
                code_out[pos] = k;
                val_out[pos] = v;
            }
        }
        __syncthreads();
        run[t] += wc[0][t] + wc[1][t] + wc[2][t] + wc[3][t];
        __syncthreads();
    }
}

SortWs sort_ws(void *ws, int64_t N, int64_t D, int64_t V, size_t *bytes) {
    Carver c(ws);
    SortWs w;
    const int64_t n_tiles = ceil_div(V, kSortTile);
    w.hsum_part = c.take<float>((size_t)kHsumParts * D);
    w.hbar = c.take<float>(D);
    w.keys = c.take<float>(V);
    w.ukeys[0] = c.take<uint32_t>(V);
    w.ukeys[1] = c.take<uint32_t>(V);
    w.vals[0] = nullptr;  // the caller's perm buffer
    w.vals[1] = c.take<int32_t>(V);
    w.hist = c.take<uint32_t>((size_t)256 * n_tiles);
    w.idx = c.take<int32_t>(N);
    w.nvalid = c.take<int32_t>(1);
    if (bytes) *bytes = c.off;
    return w;
}

template <typename T>
static hipError_t vocab_order_t(const T *H, Rows2<const T> E, const int64_t *labels, int64_t N, int64_t D, int64_t V,
                                int64_t ignore_index, int32_t *perm, float *keys_out, int32_t *idx,
                                const SortWs &w, hipStream_t st) {
    hipError_t e = launch_compact(labels, N, ignore_index, idx, w.nvalid, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_hsum<T>, dim3(kHsumParts, (unsigned)ceil_div(D, 256)), dim3(256), 0, st, H, idx, w.nvalid,
                       (int)D, w.hsum_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_hbar, dim3((unsigned)ceil_div(D, 256)), dim3(256), 0, st, w.hsum_part, w.nvalid, (int)D,
                       w.hbar);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    float *keys = keys_out ? keys_out : w.keys;
    hipLaunchKernelGGL(k_keys<T>, dim3((unsigned)ceil_div(V, 4)), dim3(256), 0, st, E, w.hbar, (int)D, (int)V, keys,
                       w.ukeys[0], perm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int n_tiles = (int)ceil_div(V, kSortTile);
    uint32_t *kb[2] = {w.ukeys[0], w.ukeys[1]};
    int32_t *vb[2] = {perm, w.vals[1]};
    for (int pass = 0; pass < 4; ++pass) {
        const int in = pass & 1, out = in ^ 1;
        hipLaunchKernelGGL(k_radix_hist, dim3(n_tiles), dim3(256), 0, st, kb[in], (int)V, 8 * pass, n_tiles, w.hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_radix_scan, dim3(1), dim3(1024), 0, st, w.hist, 256 * n_tiles);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_radix_scatter, dim3(n_tiles), dim3(256), 0, st, kb[in], vb[in], (int)V, 8 * pass,
                           n_tiles, w.hist, kb[out], vb[out]);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;  // four passes: the sorted ids are back in perm
}

hipError_t launch_vocab_order(cce_dtype dt, const void *H, const VocabRows &E, const int64_t *labels, int64_t N,
                              int64_t D, int64_t V, int64_t ignore_index, int32_t *perm, float *keys_out,
                              const SortWs &w, hipStream_t st) {
    if (dt == CCE_BF16)
        return vocab_order_t<bf16_t>(
            static_cast<const bf16_t *>(H),
            Rows2<const bf16_t>{static_cast<const bf16_t *>(E.e0), static_cast<const bf16_t *>(E.e1), E.v0, D},
            labels, N, D, V, ignore_index, perm, keys_out, w.idx, w, st);
    return vocab_order_t<float>(
        static_cast<const float *>(H),
        Rows2<const float>{static_cast<const float *>(E.e0), static_cast<const float *>(E.e1), E.v0, D}, labels, N,
        D, V, ignore_index, perm, keys_out, w.idx, w, st);
}

}  // namespace cce
