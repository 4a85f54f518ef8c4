// Device-side building blocks shared by the gfx950 kernels of libcce:
// vector types, bf16 conversion, and the MFMA tile engine (LDS-staged,
// double-buffered K loop computing C[M x N] = A[M x K] * B[N x K]^T with both
// operands K-contiguous in memory).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cce {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }

// Elements of T per 16-byte chunk.
template <typename T> struct ChunkElems;
template <> struct ChunkElems<float> { static constexpr int value = 4; };
template <> struct ChunkElems<bf16_t> { static constexpr int value = 8; };

// ------------------------------------------------------------------ MFMA step
// One K-slice of 32 bytes per row: lane l holds 16 bytes of row (l % 32) at
// K-chunk (l / 32) of the slice, for both operands.  The K order inside a
// slice is the same for A and B, so the contraction is exact whatever order
// the hardware assigns to the elements.
//  bf16: v_mfma_f32_32x32x16_bf16 (lane holds 8 consecutive k of its row).
//  f32 : four v_mfma_f32_32x32x2_f32.  MFMA j takes element j of every
//        lane's chunk: k = 4 (2 kk + l / 32) + j, so the four cover the slice.
template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ void step(const u32x4 &a, const u32x4 &b, f32x16 &acc) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static __device__ __forceinline__ void step(const u32x4 &a, const u32x4 &b, f32x16 &acc) {
        const f32x4 fa = __builtin_bit_cast(f32x4, a);
        const f32x4 fb = __builtin_bit_cast(f32x4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
    }
};

// Output layout of a 32x32 MFMA accumulator: register r of lane l holds
// C[row][col] with col = l % 32 and row = 8 (r / 4) + 4 (l / 32) + r % 4.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// ------------------------------------------------------------------ tile shape
// BM x BN output tile per workgroup, WM x WN waves, each wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA blocks.  One K stage is
// 128 bytes of every A and B row (64 bf16 or 32 fp32 values).
template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWaveM = BM / WM;
    static constexpr int kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32;
    static constexpr int TN = kWaveN / 32;
    static constexpr int kStageBytes = 128;
    static constexpr int kAChunks = BM * 8;  // 16-byte chunks of A per stage
    static constexpr int kBChunks = BN * 8;
    static constexpr int kALoads = kAChunks / kThreads;
    static constexpr int kBLoads = kBChunks / kThreads;
    static constexpr int kStage = kAChunks + kBChunks;
    static constexpr int kLdsChunks = 2 * kStage;
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 32x32 block");
    static_assert(kAChunks % kThreads == 0 && kBChunks % kThreads == 0, "stage must split evenly");
};

// LDS position (in 16-byte chunks) of chunk c of row r: rows are 128 bytes,
// chunks XOR-swizzled by the row so that 8 consecutive rows read at the same
// logical chunk hit 8 different bank groups.
__device__ __forceinline__ int lds_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// The rows of A and B that one thread stages, for the whole K loop.  A null
// row pointer stages zeros (rows past the end of the operand).
template <int NA, int NB>
struct Stager {
    const char *a[NA];
    const char *b[NB];
    int cA[NA], cB[NB];  // 16-byte chunk of the row this thread loads
    int sA[NA], sB[NB];  // LDS slot
};

template <class TL>
__device__ __forceinline__ void stager_slots(Stager<TL::kALoads, TL::kBLoads> &st, int tid) {
#pragma unroll
    for (int j = 0; j < TL::kALoads; ++j) {
        const int q = tid + TL::kThreads * j;
        st.cA[j] = q & 7;
        st.sA[j] = lds_slot(q >> 3, q & 7);
    }
#pragma unroll
    for (int j = 0; j < TL::kBLoads; ++j) {
        const int q = tid + TL::kThreads * j;
        st.cB[j] = q & 7;
        st.sB[j] = TL::kAChunks + lds_slot(q >> 3, q & 7);
    }
}

// Row (within the tile) that load j of thread tid stages.
template <class TL>
__device__ __forceinline__ int stage_row_a(int tid, int j) { return (tid + TL::kThreads * j) >> 3; }
template <class TL>
__device__ __forceinline__ int stage_row_b(int tid, int j) { return (tid + TL::kThreads * j) >> 3; }

__device__ __forceinline__ u32x4 ld16(const char *p) { return *reinterpret_cast<const u32x4 *>(p); }

// The K loop.  nsteps stages; koff(s) gives the byte offset along K of stage
// s; chunks at or beyond kvalid bytes read as zero.  after(s) runs once the
// MFMAs of stage s are issued (used to close Kahan blocks).
template <typename T, class TL, class KOff, class After>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[TL::TM][TL::TN],
                                         const Stager<TL::kALoads, TL::kBLoads> &st, int nsteps,
                                         KOff koff, int kvalid, After after, u32x4 *lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % TL::WM;
    const int wn = wave / TL::WM;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 ra[TL::kALoads], rb[TL::kBLoads];

    auto gload = [&](int s) {
        const int kb = koff(s);
#pragma unroll
        for (int j = 0; j < TL::kALoads; ++j) {
            const int off = kb + st.cA[j] * 16;
            ra[j] = (st.a[j] && off < kvalid) ? ld16(st.a[j] + off) : zero;
        }
#pragma unroll
        for (int j = 0; j < TL::kBLoads; ++j) {
            const int off = kb + st.cB[j] * 16;
            rb[j] = (st.b[j] && off < kvalid) ? ld16(st.b[j] + off) : zero;
        }
    };
    auto sstore = [&](int stage) {
        u32x4 *base = lds + stage * TL::kStage;
#pragma unroll
        for (int j = 0; j < TL::kALoads; ++j) base[st.sA[j]] = ra[j];
#pragma unroll
        for (int j = 0; j < TL::kBLoads; ++j) base[st.sB[j]] = rb[j];
    };

    if (nsteps <= 0) return;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        if (s + 1 < nsteps) gload(s + 1);
        const u32x4 *A = lds + (s & 1) * TL::kStage;
        const u32x4 *B = A + TL::kAChunks;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            u32x4 fa[TL::TM], fb[TL::TN];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm) fa[tm] = A[lds_slot(wm * TL::kWaveM + tm * 32 + (lane & 31), c)];
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) fb[tn] = B[lds_slot(wn * TL::kWaveN + tn * 32 + (lane & 31), c)];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TL::TN; ++tn) Mfma<T>::step(fa[tm], fb[tn], acc[tm][tn]);
        }
        after(s);
        if (s + 1 < nsteps) sstore((s + 1) & 1);
        __syncthreads();
    }
}

template <class TL>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[TL::TM][TL::TN]) {
#pragma unroll
    for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;
}

// Row of the workgroup tile (M index) held by register r of acc[tm][*] in
// this lane, and column (N index) held by acc[*][tn].
template <class TL>
__device__ __forceinline__ int tile_row(int tm, int r) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave % TL::WM) * TL::kWaveM + tm * 32 + acc_row(r, lane);
}
template <class TL>
__device__ __forceinline__ int tile_col(int tn) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave / TL::WM) * TL::kWaveN + tn * 32 + acc_col(lane);
}

}  // namespace cce
