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

// float -> bfloat16, round to nearest, ties to even (gfx950 converts in
// hardware: v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }

// threadIdx.x through an empty asm: the compiler cannot treat values derived
// from it as loop-invariant.
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Order-preserving map of fp32 onto int32 (for non-NaN values): a < b as
// floats iff enc(a) < enc(b) as signed integers, so an integer atomic max
// computes a float max.  dec inverts enc.
__device__ __forceinline__ int bound_enc(float f) {
    const int i = __float_as_int(f);
    return i < 0 ? i ^ 0x7FFFFFFF : i;
}
__device__ __forceinline__ float bound_dec(int i) { return __int_as_float(i < 0 ? i ^ 0x7FFFFFFF : i); }

// Largest of the 64 lanes' values, returned to every lane (a wave-uniform
// value).  DPP row operations of the GFX9 family: max within quads, within
// half-rows and rows by mirroring, then across the four rows by the row-15
// and row-31 broadcasts, which leave the wave maximum in lane 63.
__device__ __forceinline__ int wave_max_i32(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1, 0, 3, 2]
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2, 3, 0, 1]
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false));  // row_mirror
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));  // row_bcast:15 into rows 1, 3
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));  // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}

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

// Row v of a classifier (or of its gradient) held as one matrix or as the two
// row blocks of a composite head: rows v < v0 in the first block, the others
// at v - v0 in the second.  ld = elements per row.
template <typename P>
struct Rows2 {
    P *r0;
    P *r1;
    int64_t v0;
    int64_t ld;
    __device__ __forceinline__ P *row(int64_t v) const { return v < v0 ? r0 + v * ld : r1 + (v - v0) * ld; }
};

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

// LDS position (in 16-byte chunks) of chunk c of row r.  Rows are 128 bytes;
// the chunk is XOR-swizzled with f(r) = (r & 7) ^ ((r >> 3) & 1), so that the
// 8 or 16 rows one ds_read_b128 services together (lanes l % 32 = row) all
// fall in distinct 16-byte bank groups, whether the LDS serves 128 or 256
// bytes per clock.
__device__ __forceinline__ int lds_slot(int r, int c) { return r * 8 + (c ^ ((r & 7) ^ ((r >> 3) & 1))); }

__device__ __forceinline__ u32x4 ld16(const char *p) { return *reinterpret_cast<const u32x4 *>(p); }

// One workgroup's side of the K loop: global -> registers -> LDS staging of
// the A and B rows, and the MFMA over one LDS stage.
//  - Thread t stages 16-byte chunk (t & 7) of rows (t >> 3) + (threads / 8) j.
//  - pa[j] / pb[j] are the row base pointers of load j for the current tile
//    (null = row past the end: stages zeros).
//  - load(kb, kvalid): chunk at byte kb + 16 (t & 7) of every row, zero at or
//    beyond kvalid bytes.
template <typename T, class TL>
struct Engine {
    static constexpr int NA = TL::kALoads, NB = TL::kBLoads;
    static constexpr int kRowStep = TL::kThreads / 8;
    const char *pa[NA];
    const char *pb[NB];
    u32x4 ra[NA], rb[NB];
    int c16, slot0;

    __device__ __forceinline__ Engine() {
        const int t = threadIdx.x;
        c16 = (t & 7) * 16;
        slot0 = lds_slot(t >> 3, t & 7);  // row r0 + kRowStep j keeps r0's swizzle (kRowStep % 16 == 0)
        static_assert(kRowStep % 16 == 0, "row step must preserve the swizzle phase");
    }
    static __device__ __forceinline__ int row(int j) { return (threadIdx.x >> 3) + kRowStep * j; }

    __device__ __forceinline__ void load(int kb, int kvalid) {
        const int off = kb + c16;
        const bool kok = off < kvalid;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NA; ++j) ra[j] = (pa[j] && kok) ? ld16(pa[j] + off) : z;
#pragma unroll
        for (int j = 0; j < NB; ++j) rb[j] = (pb[j] && kok) ? ld16(pb[j] + off) : z;
    }
    __device__ __forceinline__ void store(u32x4 *stage) const {
#pragma unroll
        for (int j = 0; j < NA; ++j) stage[slot0 + 8 * kRowStep * j] = ra[j];
#pragma unroll
        for (int j = 0; j < NB; ++j) stage[TL::kAChunks + slot0 + 8 * kRowStep * j] = rb[j];
    }
    __device__ __forceinline__ void compute(const u32x4 *stage, f32x16 (&acc)[TL::TM][TL::TN]) const {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int ra0 = (wave % TL::WM) * TL::kWaveM + (lane & 31);
        const int rb0 = (wave / TL::WM) * TL::kWaveN + (lane & 31);
        const u32x4 *A = stage;
        const u32x4 *B = stage + TL::kAChunks;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            u32x4 fa[TL::TM], fb[TL::TN];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm) fa[tm] = A[lds_slot(ra0 + tm * 32, c)];
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) fb[tn] = B[lds_slot(rb0 + tn * 32, c)];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TL::TN; ++tn) Mfma<T>::step(fa[tm], fb[tn], acc[tm][tn]);
        }
    }
};

// ------------------------------------------------------- DMA K pipeline
// gfx950 moves 16 bytes per lane straight from global memory into LDS
// (global_load_lds_dwordx4): lane i of a wave-instruction lands at
// base + 16 i.  The pipeline keeps kStages LDS stages of kRowBytes K-bytes per
// row and kStages - 1 of them in flight, so no VGPR staging is needed.
//
// Stage layout: rows of kRowBytes (64 or 128 bytes, 4 or 8 chunks of 16);
// chunk c of row r sits at position c ^ g(r), chosen so that the 8 or 16
// rows one ds_read_b128 services together fall in distinct bank groups
// (64-byte rows: g(r) = ((r >> 1) ^ (r >> 2)) & 3; 128-byte rows:
// g(r) = (r & 7) ^ ((r >> 3) & 1)).  The swizzle is applied on the global
// side: lane i of an instruction fetches the logical chunk that belongs at
// slot base + i.
//
// Synchronisation: each wave waits for its own DMAs of the stage with
// s_waitcnt vmcnt, then s_barrier; the barrier also certifies that every wave
// finished reading the stage the next DMA overwrites.  The empty asm
// statements keep the compiler from moving memory operations across.
typedef __attribute__((address_space(3))) void lds_void_t;

template <int kRowBytes>
__device__ __forceinline__ int dma_swz(int r) {
    if constexpr (kRowBytes == 64) return ((r >> 1) ^ (r >> 2)) & 3;
    else if constexpr (kRowBytes == 96) return 0;  // 6 chunks: 8 consecutive rows already hit distinct banks
    else return (r & 7) ^ ((r >> 3) & 1);
}
template <int kRowBytes>
__device__ __forceinline__ int dma_slot(int r, int c) {
    return r * (kRowBytes / 16) + (c ^ dma_swz<kRowBytes>(r));
}

// One wave-instruction of global -> LDS DMA: this lane's 16 bytes at src go
// to wave_dst + 16 * lane (wave_dst is the same for the whole wave).  Issued
// as inline assembly so that the compiler's wait-count pass does not treat
// every later LDS read as dependent on it; the pipeline waits explicitly.
// M0 holds the LDS address; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_at(const char *src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "memory", "m0");
}
// Wave-uniform read of a[i] through the scalar data cache (an SMEM load,
// counted by lgkmcnt).  A vector load would be counted by vmcnt together with
// the LDS-DMA stages in flight, and waiting for it would drain them.  Only for
// data no kernel of the launch writes.
__device__ __forceinline__ int32_t uniform_load(const int32_t *a, int64_t i) {
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    return ((const_i32 *)a)[i];
}
// LDS byte address (32 bits, wave-uniform) of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t *)p);
}
__device__ __forceinline__ void dma16(const char *src, u32x4 *wave_dst) { dma16_at(src, lds_addr(wave_dst)); }
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x3F70 | (N & 0xF) | ((N >> 4) << 14));
}
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename T, class TL, int kRowBytes_ = 64, int kStages_ = 4>
struct DmaEngine {
    static constexpr int kStages = kStages_;
    static constexpr int kDepth = kStages - 1;  // stages in flight ahead of the one computed
    static constexpr int kStageBytes = kRowBytes_;
    static constexpr int kCpr = kRowBytes_ / 16;  // chunks per row
    static constexpr int kStageA = TL::BM * kCpr;  // chunks of A per stage
    static constexpr int kStageB = TL::BN * kCpr;
    static constexpr int kStage = kStageA + kStageB;
    static constexpr int kLdsChunks = kStages * kStage;
    static constexpr int NIA = kStageA / 64 / TL::kWaves;  // DMA instructions per wave per stage
    static constexpr int NIB = kStageB / 64 / TL::kWaves;
    static constexpr int NI = NIA + NIB;
    static_assert(kRowBytes_ == 64 || kRowBytes_ == 96 || kRowBytes_ == 128, "64-, 96- or 128-byte stage rows");
    static_assert(kStages >= 2 && kStages <= 4, "2 to 4 stages");
    static_assert(NIA * 64 * TL::kWaves == kStageA && NIB * 64 * TL::kWaves == kStageB,
                  "tile rows must split into whole wave-instructions");

    const char *pa[NIA];  // this lane's source address (row base + swizzled chunk) at K offset 0
    const char *pb[NIB];
    u32x4 *lds;
    uint32_t lds0;        // LDS byte address of the stages (wave-uniform)

    __device__ __forceinline__ explicit DmaEngine(u32x4 *l) : lds(l), lds0(lds_addr(l)) {}

    // Tile row fed by this lane in instruction j, and the byte offset of its
    // chunk: lane i of instruction j fills stage slot 64 (j waves + wave) + i,
    // which is row slot / kCpr, position slot % kCpr.
    static __device__ __forceinline__ int slot_of(int j, int tid) { return 64 * (j * TL::kWaves + (tid >> 6)) + (tid & 63); }
    static __device__ __forceinline__ int row_a(int j, int tid = threadIdx.x) { return slot_of(j, tid) / kCpr; }
    static __device__ __forceinline__ int row_b(int j, int tid = threadIdx.x) { return row_a(j, tid); }
    static __device__ __forceinline__ int chunk_off(int j, int r, int tid) {
        return 16 * ((slot_of(j, tid) % kCpr) ^ dma_swz<kRowBytes_>(r));
    }

    __device__ __forceinline__ void issue(int buf, int kb) const { issue2(buf, kb, kb); }

    // Half of the A (or B) rows that instruction j fills (every wave's part of
    // instruction j lies in one half).
    static constexpr int kRowsPerInstr = 64 * TL::kWaves / kCpr;
    static constexpr int half_a(int j) { return j * kRowsPerInstr / (TL::BM / 2); }
    static constexpr int half_b(int j) { return j * kRowsPerInstr / (TL::BN / 2); }
    // issue() for only some halves of the tile: bit h of `halves` = A rows
    // [h BM/2, (h+1) BM/2), bit 2 + h = the same for B.  Uniform over the
    // workgroup; the rows left out keep whatever the stage held.
    __device__ __forceinline__ void issue_halves(int buf, int kb, int halves) const {
        static_assert((TL::BM / 2) % kRowsPerInstr == 0 && (TL::BN / 2) % kRowsPerInstr == 0,
                      "an instruction's rows lie in one half");
        const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t st = lds0 + (uint32_t)(buf * kStage) * 16u;
#pragma unroll
        for (int j = 0; j < NIA; ++j)
            if ((halves >> half_a(j)) & 1) dma16_at(pa[j] + kb, st + 1024u * (j * TL::kWaves + w));
#pragma unroll
        for (int j = 0; j < NIB; ++j)
            if ((halves >> (2 + half_b(j))) & 1)
                dma16_at(pb[j] + kb, st + 16u * kStageA + 1024u * (j * TL::kWaves + w));
    }
    // The same with separate byte offsets for the A and the B rows.
    __device__ __forceinline__ void issue2(int buf, int64_t kba, int64_t kbb) const {
        const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t st = lds0 + (uint32_t)(buf * kStage) * 16u;
#pragma unroll
        for (int j = 0; j < NIA; ++j) dma16_at(pa[j] + kba, st + 1024u * (j * TL::kWaves + w));
#pragma unroll
        for (int j = 0; j < NIB; ++j) dma16_at(pb[j] + kbb, st + 16u * kStageA + 1024u * (j * TL::kWaves + w));
    }

    // Wait until at most `ahead` later stages are still in flight for this
    // wave (ahead <= kDepth - 1), then barrier.
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

    // The MFMAs of K-slices [kk0, kk1) of stage buf (32 bytes of every row per
    // slice, in K order).
    __device__ __forceinline__ void compute(int buf, f32x16 (&acc)[TL::TM][TL::TN], int tid = threadIdx.x,
                                           int kk0 = 0, int kk1 = kCpr / 2) const {
        const int lane = tid & 63, wave = tid >> 6;
        const int ra0 = (wave % TL::WM) * TL::kWaveM + (lane & 31);
        const int rb0 = (wave / TL::WM) * TL::kWaveN + (lane & 31);
        const u32x4 *A = lds + buf * kStage;
        const u32x4 *B = A + kStageA;
#pragma unroll
        for (int kk = kk0; kk < kk1; ++kk) {
            const int c = 2 * kk + (lane >> 5);
            u32x4 fa[TL::TM], fb[TL::TN];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm) fa[tm] = A[dma_slot<kRowBytes_>(ra0 + tm * 32, c)];
#pragma unroll
            for (int tn = 0; tn < TL::TN; ++tn) fb[tn] = B[dma_slot<kRowBytes_>(rb0 + tn * 32, c)];
#pragma unroll
            for (int tm = 0; tm < TL::TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TL::TN; ++tn) Mfma<T>::step(fa[tm], fb[tn], acc[tm][tn]);
        }
    }
};

// The MFMAs of a whole stage for the accumulator rows tm with bit tm of
// rows set (wave-uniform); the other rows' operands are not read.
template <typename T, class TL, class DE>
__device__ __forceinline__ void compute_rows(const DE &eng, int buf, f32x16 (&acc)[TL::TM][TL::TN], int tid,
                                             uint32_t rows) {
    constexpr int kRowBytes = DE::kStageBytes;
    const int lane = tid & 63, wave = tid >> 6;
    const int ra0 = (wave % TL::WM) * TL::kWaveM + (lane & 31);
    const int rb0 = (wave / TL::WM) * TL::kWaveN + (lane & 31);
    const u32x4 *A = eng.lds + buf * DE::kStage;
    const u32x4 *B = A + DE::kStageA;
#pragma unroll
    for (int kk = 0; kk < DE::kCpr / 2; ++kk) {
        const int c = 2 * kk + (lane >> 5);
        u32x4 fa[TL::TM], fb[TL::TN];
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
            if ((rows >> tm) & 1) fa[tm] = A[dma_slot<kRowBytes>(ra0 + tm * 32, c)];
#pragma unroll
        for (int tn = 0; tn < TL::TN; ++tn) fb[tn] = B[dma_slot<kRowBytes>(rb0 + tn * 32, c)];
#pragma unroll
        for (int tm = 0; tm < TL::TM; ++tm)
            if ((rows >> tm) & 1)
#pragma unroll
                for (int tn = 0; tn < TL::TN; ++tn) Mfma<T>::step(fa[tm], fb[tn], acc[tm][tn]);
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
// The tid argument lets a caller pass a thread index it has made opaque
// (so that per-lane address arithmetic is redone in each iteration of a
// persistent loop instead of being hoisted into registers for all of it).
template <class TL>
__device__ __forceinline__ int tile_row(int tm, int r, int tid = threadIdx.x) {
    const int lane = tid & 63, wave = tid >> 6;
    return (wave % TL::WM) * TL::kWaveM + tm * 32 + acc_row(r, lane);
}
// Row of register r of acc[tm][*] within the wave's sub-tile, without the
// lane term: tile_row = wave row base + 4 (lane / 32) + acc_row_const(tm, r).
// A compile-time constant, so a bound check against a per-lane limit costs
// one compare with an immediate.
__device__ __forceinline__ constexpr int acc_row_const(int tm, int r) { return tm * 32 + 8 * (r >> 2) + (r & 3); }

// Per-lane limit: acc[tm][*][r] holds tile row < rows iff acc_row_const(tm, r) < row_limit(rows).
template <class TL>
__device__ __forceinline__ int row_limit(int rows, int tid = threadIdx.x) {
    const int lane = tid & 63, wave = tid >> 6;
    return rows - (wave % TL::WM) * TL::kWaveM - 4 * (lane >> 5);
}

template <class TL>
__device__ __forceinline__ int tile_col(int tn, int tid = threadIdx.x) {
    const int lane = tid & 63, wave = tid >> 6;
    return (wave / TL::WM) * TL::kWaveN + tn * 32 + acc_col(lane);
}

}  // namespace cce
