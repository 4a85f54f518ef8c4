// The K loop of the 4-wave MFMA kernels on gfx950: 256 x 256 logit tiles,
// C = A B^T with A = classifier rows (MFMA M side) and B = token rows (N
// side), both K-contiguous bf16, on 4 waves of 128 x 128 (wave w: rows
// 128 (w % 2), tokens 128 (w / 2)), 256 fp32 accumulators per lane in AGPRs.
// Used by the forward (k_fwd4), whose per-tile epilogue is light enough to
// run with nothing to overlap it.
#pragma once

#include "cce_device.hpp"

// k_fwd4 serves bf16 whenever the DMA path applies; building with
// -DCCE_K4=0 puts the 8-wave k_fwd_dma there instead (for comparisons).
#ifndef CCE_K4
#define CCE_K4 1
#endif

namespace cce {

using Tile4 = Tile<256, 256, 2, 2>;

// Per 128 bytes of K the waves read 128 KB of operand
// fragments from LDS instead of the 8-wave layout's 192 KB.  With one wave
// per SIMD nothing else hides the LDS latency, the barrier or the DMA issue
// (a wave whose next instruction is a DMA that the memory pipeline cannot
// take yet stalls, MFMAs included), so the K loop is written as assembly
// blocks whose order is fixed here.
//
// K is streamed in half-stages of 64 bytes per row (two K-slices of 32 bytes,
// 16 MFMAs of 32x32x16 each) through 4 LDS buffers of 32 KB (A rows, then B
// rows, 64-byte rows with the dma_swz<64> chunk swizzle).  Half-stage h sits
// in buffer h % 4.  Its slice a reads slice b's fragments under its MFMAs;
// then every wave waits for its DMA of half-stage h + 1 and meets the others
// at a barrier (h + 1 is in LDS, and nobody reads buffer h % 4 any more);
// slice b reads h + 1's first fragments (except in a tile's last half-stage:
// those are read after the tile's epilogue, so that they are not live across
// it).  The DMA of half-stage h + 4 into buffer h % 4 is spread evenly: its
// A rows (4 instructions per wave) under slice b of h, its B rows under slice
// a of h + 1, one instruction per 4 MFMAs.  A tile's first half-stage starts
// its MFMAs from zero (src2 = 0), so no accumulator is cleared.
//
// Fragments: P holds a half-stage's slice-a fragments on entry (A rows of
// blocks tm = 0-3 in P0-P3, B rows of tn = 0-3 in P4-P7), Q is scratch.
// Hazards the blocks respect themselves: each slice waits for its own LDS
// reads before the next slice's MFMAs use them; a slice uses each accumulator
// once, 16 MFMAs from its next use; the results are read by vector
// instructions only after acc_settle's wait states.
#define CCE_MF(c, a, b) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[" #b "], %[" #c "]\n\t"
#define CCE_MFZ(c, a, b) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[" #b "], 0\n\t"
#define CCE_RD(n, r, off) "ds_read_b128 %[" #n "], %[" #r "] offset:" #off "\n\t"
// LDS byte addresses of a slice's A and B fragment rows: wave base + lane offset.
#define CCE_ADDR(x, a, b) "v_add_u32 %[ra], %[" #a "], %[" #x "]\n\tv_add_u32 %[rb], %[" #b "], %[" #x "]\n\t"
// One DMA instruction: row pointer + the half-stage's K offset, to LDS m0 = mb + moff.
#define CCE_DMA(p, moff, t, kb, mb)                                                                         \
    "v_lshl_add_u64 %[" #t "], %[" #p "], 0, %[" #kb "]\n\ts_add_u32 m0, %[" #mb "], " #moff                 \
    "\n\tglobal_load_lds_dwordx4 %[" #t "], off\n\t"
#define CCE_WAIT_LDS "s_waitcnt lgkmcnt(0)\n\t"

// A slice: 16 MFMAs on fragments C (tm-major), the next slice's 8 reads into
// N after the first 8, and 4 DMA instructions (row pointers P0-P3 at LDS
// offsets O0-O3 from mb).
#define CCE_SLICE(MF, C, N, P0, P1, P2, P3, KB, MB, O0, O1, O2, O3)                                         \
    MF(c00, C##0, C##4) CCE_RD(N##0, ra, 0) MF(c01, C##0, C##5) CCE_RD(N##1, ra, 2048)                      \
    CCE_DMA(P0, O0, t0, KB, MB) MF(c02, C##0, C##6) CCE_RD(N##2, ra, 4096) MF(c03, C##0, C##7)              \
    CCE_RD(N##3, ra, 6144) MF(c10, C##1, C##4) CCE_RD(N##4, rb, 0) MF(c11, C##1, C##5) CCE_RD(N##5, rb, 2048) \
    CCE_DMA(P1, O1, t1, KB, MB) MF(c12, C##1, C##6) CCE_RD(N##6, rb, 4096) MF(c13, C##1, C##7)              \
    CCE_RD(N##7, rb, 6144) MF(c20, C##2, C##4) MF(c21, C##2, C##5) CCE_DMA(P2, O2, t0, KB, MB)              \
    MF(c22, C##2, C##6) MF(c23, C##2, C##7) MF(c30, C##3, C##4) MF(c31, C##3, C##5)                        \
    CCE_DMA(P3, O3, t1, KB, MB) MF(c32, C##3, C##6) MF(c33, C##3, C##7) CCE_WAIT_LDS
// ... without the reads.
#define CCE_SLICE_NR(MF, C, P0, P1, P2, P3, KB, MB, O0, O1, O2, O3)                                         \
    MF(c00, C##0, C##4) MF(c01, C##0, C##5) CCE_DMA(P0, O0, t0, KB, MB) MF(c02, C##0, C##6)                 \
    MF(c03, C##0, C##7) MF(c10, C##1, C##4) MF(c11, C##1, C##5) CCE_DMA(P1, O1, t1, KB, MB)                 \
    MF(c12, C##1, C##6) MF(c13, C##1, C##7) MF(c20, C##2, C##4) MF(c21, C##2, C##5)                        \
    CCE_DMA(P2, O2, t0, KB, MB) MF(c22, C##2, C##6) MF(c23, C##2, C##7) MF(c30, C##3, C##4)                 \
    MF(c31, C##3, C##5) CCE_DMA(P3, O3, t1, KB, MB) MF(c32, C##3, C##6) MF(c33, C##3, C##7)

// A half-stage: slice a (MF0: from zero or accumulating) with the pending B
// rows' DMA, the wait for half-stage h + 1 (the 16 DMA instructions issued
// after its last one may still be in flight) and the barrier, then TAIL =
// slice b with the A rows' DMA of half-stage h + 4.
#define CCE_HALF(MF0, TAIL)                                                                                 \
    CCE_ADDR(x1, sa, sb) CCE_SLICE(MF0, p, q, pb0, pb1, pb2, pb3, kbb, mbb, 16384, 20480, 24576, 28672)    \
    "s_waitcnt vmcnt(16)\n\ts_barrier\n\t" TAIL
#define CCE_TAIL_NEXT CCE_ADDR(x0, na, nb) CCE_SLICE(CCE_MF, q, p, pa0, pa1, pa2, pa3, kba, mba, 0, 4096, 8192, 12288)
#define CCE_TAIL_LAST CCE_SLICE_NR(CCE_MF, q, pa0, pa1, pa2, pa3, kba, mba, 0, 4096, 8192, 12288)
// A whole half-stage's DMA (prologue), and its A rows only.
#define CCE_DMA_A                                                                                           \
    CCE_DMA(pa0, 0, t0, kba, mba) CCE_DMA(pa1, 4096, t1, kba, mba) CCE_DMA(pa2, 8192, t0, kba, mba)         \
    CCE_DMA(pa3, 12288, t1, kba, mba)
#define CCE_DMA_B                                                                                           \
    CCE_DMA(pb0, 16384, t0, kba, mba) CCE_DMA(pb1, 20480, t1, kba, mba) CCE_DMA(pb2, 24576, t0, kba, mba)   \
    CCE_DMA(pb3, 28672, t1, kba, mba)
#define CCE_READ_ONLY                                                                                       \
    CCE_ADDR(x0, na, nb) CCE_RD(p0, ra, 0) CCE_RD(p1, ra, 2048) CCE_RD(p2, ra, 4096) CCE_RD(p3, ra, 6144)   \
    CCE_RD(p4, rb, 0) CCE_RD(p5, rb, 2048) CCE_RD(p6, rb, 4096) CCE_RD(p7, rb, 6144) CCE_WAIT_LDS

#define CCE_ACC(K, acc)                                                                                     \
    [c00] K(acc[0][0]), [c01] K(acc[0][1]), [c02] K(acc[0][2]), [c03] K(acc[0][3]), [c10] K(acc[1][0]),     \
        [c11] K(acc[1][1]), [c12] K(acc[1][2]), [c13] K(acc[1][3]), [c20] K(acc[2][0]), [c21] K(acc[2][1]), \
        [c22] K(acc[2][2]), [c23] K(acc[2][3]), [c30] K(acc[3][0]), [c31] K(acc[3][1]), [c32] K(acc[3][2]), \
        [c33] K(acc[3][3])
#define CCE_FRAGS(n, K, f)                                                                                  \
    [n##0] K(f[0]), [n##1] K(f[1]), [n##2] K(f[2]), [n##3] K(f[3]), [n##4] K(f[4]), [n##5] K(f[5]),         \
        [n##6] K(f[6]), [n##7] K(f[7])
#define CCE_PTRS(pa, pb)                                                                                    \
    [pa0] "v"(pa[0]), [pa1] "v"(pa[1]), [pa2] "v"(pa[2]), [pa3] "v"(pa[3]), [pb0] "v"(pb[0]),               \
        [pb1] "v"(pb[1]), [pb2] "v"(pb[2]), [pb3] "v"(pb[3])
#define CCE_K_INOUT_A(x) "+a"(x)
#define CCE_K_OUT_A(x) "=a"(x)
#define CCE_K_INOUT_V(x) "+v"(x)
#define CCE_K_TMP_V(x) "=&v"(x)

typedef f32x16 Acc4[4][4];

// The scalar operands of a half-stage.
struct F4Half {
    uint32_t sa, sb;    // LDS byte address of this wave's A / B fragment rows in the half-stage's buffer
    uint32_t na, nb;    // the same in the next half-stage's buffer
    uint32_t mba;       // LDS byte address of the buffer the A rows' DMA fills, plus 1024 * wave
    uint32_t mbb;       // the same for the pending B rows' DMA
    uint64_t kba, kbb;  // K byte offsets of those two DMAs
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#define CCE_F4_HALF_FN(name, ACCK, MF0, TAIL)                                                              \
    __device__ __forceinline__ void name(Acc4 &acc, u32x4 (&P)[8], const uint32_t (&x)[2], const F4Half &g, \
                                         const char *const (&pa)[4], const char *const (&pb)[4]) {           \
        u32x4 Q[8];                                                                                         \
        uint32_t ra, rb;                                                                                    \
        uint64_t t0, t1;                                                                                    \
        asm volatile(CCE_HALF(MF0, TAIL)                                                                    \
                     : CCE_ACC(ACCK, acc), CCE_FRAGS(p, CCE_K_INOUT_V, P), CCE_FRAGS(q, CCE_K_TMP_V, Q),    \
                       [ra] "=&v"(ra), [rb] "=&v"(rb), [t0] "=&v"(t0), [t1] "=&v"(t1)                       \
                     : [x0] "v"(x[0]), [x1] "v"(x[1]), [sa] "s"(g.sa), [sb] "s"(g.sb), [na] "s"(g.na),       \
                       [nb] "s"(g.nb), [mba] "s"(g.mba), [mbb] "s"(g.mbb), [kba] "s"(g.kba), [kbb] "s"(g.kbb), \
                       CCE_PTRS(pa, pb)                                                                     \
                     : "memory", "m0", "scc");                                                             \
    }
CCE_F4_HALF_FN(f4_half_first, CCE_K_OUT_A, CCE_MFZ, CCE_TAIL_NEXT)
CCE_F4_HALF_FN(f4_half_next, CCE_K_INOUT_A, CCE_MF, CCE_TAIL_NEXT)
CCE_F4_HALF_FN(f4_half_last, CCE_K_INOUT_A, CCE_MF, CCE_TAIL_LAST)
#undef CCE_F4_HALF_FN

// Prologue DMA of one half-stage: its A rows, and (B) its B rows too.
template <bool B>
__device__ __forceinline__ void f4_dma(uint32_t mba, uint64_t kba, const char *const (&pa)[4],
                                       const char *const (&pb)[4]) {
    uint64_t t0, t1;
    if constexpr (B)
        asm volatile(CCE_DMA_A CCE_DMA_B : [t0] "=&v"(t0), [t1] "=&v"(t1)
                     : [mba] "s"(mba), [kba] "s"(kba), CCE_PTRS(pa, pb) : "memory", "m0", "scc");
    else
        asm volatile(CCE_DMA_A : [t0] "=&v"(t0), [t1] "=&v"(t1)
                     : [mba] "s"(mba), [kba] "s"(kba), CCE_PTRS(pa, pb) : "memory", "m0", "scc");
}
// Reads a half-stage's slice-a fragments into P (x0 = the lane's slice-a offset).
__device__ __forceinline__ void f4_read(u32x4 (&P)[8], uint32_t x0, uint32_t na, uint32_t nb) {
    uint32_t ra, rb;
    asm volatile(CCE_READ_ONLY : CCE_FRAGS(p, CCE_K_TMP_V, P), [ra] "=&v"(ra), [rb] "=&v"(rb)
                 : [x0] "v"(x0), [na] "s"(na), [nb] "s"(nb) : "memory");
}
// Wait states between the last MFMAs of a tile and the vector instructions
// that read or overwrite their results (the MFMA latency is not interlocked).
__device__ __forceinline__ void acc_settle(Acc4 &acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : CCE_ACC(CCE_K_INOUT_A, acc));
}
#pragma clang diagnostic pop

// One accumulator value into a vector register.  (Through an assembly
// statement: reading the accumulators as plain values, the compiler copied
// all 256 of them to vector registers at once, ahead of the per-column
// loop, and spilled.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ float acc_read(const f32x16 &v, int r) {
    float o;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(o) : "a"(v[r]));
    return o;
}
#pragma clang diagnostic pop

// The K loop over logit tiles t0 .. t0 + ntile - 1 of the processing order
// (A: classifier rows p = vt * 256 + r, through perm when given, clamped to
// V - 1) against token tile tok0 (B: rows idx[tok0 + r], clamped to nv - 1).
// After each tile's MFMAs, epi(ct, acc) runs on the settled accumulators
// while the DMA of the next tile's first half-stages is in flight.  Returns
// with every DMA complete and no LDS access pending, so the caller may reuse
// the LDS.  Needs D * 2 to be a multiple of 128.
template <class Epi>
__device__ __forceinline__ void k4_run(const bf16_t *__restrict__ H, Rows2<const bf16_t> E,
                                       const int32_t *__restrict__ idx, int nv, const int32_t *__restrict__ perm,
                                       int D, int V, int tok0, int t0, int ntile, u32x4 *lds, Epi &&epi) {
    using TL = Tile4;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, held in a scalar register
    const int64_t rowb = (int64_t)D * (int64_t)sizeof(bf16_t);
    const int nh = (int)(rowb / 64);  // half-stages per tile (even: rowb is a multiple of 128)

    // DMA sources: instruction j (0-3) of this wave fills row 64 j + 16 w +
    // lane / 4 of a half-stage's A (and B) rows at position lane % 4, with the
    // logical chunk that the swizzle puts there.
    const char *pa[4], *pb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 64 * j + 16 * w + (lane >> 2);
        pb[j] = reinterpret_cast<const char *>(H) + (int64_t)idx[min(tok0 + r, nv - 1)] * rowb +
                16 * ((lane & 3) ^ dma_swz<64>(r));
    }
    // (Two loops on the uniform perm test: without a permutation no load is
    // issued, so nothing waits for the DMA in flight.)
    auto set_tile = [&](int vt) {
        if (perm) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 64 * j + 16 * w + (lane >> 2);
                int v = perm[min(vt * TL::BM + r, V - 1)];
                v = (v >= 0 && v < V) ? v : 0;
                pa[j] = reinterpret_cast<const char *>(E.row(v)) + 16 * ((lane & 3) ^ dma_swz<64>(r));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 64 * j + 16 * w + (lane >> 2);
                pa[j] = reinterpret_cast<const char *>(E.row(min(vt * TL::BM + r, V - 1))) +
                        16 * ((lane & 3) ^ dma_swz<64>(r));
            }
        }
    };
    // The DMA cursor (tile qt, half-stage qk, global count qg) runs four
    // half-stages ahead of the computation, across tiles; pa / pb point at K
    // offset 0 of their rows and the half-stage's offset qk * 64 is added as
    // each DMA is issued.  Past the last half-stage the cursor stays on it:
    // the extra DMAs re-read it into buffers nobody reads any more, and are
    // waited for before returning.
    int qt = 0, qk = 0, qg = 0;
    auto advance = [&]() {
        ++qg;
        if (++qk < nh) return;
        if (qt + 1 < ntile) {
            qk = 0;
            set_tile(t0 + ++qt);
        } else {
            qk = nh - 1;
        }
    };

    // LDS: the lane's byte offset of its chunk of slice kk in fragment row
    // lane % 32 (a 64-byte row), and the wave's A and B fragment rows.
    const uint32_t lds0 = lds_addr(lds);
    const uint32_t mb0 = lds0 + 1024u * (uint32_t)w;
    uint32_t xk[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        xk[kk] = 64u * (lane & 31) + 16u * ((2 * kk + (lane >> 5)) ^ dma_swz<64>(lane & 31));
    const uint32_t offa = lds0 + 8192u * (uint32_t)(w & 1), offb = lds0 + 16384u + 8192u * (uint32_t)(w >> 1);
    auto buf = [](int h) { return (uint32_t)(h & 3) * 32768u; };

    // Prologue: half-stages 0-2 whole and the A rows of 3.
    set_tile(t0);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        f4_dma<true>(mb0 + buf(qg), (uint64_t)qk * 64u, pa, pb);
        advance();
    }
    uint32_t mbb = mb0 + buf(qg);
    uint64_t kbb = (uint64_t)qk * 64u;
    f4_dma<false>(mbb, kbb, pa, pb);
    advance();
    wait_vmcnt<20>();
    block_sync();

    u32x4 P[8];
    Acc4 acc;
    int h = 0;  // half-stage counter
    auto args = [&]() {
        return F4Half{offa + buf(h), offb + buf(h), offa + buf(h + 1), offb + buf(h + 1),
                      mb0 + buf(qg), mbb, (uint64_t)qk * 64u, kbb};
    };
    // After a half-stage: its A rows' DMA becomes the pending B rows' DMA.
    auto step = [&]() {
        mbb = mb0 + buf(qg);
        kbb = (uint64_t)qk * 64u;
        advance();
        ++h;
    };
    for (int ct = 0; ct < ntile; ++ct) {
        f4_read(P, xk[0], offa + buf(h), offb + buf(h));
        f4_half_first(acc, P, xk, args(), pa, pb);
        step();
        for (int k = 1; k + 1 < nh; ++k) {
            f4_half_next(acc, P, xk, args(), pa, pb);
            step();
        }
        f4_half_last(acc, P, xk, args(), pa, pb);
        step();
        acc_settle(acc);
        epi(ct, acc);
    }
    wait_vmcnt<0>();  // the extra half-stages
}

}  // namespace cce
