// gemm_dma.hpp -- the DMA-fed MFMA main loop shared by the INT8 GEMM (i8
// operands, int32 accumulators) and the BF16 GEMM of the full-precision route
// (bf16 operands, fp32 accumulators).  Both operands are K-contiguous rows;
// the loop works in bytes, and one MFMA k-step consumes 32 bytes of a row in
// either type (32 int8 or 16 bf16 values).
//
// Operand rows go from global memory straight into LDS with gfx950's
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane of a
// wave's 1 KB block), so no staging registers and no LDS write instructions
// are needed.  A stage is 128 bytes of every row; the 16-byte chunk kc of row
// r is stored at slot kc ^ ((r >> 1) & 7), which makes the 32-row fragment
// reads conflict-free on the 64-bank LDS.  Two stage buffers: the DMA of stage
// kt+2 goes out during stage kt, one instruction after every two MFMAs, half
// with the last k-step of stage kt and half with the first k-step of stage
// kt+1, and fragments are read one k-step ahead of the MFMAs that use them,
// across stage boundaries too.  Rows past M or N load a clamped row; their
// outputs are never stored.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid.  Workgroup tile 256 x 256,
// wave tile 128 x 128 = 4 x 4 MFMA 32x32 tiles.  The W fragment is the MFMA's
// first operand, so the accumulators come out transposed: lane l holds row
// l % 32 of an A-subtile and 4 consecutive output columns per register group.
//
// K tail (TAIL = true): when K bytes are not a multiple of 128, the last stage
// is partial.  Its chunks past K are loaded from the stage's first chunk (in
// bounds) and the fragments of its k-steps past K are zeroed in both operands.
//
// Addressing: a DMA source is a scalar base (the operand's tile rows plus the
// stage offset) plus the lane's 32-bit byte offset within those 256 rows
// (K <= 2^22 keeps it below 2^32), so the instruction takes the scalar-base
// form and the loop does no 64-bit vector address arithmetic.
#pragma once

#include "device.hpp"
#include "gemm_common.hpp"

namespace dmpq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace gdma {
constexpr int BM = 256, BN = 256, BK = 128;  // BK: bytes of every row per stage
constexpr int TILE = BM * BK;                // bytes per operand per stage
constexpr int STAGE = 2 * TILE;              // A tile + W tile
constexpr int NBUF = 2;
constexpr int BLOCKS = TILE / 1024 / 4;      // 1 KB load blocks per wave per operand
constexpr size_t LDS_BYTES = NBUF * STAGE > 4 * EpiBand<4>::BYTES ? NBUF * STAGE : 4 * EpiBand<4>::BYTES;
constexpr unsigned GROUP_M = 8;
}  // namespace gdma

struct OpI8 {
    typedef v16i acc_t;
    __device__ static __forceinline__ void mfma(acc_t &c, const v4i &a, const v4i &w) {
        c = __builtin_amdgcn_mfma_i32_32x32x32_i8(w, a, c, 0, 0, 0);
    }
};

struct OpBF16 {
    typedef v16f acc_t;
    __device__ static __forceinline__ void mfma(acc_t &c, const v4i &a, const v4i &w) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, w),
                                                    __builtin_bit_cast(v8bf, a), c, 0, 0, 0);
    }
};

__device__ __forceinline__ int swz128(int row, int kc) { return kc ^ ((row >> 1) & 7); }

// waitcnt immediate that waits for at most n outstanding vector memory ops
// (expcnt and lgkmcnt left free)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Per-lane state: DMA sources (the tile's scalar bases and the lane's byte
// offsets from them: its row and chunk) and fragment rows.
struct DmaLane {
    const uint8_t *A, *W;                           // first rows of the A and W tiles
    uint32_t goA[gdma::BLOCKS], goW[gdma::BLOCKS];  // the lane's DMA byte offsets
    int kc[gdma::BLOCKS];  // the lane's 16-byte chunk of its DMA rows
    int offA, offW;        // byte offset of the lane's first fragment row (A; W incl. the A tile)
    int sw, hk;            // swizzle key of the lane's rows, K half
    int wave;              // wave index (uniform)
};

// Fragments of k-step s (32 bytes of each row) of the stage in `buf`.  Rows
// ra = wm*128 + 32i + lane%32 all share the swizzle key ((lane%32) >> 1) & 7,
// so the row block i only adds the constant 32*i*BK (an immediate offset).
// TAIL: a k-step at or past the stage's valid bytes reads as zeros.
template <bool TAIL>
__device__ __forceinline__ void dma_frags(const uint8_t *buf, const DmaLane &L, int s, int valid,
                                          v4i a[4], v4i b[4]) {
    using namespace gdma;
    const int slot = ((2 * s + L.hk) ^ L.sw) * 16;
    const uint8_t *pa = buf + L.offA + slot;
    const uint8_t *pb = buf + L.offW + slot;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        a[i] = *reinterpret_cast<const v4i *>(pa + i * 32 * BK);
        b[i] = *reinterpret_cast<const v4i *>(pb + i * 32 * BK);
        if (TAIL && 32 * s >= valid) {
            a[i] = (v4i){0, 0, 0, 0};
            b[i] = (v4i){0, 0, 0, 0};
        }
    }
}

// One DMA instruction of a stage at byte offset k0 of every row: the q-th
// 1 KB block of operand op (0 = A, 1 = W).  TAIL: a chunk past the row's
// Kb bytes is loaded from the stage's first chunk instead (in bounds: a stage
// holds at least 32 valid bytes; its values are never used).  The empty asm
// statement keeps the scalar base opaque, so that the compiler cannot fold
// the stage offset into a per-lane 64-bit address.
template <bool TAIL>
__device__ __forceinline__ void dma_one(uint8_t *dst, const DmaLane &L, int64_t k0, int64_t Kb,
                                        int q, int op) {
    using namespace gdma;
    typedef __attribute__((address_space(3))) void lds_void;
    const int b = L.wave + 4 * q;
    const uint8_t *base = (op ? L.W : L.A) + k0;
    asm("" : "+s"(base));
    uint32_t off = op ? L.goW[q] : L.goA[q];
    if (TAIL && !(k0 + 16 * L.kc[q] < Kb)) off -= (uint32_t)(16 * L.kc[q]);
    __builtin_amdgcn_global_load_lds((const void *)(base + off), (lds_void *)(dst + op * TILE + b * 1024), 16, 0,
                                     0);
}

template <bool TAIL>
__device__ __forceinline__ void dma_issue(uint8_t *dst, const DmaLane &L, int64_t k0, int64_t Kb) {
#pragma unroll
    for (int q = 0; q < gdma::BLOCKS; q++) {
        dma_one<TAIL>(dst, L, k0, Kb, q, 0);
        dma_one<TAIL>(dst, L, k0, Kb, q, 1);
    }
}

template <class Op>
__device__ __forceinline__ void mfma16(typename Op::acc_t (&acc)[4][4], const v4i a[4], const v4i b[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) Op::mfma(acc[i][j], a[i], b[j]);
}

// 16 MFMAs with half of a stage's DMA (blocks q = 4h .. 4h+3 of both
// operands) placed one instruction after every two MFMAs, so that the
// workgroup's DMA reaches the texture unit spread over the MFMA stream
// instead of in one burst that stalls instruction issue.
template <class Op, bool TAIL>
__device__ __forceinline__ void mfma16_dma(typename Op::acc_t (&acc)[4][4], const v4i a[4],
                                           const v4i b[4], uint8_t *dst, const DmaLane &L,
                                           int64_t k0, int64_t Kb, int h) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            Op::mfma(acc[i][j], a[i], b[j]);
            const int t = 4 * i + j;
            if (t & 1) dma_one<TAIL>(dst, L, k0, Kb, 4 * h + (t >> 2), (t >> 1) & 1);
        }
#pragma unroll
    for (int t = 0; t < 8; t++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 VMEM read (the DMA)
    }
}

// One stage.  On entry a0/b0 and a1/b1 hold k-steps 0 and 1 of the stage in
// `cur`.  With the MFMAs of k-step 0 the wave issues the second half of the
// next stage's DMA into `nxt` (its first half went out with the previous
// stage's last k-step).  After k-step 2 it waits for that DMA and for every
// wave to finish reading `cur`, reads k-step 0 of the next stage, and with the
// MFMAs of k-step 3 issues the first half of the DMA two stages ahead into
// `cur`.  Both DMA halves are issued on every stage so that the MFMA code has
// no branches (the accumulators would not survive them in registers); where
// no such stage exists the caller passes a stage whose bytes the target
// buffer already holds or that nobody reads again, so any read racing with
// it sees unchanged data.  `cur` and `nxt` are separate restrict parameters
// so that, once inlined, the compiler knows the reads of `nxt` cannot alias
// the DMA into `cur` and does not wait for it.  valid_cur / valid_nxt: the
// valid bytes per row of the two stages (BK except a partial last stage).
template <class Op, bool TAIL>
__device__ __forceinline__ void dma_stage(uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt,
                                          bool has_next, int64_t k_second, int64_t k_first,
                                          int64_t Kb, int valid_cur, int valid_nxt,
                                          const DmaLane &L, typename Op::acc_t (&acc)[4][4],
                                          v4i (&a0)[4], v4i (&b0)[4], v4i (&a1)[4], v4i (&b1)[4]) {
    mfma16_dma<Op, TAIL>(acc, a0, b0, nxt, L, k_second, Kb, 1);
    dma_frags<TAIL>(cur, L, 2, valid_cur, a0, b0);
    mfma16<Op>(acc, a1, b1);
    dma_frags<TAIL>(cur, L, 3, valid_cur, a1, b1);
    mfma16<Op>(acc, a0, b0);
    if (has_next) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's DMA of the next stage
        __syncthreads();                           // ... every wave's, and `cur` is free
        dma_frags<TAIL>(nxt, L, 0, valid_nxt, a0, b0);
    }
    mfma16_dma<Op, TAIL>(acc, a1, b1, cur, L, k_first, Kb, 0);
    if (has_next) dma_frags<TAIL>(nxt, L, 1, valid_nxt, a1, b1);
}

// Valid bytes per row of stage kt: BK, or what is left in a partial last stage.
__device__ __forceinline__ int dma_valid(int64_t Kb, int kt) {
    const int64_t left = Kb - (int64_t)kt * gdma::BK;
    return (int)(left < gdma::BK ? left : gdma::BK);
}

// The whole main loop of one workgroup tile over a K range: acc = A[m0.., k]
// W[n0.., k]^T for the Kb bytes of every row that start at A and W (the
// range's first byte; rows are ld bytes apart).  Kb % 32 == 0, and
// Kb % 128 == 0 unless TAIL.  On return every DMA has landed and every wave
// has left the stage buffers, so `lds` is free for the epilogue.  An LDS DMA
// that the workgroup issued before the call (outside the stage buffers) has
// landed and is visible to every wave once the first stage is: the wait for
// that stage counts it, and the barrier after it publishes it.
template <class Op, bool TAIL>
__device__ __forceinline__ void dma_gemm_mainloop(const uint8_t *__restrict__ A,
                                                  const uint8_t *__restrict__ W, int64_t M,
                                                  int64_t N, int64_t ld, int64_t Kb, int64_t m0,
                                                  int64_t n0, uint8_t *lds,
                                                  typename Op::acc_t (&acc)[4][4]) {
    using namespace gdma;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    // Per-lane source offsets of this wave's load blocks: block b = wave + 4q
    // covers tile rows 8b .. 8b+7; lane l fills row 8b + l/8, slot l%8.  Rows
    // past M or N load a clamped row (at or after the tile's first row).
    DmaLane L;
    L.A = A + m0 * ld;
    L.W = W + n0 * ld;
    L.wave = wave;
    L.hk = lane >> 5;
#pragma unroll
    for (int q = 0; q < BLOCKS; q++) {
        const int b = wave + 4 * q;
        const int row = 8 * b + (lane >> 3);
        const int kc = swz128(row, lane & 7);
        const int64_t gm = m0 + row < M ? m0 + row : M - 1;
        const int64_t gn = n0 + row < N ? n0 + row : N - 1;
        L.kc[q] = kc;
        L.goA[q] = (uint32_t)((gm - m0) * ld + kc * 16);
        L.goW[q] = (uint32_t)((gn - n0) * ld + kc * 16);
    }
    L.offA = (wm * 128 + (lane & 31)) * BK;
    L.offW = TILE + (wn * 128 + (lane & 31)) * BK;
    L.sw = ((lane & 31) >> 1) & 7;

    const int nk = (int)((Kb + BK - 1) / BK);
    dma_issue<TAIL>(lds, L, 0, Kb);
    if (nk > 1) {
        dma_issue<TAIL>(lds + STAGE, L, BK, Kb);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * BLOCKS));  // stage 0 only
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    // A bare barrier: __syncthreads() would also wait for the second stage's
    // DMA (its fence covers every outstanding load), which nothing reads yet.
    // The empty asm statements keep the compiler from moving the first
    // stage's LDS reads above it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    v4i a0[4], b0[4], a1[4], b1[4];
    dma_frags<TAIL>(lds, L, 0, dma_valid(Kb, 0), a0, b0);
    dma_frags<TAIL>(lds, L, 1, dma_valid(Kb, 0), a1, b1);
    for (int kt = 0; kt < nk; kt++) {
        // the offsets become opaque values that change (in place, with no
        // instruction) every stage, so their 64-bit extension stays in the
        // loop and each DMA keeps the scalar-base form
#pragma unroll
        for (int q = 0; q < BLOCKS; q++) asm("" : "+v"(L.goA[q]), "+v"(L.goW[q]));
        uint8_t *cur = lds + (kt & 1) * STAGE;
        uint8_t *nxt = lds + ((kt & 1) ^ 1) * STAGE;
        // second half into nxt: stage kt+1 (kt = 0 repeats the prologue's
        // copy of it; after the last stage nxt is never read); first half
        // into cur: stage kt+2, or stage kt itself when there is none
        const int64_t k_second = (int64_t)(kt + 1 < nk ? kt + 1 : nk - 1) * BK;
        const int64_t k_first = (int64_t)(kt + 2 < nk ? kt + 2 : kt) * BK;
        dma_stage<Op, TAIL>(cur, nxt, kt + 1 < nk, k_second, k_first, Kb, dma_valid(Kb, kt),
                            dma_valid(Kb, kt + 1 < nk ? kt + 1 : kt), L, acc, a0, b0, a1, b1);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the last stage's DMA has landed
    __syncthreads();  // every wave is done reading the stage buffers
}

}  // namespace dmpq
