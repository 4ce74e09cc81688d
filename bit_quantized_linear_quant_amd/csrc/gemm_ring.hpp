// The main loop of the 256 x 256 tile matrix-core kernels, shared by the
// int8 product (gemm_i8.hip) and the 16-bit products of the Q4Linear
// backward (q4_backward.hip).
//
// Operands are row-major with k contiguous, K bytes per row (K % BK == 0);
// A has rows_a rows, B rows_b, and out = A B^T.  A 256-thread workgroup owns
// a 256 x 256 output tile, each wave a 128 x 128 quarter (wm, wn) held as
// 4 x 4 blocks of a 32 x 32 matrix-core product: 256 accumulators per lane,
// one wave per SIMD.  Every 32-byte k step gives lane l the 16 bytes
// 16(l/32) .. +15 of row l%32 of a block, for the int8 32x32x32 product and
// for the fp16 / bf16 32x32x16 products alike (16 bytes are 16 int8 or 8
// 16-bit values; A and B take the same k positions, so the products are the
// same whatever order the instruction sums them in).
//
// BK-byte k-slices of A and B move from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of NBUF
// slices, so NBUF - 1 slices stream in while the matrix cores consume one;
// one explicit vmcnt wait and one barrier per slice.  In LDS each 16-byte
// chunk c of row r sits at chunk position c ^ swz(r), which puts the 16 rows
// read together by a fragment load in distinct bank groups.  Rows past
// rows_a or rows_b are loaded clamped; their outputs are never stored.
#pragma once

#include "ql_device.hpp"

namespace ql {

constexpr int LB = 256;        // tile rows and columns
constexpr int LThreads = 256;
constexpr int kGroupM = 4;     // tile rows walked together per XCD

typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Matrix-core product kind of the ring.
enum MfmaKind : int { MK_I8 = 0, MK_F16 = 1, MK_BF16 = 2 };

template <int CH>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CH == 4) return ((r >> 1) ^ (r >> 2)) & 3;
    else return (r & 7) ^ ((r >> 3) & 3);
}

template <int BK>
struct BigTile {
    static constexpr int CH = BK / 16;                // 16-byte chunks per LDS row
    static constexpr int TILE = LB * BK;              // bytes of one A or B slice
    static constexpr int PER_WAVE = TILE / 1024 / 4;  // 1 KB direct loads per wave per slice and operand
    static constexpr int S = BK / 32;                 // 32-byte MFMA steps per slice
};

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

template <int MK>
__device__ __forceinline__ v16f mfma32(v4i a, v4i b, v16f c) {
    if constexpr (MK == MK_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0,
                                                      0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                       0, 0, 0);
}

// One k-slice: the direct loads of a later slice into `nxt`, then the MFMAs of
// `cur`, each step's fragments read from LDS while the previous step's
// MFMAs issue.  `cur` and `nxt` are distinct restrict pointers, so the
// compiler does not make the LDS reads of `cur` wait for the loads into `nxt`.
template <int BK, int MK, typename ACC>
__device__ __forceinline__ void big_slice(ACC (&acc)[4][4], const int8_t *__restrict__ cur,
                                          int8_t *__restrict__ nxt, const int8_t *const (&srcA)[BigTile<BK>::PER_WAVE],
                                          const int8_t *const (&srcB)[BigTile<BK>::PER_WAVE], int64_t nxt_k0,
                                          const int (&offA)[BigTile<BK>::S], const int (&offB)[BigTile<BK>::S],
                                          int wave) {
    constexpr int CH = BigTile<BK>::CH, TILE = BigTile<BK>::TILE, PER_WAVE = BigTile<BK>::PER_WAVE;
    constexpr int S = BigTile<BK>::S;
#pragma unroll
    for (int ii = 0; ii < PER_WAVE; ii++) {
        const int inst = wave * PER_WAVE + ii;
        lds_load16(srcA[ii] + nxt_k0, nxt + 1024 * inst);
        lds_load16(srcB[ii] + nxt_k0, nxt + TILE + 1024 * inst);
    }
    v4i fa[2][4], fb[2][4];
    auto frags = [&](int s) {
#pragma unroll
        for (int i = 0; i < 4; i++) fa[s & 1][i] = *reinterpret_cast<const v4i *>(cur + offA[s] + i * 32 * CH * 16);
#pragma unroll
        for (int j = 0; j < 4; j++) fb[s & 1][j] = *reinterpret_cast<const v4i *>(cur + TILE + offB[s] + j * 32 * CH * 16);
    };
    frags(0);
#pragma unroll
    for (int s = 0; s < S; s++) {
        if (s + 1 < S) frags(s + 1);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                if constexpr (MK == MK_I8) acc[i][j] = mfma32(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                else acc[i][j] = mfma32<MK>(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
            }
        // matrix-core issue interleaved with the next step's LDS reads
        if (s + 1 < S) {
#pragma unroll
            for (int q = 0; q < 8; q++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    }
}

// The whole k loop of one 256 x 256 tile at (m0, n0): zeroes `acc`, runs the
// ring over K bytes and leaves every load drained and every wave past a
// barrier, so `smem` may be reused by the epilogue.  `smem` holds NBUF
// stages of 2 * BigTile<BK>::TILE bytes.
template <int BK, int NBUF, int MK, typename ACC>
__device__ __forceinline__ void ring_gemm(ACC (&acc)[4][4], int8_t *smem, const int8_t *A, const int8_t *B,
                                          int64_t rows_a, int64_t rows_b, int64_t K, int64_t m0, int64_t n0, int wm,
                                          int wn, int lane, int wave) {
    constexpr int CH = BigTile<BK>::CH, TILE = BigTile<BK>::TILE, PER_WAVE = BigTile<BK>::PER_WAVE;
    constexpr int S = BigTile<BK>::S;
    constexpr int STAGE = 2 * TILE;
    const int64_t nk = K / BK;

    // Global source of each direct load issued by this lane (for k = 0).
    const int8_t *srcA[PER_WAVE];
    const int8_t *srcB[PER_WAVE];
#pragma unroll
    for (int ii = 0; ii < PER_WAVE; ii++) {
        const int pos = 64 * (wave * PER_WAVE + ii) + lane;   // chunk position in the slice
        const int row = pos / CH;
        const int c = (pos % CH) ^ swz<CH>(row);
        const int64_t ra = min(m0 + row, rows_a - 1), rb = min(n0 + row, rows_b - 1);
        srcA[ii] = A + ra * K + 16 * c;
        srcB[ii] = B + rb * K + 16 * c;
    }
    // LDS byte offsets of this lane's fragments: block row 32i + lane%32,
    // chunk 2s + lane/32.  swz depends only on the low 5 row bits, so the
    // offset of block i is that of block 0 plus 32 rows.
    const int fr = lane % 32;
    int offA[S], offB[S];
#pragma unroll
    for (int s = 0; s < S; s++) {
        const int c = 2 * s + lane / 32;
        const int ra = wm * 128 + fr, rb = wn * 128 + fr;
        offA[s] = 16 * (CH * ra + (c ^ swz<CH>(ra)));
        offB[s] = 16 * (CH * rb + (c ^ swz<CH>(rb)));
    }

#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = ACC{};

    // Slices 0 .. NBUF-2 in flight before the loop; iteration kt consumes
    // slice kt and starts slice kt + NBUF - 1 (clamped: the last iterations
    // reload the final slice, keeping the loop body free of branches) into
    // the buffer that iteration kt - 1 consumed.
#pragma unroll
    for (int b = 0; b < NBUF - 1; b++) {
        const int64_t k0 = (int64_t)(b < nk ? b : nk - 1) * BK;
#pragma unroll
        for (int ii = 0; ii < PER_WAVE; ii++) {
            const int inst = wave * PER_WAVE + ii;
            lds_load16(srcA[ii] + k0, smem + b * STAGE + 1024 * inst);
            lds_load16(srcB[ii] + k0, smem + b * STAGE + TILE + 1024 * inst);
        }
    }
    for (int64_t kt = 0; kt < nk; kt++) {
        // this wave's loads of slice kt are done (the NBUF - 2 newer slices
        // may still be in flight); after the barrier every wave's are, and
        // every wave has finished reading the buffer refilled below
        wait_vmcnt<(NBUF - 2) * 2 * PER_WAVE>();
        barrier_only();
        const int cur = (int)(kt % NBUF), nxt = (int)((kt + NBUF - 1) % NBUF);
        const int64_t nxt_k0 = (kt + NBUF - 1 < nk ? kt + NBUF - 1 : nk - 1) * BK;
        big_slice<BK, MK>(acc, smem + cur * STAGE, smem + nxt * STAGE, srcA, srcB, nxt_k0, offA, offB, wave);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

}  // namespace ql
