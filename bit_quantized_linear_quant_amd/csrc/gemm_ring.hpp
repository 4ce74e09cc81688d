// The main loop of the 256 x 256 tile matrix-core kernels, shared by the
// int8 product (gemm_i8.hip) and the 16-bit products of the Q4Linear
// backward (q4_backward.hip).
//
// Operands are row-major with k contiguous, K bytes per row (K % BK == 0);
// A has rows_a rows, B rows_b, and out = A B^T.  A 512-thread workgroup owns
// a 256 x 256 output tile, each of its eight waves a 128 x 64 part (wm, wn)
// held as 4 x 2 blocks of a 32 x 32 matrix-core product: 128 accumulators
// per lane, two waves per SIMD.  Every 32-byte k step gives lane l the 16 bytes
// 16(l/32) .. +15 of row l%32 of a block, for the int8 32x32x32 product and
// for the fp16 / bf16 32x32x16 products alike (16 bytes are 16 int8 or 8
// 16-bit values; A and B take the same k positions, so the products are the
// same whatever order the instruction sums them in).
//
// BK-byte k-slices of A and B move from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of NBUF
// slices, so NBUF - 1 slices stream in while the matrix cores consume one;
// explicit vmcnt waits and two barriers per slice.  In LDS each 16-byte
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

// The k loop of one 256 x 256 tile at (m0, n0) for a 512-thread workgroup:
// zeroes `acc` and runs the ring over K bytes (`smem` holds NBUF stages of
// 2 * BigTile<BK>::TILE bytes).  Eight waves, two per SIMD
// (waves w and w + 4 share SIMD w % 4), each a 128 x 64 sub-tile (wm in
// 0..1 selects 128 rows, wn in 0..3 64 columns) held as 4 x 2 blocks.  The
// groups of waves 0-3 and 4-7 run opposite phases of every slice: one reads
// its fragments of the slice from LDS and issues its direct loads NBUF - 1
// slices ahead while the other issues its products, so each SIMD's matrix
// core has a ready wave in both phases.  Two barriers per slice separate
// the phases; the second group passes one extra barrier before the loop
// and the first group one after it.  Before every barrier a wave waits
// until at most NBUF - 2 slices of its own loads are in flight, so a slice
// has landed (every wave's loads) at the barrier before its first read and
// no stage is refilled while a partner still reads it.  Leaves every load
// drained and every wave past a barrier, so `smem` may be reused by the
// epilogue.
template <int BK, int NBUF, int MK, typename ACC>
__device__ __forceinline__ void ring_gemm_pp(ACC (&acc)[4][2], int8_t *smem, const int8_t *A, const int8_t *B,
                                             int64_t rows_a, int64_t rows_b, int64_t K, int64_t m0, int64_t n0,
                                             int wm, int wn, int lane, int wave) {
    constexpr int CH = BigTile<BK>::CH, TILE = BigTile<BK>::TILE;
    constexpr int PW = TILE / 1024 / 8;     // direct loads per wave, slice and operand
    constexpr int S = BigTile<BK>::S;
    constexpr int STAGE = 2 * TILE;
    const int group = wave / 4;
    const int64_t nk = K / BK;
    const int8_t *srcA[PW];
    const int8_t *srcB[PW];
#pragma unroll
    for (int ii = 0; ii < PW; ii++) {
        const int pos = 64 * (wave * PW + ii) + lane;
        const int row = pos / CH;
        const int c = (pos % CH) ^ swz<CH>(row);
        const int64_t ra = min(m0 + row, rows_a - 1), rb = min(n0 + row, rows_b - 1);
        srcA[ii] = A + ra * K + 16 * c;
        srcB[ii] = B + rb * K + 16 * c;
    }
    const int fr = lane % 32;
    int offA[S], offB[S];
#pragma unroll
    for (int s = 0; s < S; s++) {
        const int c = 2 * s + lane / 32;
        const int ra = wm * 128 + fr, rb = wn * 64 + fr;
        offA[s] = 16 * (CH * ra + (c ^ swz<CH>(ra)));
        offB[s] = 16 * (CH * rb + (c ^ swz<CH>(rb)));
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = ACC{};
    auto issue = [&](int64_t slice, int buf) __attribute__((always_inline)) {
        const int64_t k0 = (slice < nk ? slice : nk - 1) * BK;
#pragma unroll
        for (int ii = 0; ii < PW; ii++) {
            const int inst = wave * PW + ii;
            lds_load16(srcA[ii] + k0, smem + buf * STAGE + 1024 * inst);
            lds_load16(srcB[ii] + k0, smem + buf * STAGE + TILE + 1024 * inst);
        }
    };
#pragma unroll
    for (int b = 0; b < NBUF - 1; b++) issue(b, b);
    if (group == 1) {
        wait_vmcnt<(NBUF - 2) * 2 * PW>();
        barrier_only();
    }
    for (int64_t kt = 0; kt < nk; kt++) {
        wait_vmcnt<(NBUF - 2) * 2 * PW>();
        barrier_only();
        const int8_t *cur = smem + (int)(kt % NBUF) * STAGE;
        v4i fa[S][4], fb[S][2];
#pragma unroll
        for (int s = 0; s < S; s++) {
#pragma unroll
            for (int i = 0; i < 4; i++) fa[s][i] = *reinterpret_cast<const v4i *>(cur + offA[s] + i * 32 * CH * 16);
#pragma unroll
            for (int j = 0; j < 2; j++) fb[s][j] = *reinterpret_cast<const v4i *>(cur + TILE + offB[s] + j * 32 * CH * 16);
        }
        issue(kt + NBUF - 1, (int)((kt + NBUF - 1) % NBUF));
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
        wait_vmcnt<(NBUF - 2) * 2 * PW>();
        barrier_only();
#pragma unroll
        for (int s = 0; s < S; s++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    if constexpr (MK == MK_I8) acc[i][j] = mfma32(fa[s][i], fb[s][j], acc[i][j]);
                    else acc[i][j] = mfma32<MK>(fa[s][i], fb[s][j], acc[i][j]);
                }
    }
    if (group == 0) barrier_only();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}


}  // namespace ql
