// Grouped affine INT4 linear with fp16 activations, gfx950
// ("linear_4bit/mod.rs" module doc: the packed u32 weight is unpacked inside
// the k loop and combined with its group's scale and zero-point; nothing is
// dequantized into memory).
//
// The 4-bit layout is fragment-ordered for v_mfma_f32_16x16x32_f16: word t
// of lane l holds the 8 k of the B operand of lane l in step t, with nibble
// pairs arranged so (word >> 4i) & 0x000F000F is the fp16 pair
// (k0+2i, k0+2i+1).  OR-ing 0x6400 (fp16 1024.0) into each half makes it
// exactly 1024+q, and subtracting the pair (1024+z, 1024+z) gives (q - z)
// exactly in fp16.  The x fragment of lane l in step t is the 8 halves of
// its row at k = 128kb + 32(l/16) + 8t, the same k as the weight fragment.
// One 128-k block is four MFMA steps; when group_size is a multiple of 128
// its fp32 partial sum is closed before the group scale multiplies it once.
//
// Smaller groups (group_size a multiple of 32): in the packed layout one step
// takes its 32 k from four different 32-k sub-blocks (8 k from each 16-lane
// row of the wave), so a per-step scale cannot be applied.  These launches
// transpose each lane's four words across the four 16-lane rows
// (quad_transpose), after which step t covers exactly the 32-k sub-block t
// of the block (k 32t + 8q in row q, and the x fragments are read in the same
// order), and every step's fp32 partial is scaled by its own group's scale
// and offset by its own zero-point.
//
// x fragments reach the lanes through the wave's own LDS block
// (rows256_to_fragments): x is loaded in whole cache lines, lane (r, q) taking
// the 8 halves at k offset 8r of row 4t + q in load t.
//
// Workgroup: WAVES waves split the k blocks of NBLK column blocks for one
// slice of RB 16-row blocks of x (with RB = 2 every unpacked weight fragment
// feeds two MFMA row blocks; m <= 16 uses RB = 1).  Each wave keeps two
// register stages: while the matrix cores consume one k block, the weight
// fragments (non-temporal: read once), scales, zero-points and x fragments
// of its next k block are in flight; with one row block, a wave with at most
// four k blocks (k <= 4096 with 8 waves) issues all of their loads at once
// instead.
// The fp32 partials of the waves are added in LDS in a fixed wave order.
#include <type_traits>

#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int t) {
    return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

// 8 exact fp16 (q - z) values from one packed word; zz is the pair (1024+z).
// lo / hi hold the even / odd nibbles in their bytes; one byte permute
// against 0x64 bytes forms the pair (1024 + q_{2i}, 1024 + q_{2i+1}), i.e.
// nibbles (i, i + 4) = bytes (i/2, i/2 + 2) of lo (even i) or hi (odd i).
__device__ __forceinline__ v8h unpack_int4(uint32_t w, h2 zz) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu, c64 = 0x64646464u;
    const uint32_t pr[4] = {__builtin_amdgcn_perm(c64, lo, 0x04020400u), __builtin_amdgcn_perm(c64, hi, 0x04020400u),
                            __builtin_amdgcn_perm(c64, lo, 0x04030401u), __builtin_amdgcn_perm(c64, hi, 0x04030401u)};
    v8h r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const h2 d = __builtin_bit_cast(h2, pr[i]) - zz;
        r[2 * i] = d[0];
        r[2 * i + 1] = d[1];
    }
    return r;
}

// One k block's operands for the NBLK column blocks of a wave: packed
// weight fragments, raw fp16 scales, zero-point words and the x fragments of
// RB 16-row blocks.
template <int NBLK, int RB, bool SUB>
struct Stage {
    uint4 w[NBLK];
    // SUB: the scale's fp16 bits | zero-point << 16 of this lane's 32-k
    // step lane / 16 (sub_scale_zero hands each lane the other steps').
    uint32_t s[NBLK][1], z[NBLK];
    v8h a[RB][4];
};

// Groups of the four 32-k sub-blocks 4 kb + t (t = 0..3) for group_size =
// 32 * g32: one division, then a running remainder.
__device__ __forceinline__ void subblock_groups(int64_t kb, int64_t g32, int64_t (&gt)[4]) {
    const int64_t u0 = kb * 4;
    int64_t g = u0 / g32, r = u0 - g * g32;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        gt[t] = g;
        if (++r == g32) {
            r = 0;
            g++;
        }
    }
}

// Scale bits | zero-point << 16 of column col in group g.
__device__ __forceinline__ uint32_t scale_zero(const uint16_t *__restrict__ scales,
                                               const uint32_t *__restrict__ packed_z, int64_t col, int64_t g,
                                               int64_t groups, int64_t n) {
    const uint32_t zw = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
    return (uint32_t)scales[col * groups + g] | ((zw & 15u) << 16);
}

// Per-step scales of k block kbc, one load pair per lane: lane (fr, q)
// loads the word of its column's 32-k step q (group gt[q]); at use, the
// word of step t comes from lane fr + 16 t of the same column.
__device__ __forceinline__ uint32_t lane_scale_zero(const uint16_t *__restrict__ scales,
                                                    const uint32_t *__restrict__ packed_z, int64_t col,
                                                    const int64_t (&gt)[4], int64_t groups, int64_t n, int lane) {
    const int q = lane / 16;
    const int64_t g = q == 0 ? gt[0] : q == 1 ? gt[1] : q == 2 ? gt[2] : gt[3];
    return scale_zero(scales, packed_z, col, g, groups, n);
}

__device__ __forceinline__ uint32_t sub_scale_zero(uint32_t own, int t, int lane) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (lane % 16 + 16 * t), (int)own);
}

// Issue every load of k block kb (clamped into range; the caller masks a
// block past the end).  All loads are unconditional, so none of them waits
// for another.
template <int NBLK, int RB, bool SUB>
__device__ __forceinline__ void load_stage(Stage<NBLK, RB, SUB> &st, const uint16_t *__restrict__ x, int64_t row0,
                                           int64_t m, int64_t k,
                                           const uint32_t *__restrict__ packed_w,
                                           const uint16_t *__restrict__ scales,
                                           const uint32_t *__restrict__ packed_z, int64_t kb,
                                           int64_t nb0, int64_t nblocks, int64_t kblocks,
                                           int64_t group_size, int64_t groups, int64_t n, int lane) {
    const int fr = lane % 16;
    const int64_t kbc = kb < kblocks ? kb : kblocks - 1;
    if constexpr (SUB) {
        int64_t gt[4];
        subblock_groups(kbc, group_size / 32, gt);
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            const int64_t col = nbc * 16 + fr;
            st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
            st.s[j][0] = lane_scale_zero(scales, packed_z, col, gt, groups, n, lane);
        }
    } else {
        const int64_t g = kbc * 128 / group_size;
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            const int64_t col = nbc * 16 + fr;
            st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
            st.s[j][0] = scales[col * groups + g];
            st.z[j] = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
        }
    }
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++) {
            // Load t of row block b covers rows 16b + 4t + lane/16.  Rows
            // past m read row 0: an MFMA row only feeds its own output row,
            // which is never stored.
            const int64_t r = row0 + 16 * b + 4 * t + lane / 16;
            st.a[b][t] = *reinterpret_cast<const v8h *>(x + (r < m ? r : 0) * k + kbc * 128 + 8 * fr);
        }
}

// Accumulate one k block from its x fragments: per column block, four MFMA
// steps per row block into a fresh fp32 partial, then one multiply by the
// group scale (SUB: per step, after the cross-row transpose of the words).
template <int NBLK, int RB, bool SUB>
__device__ __forceinline__ void block_mma(const v8h (&a)[RB][4], const uint4 (&w)[NBLK],
                                          const uint32_t (&s)[NBLK][1], const uint32_t (&z)[NBLK],
                                          v4f (&acc)[RB][NBLK], bool kb_ok, int64_t nb0, int64_t nblocks, int lane) {
    if constexpr (SUB) {
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const bool ok = kb_ok && nb0 + j < nblocks;
            const uint4 wt = quad_transpose(w[j]);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t sz = sub_scale_zero(s[j][0], t, lane);
                const float sc = ok ? f16_bits_to_f32(sz & 0xffffu) : 0.0f;
                const h2 zz = __builtin_bit_cast(h2, (0x6400u | ((sz >> 16) & 15u)) * 0x00010001u);
                const v8h wv = unpack_int4(word_of(wt, t), zz);
#pragma unroll
                for (int b = 0; b < RB; b++) {
                    const v4f p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b][t], wv, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[b][j][r] = __builtin_fmaf(sc, p[r], acc[b][j][r]);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const bool ok = kb_ok && nb0 + j < nblocks;
        const float sc = ok ? f16_bits_to_f32(s[j][0]) : 0.0f;
        const h2 zz = __builtin_bit_cast(h2, (0x6400u | (z[j] & 15u)) * 0x00010001u);
        v4f p[RB];
#pragma unroll
        for (int b = 0; b < RB; b++) p[b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const v8h wv = unpack_int4(word_of(w[j], t), zz);
#pragma unroll
            for (int b = 0; b < RB; b++) p[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b][t], wv, p[b], 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[b][j][r] = __builtin_fmaf(sc, p[b][r], acc[b][j][r]);
    }
}

// One register stage: x pieces to fragments through the wave's LDS block,
// then block_mma.
template <int NBLK, int RB, bool SUB>
__device__ __forceinline__ void compute_stage(const Stage<NBLK, RB, SUB> &st, v4f (&acc)[RB][NBLK], bool kb_ok,
                                              int64_t nb0, int64_t nblocks, uint8_t *xb, int lane) {
    v8h a[RB][4];
    if constexpr (SUB) rows256_to_subblock_fragments<RB>(st.a, a, xb, lane);
    else rows256_to_fragments<RB>(st.a, a, xb, lane);
    block_mma<NBLK, RB, SUB>(a, st.w, st.s, st.z, acc, kb_ok, nb0, nblocks, lane);
}

template <int NBLK, int WAVES, int RB, int OUT, int NST, bool SUB>
__global__ __launch_bounds__(WAVES * 64) void int4_grouped_kernel(const uint16_t *__restrict__ x,
                                                                  const uint32_t *__restrict__ packed_w,
                                                                  const uint16_t *__restrict__ scales,
                                                                  const uint32_t *__restrict__ packed_z,
                                                                  const float *__restrict__ bias,
                                                                  int64_t group_size, int64_t m,
                                                                  int64_t n, int64_t k,
                                                                  void *__restrict__ out) {
    __shared__ v4f red[WAVES][RB * NBLK][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xlds[WAVES][16 * RB * kRow256Pitch];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t row0 = (int64_t)blockIdx.y * 16 * RB;
    const int64_t nblocks = n / 16, kblocks = k / 128, groups = k / group_size;
    const int fr = lane % 16;
    uint8_t *xb = xlds[wave];
    // Batched launches: blockIdx.z selects one independent product.
    const int64_t z = blockIdx.z;
    x += z * m * k;
    packed_w += z * (n * k / 8);
    scales += z * n * groups;
    packed_z += z * groups * (n / 8);
    if (bias) bias += z * n;
    const int64_t obase = z * m * n;

    v4f acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // The wave owns k blocks wave, wave + WAVES, ...  NST > 0: the loads of
    // NST of them are issued together, then consumed in k order (one memory
    // round trip when the wave has at most NST blocks).  NST = 0: two
    // register stages, the loads of the next k block in flight while the
    // matrix cores work on the current one.  Both add the blocks in the same
    // order, so both give the same bits.
    if constexpr (NST > 0) {
        for (int64_t kb0 = wave; kb0 < kblocks; kb0 += (int64_t)WAVES * NST) {
            Stage<NBLK, RB, SUB> st[NST];
#pragma unroll
            for (int u = 0; u < NST; u++)
                load_stage(st[u], x, row0, m, k, packed_w, scales, packed_z, kb0 + (int64_t)u * WAVES, nb0, nblocks, kblocks,
                           group_size, groups, n, lane);
#pragma unroll
            for (int u = 0; u < NST; u++)
                compute_stage(st[u], acc, kb0 + (int64_t)u * WAVES < kblocks, nb0, nblocks, xb, lane);
        }
    } else {
        Stage<NBLK, RB, SUB> s0, s1;
        int64_t kb = wave;
        load_stage(s0, x, row0, m, k, packed_w, scales, packed_z, kb, nb0, nblocks, kblocks, group_size, groups, n, lane);
        while (kb < kblocks) {
            const int64_t kb1 = kb + WAVES;
            if (kb1 < kblocks)
                load_stage(s1, x, row0, m, k, packed_w, scales, packed_z, kb1, nb0, nblocks, kblocks, group_size, groups, n,
                           lane);
            compute_stage(s0, acc, true, nb0, nblocks, xb, lane);
            if (kb1 >= kblocks) break;
            const int64_t kb2 = kb1 + WAVES;
            if (kb2 < kblocks)
                load_stage(s0, x, row0, m, k, packed_w, scales, packed_z, kb2, nb0, nblocks, kblocks, group_size, groups, n,
                           lane);
            compute_stage(s1, acc, true, nb0, nblocks, xb, lane);
            kb = kb2;
        }
    }

#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[wave][b * NBLK + j][lane] = acc[b][j];
    __syncthreads();
    for (int e = wave; e < RB * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t nb = nb0 + j;
        if (nb >= nblocks) continue;
        v4f s = red[0][e][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) s += red[w][e][lane];
        const int64_t col = nb * 16 + fr;
        const float cb = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = row0 + b * 16 + 4 * (lane / 16) + r;
            if (row < m) store_out<OUT>(out, obase + row * n + col, bias ? __fadd_rn(s[r], cb) : s[r]);
        }
    }
}


// global_load_lds_dwordx4 issued from inline asm: lane l writes lds_base + 16 l.
// The compiler does not see it, so its own waits for register loads are not
// widened to vmcnt(0); the caller waits for it explicitly (s_waitcnt vmcnt).
__device__ __forceinline__ void lds_load16_hidden(const void *src, const void *lds_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m) : "memory", "m0");
}

// Direct-load form for waves with at most NKB k blocks (k <= 128 * WAVES *
// NKB).  The two-stage pipeline above issues a k block's weight loads only
// after the block two earlier has arrived, so the HBM latency is paid once
// per two blocks.  Here every weight, scale and zero-point load of the wave
// is issued at the start (NKB * NBLK 16-byte weight fragments in registers),
// and x moves L2 -> LDS with global_load_lds_dwordx4 into two buffers that
// belong to the wave alone (no registers, no workgroup barrier): direct load
// i of a k block writes rows 4i .. 4i + 3 of its RB * 16-row slice, lane l
// taking 16-byte piece (l % 16) ^ (row % 16) of row 4i + l / 16 to LDS
// position l % 16, so that the fragment reads of 16 rows (piece 4q + t, or
// 4t + q for per-step groups, of row r at position piece ^ r) fall in
// distinct banks.  The wave walks the same k blocks in the same order as the
// pipelined kernel (kb = wave + u * WAVES), so the sums are the same bits.
//
// When the compiler sees a direct load pending it waits for every
// outstanding load (vmcnt(0)) before the first use of any loaded register,
// which would hold block 0 back until the wave's last weight arrived.  So
// the direct loads and the fragment reads are issued from inline asm, in a
// fixed order (weights of block 0, x(0), x(1), weights of the other blocks,
// then x(u) after block u - 2, kept by scheduling barriers), the waits for
// x are explicit vmcnt counts of the loads issued after it, and the
// compiler's own waits for the register loads stay precise (they may only
// over-wait, since the hidden loads are not in its count).
template <int NBLK, int WAVES, int RB, int OUT, int NKB, bool SUB>
__global__ __launch_bounds__(WAVES * 64) void int4_grouped_dl_kernel(const uint16_t *__restrict__ x,
                                                                     const uint32_t *__restrict__ packed_w,
                                                                     const uint16_t *__restrict__ scales,
                                                                     const uint32_t *__restrict__ packed_z,
                                                                     const float *__restrict__ bias,
                                                                     int64_t group_size, int64_t m, int64_t n,
                                                                     int64_t k, void *__restrict__ out) {
    constexpr int XBUF = RB * 16 * 256;            // one k block of x for the row slice
    constexpr int XL = XBUF / 1024;                // direct loads per k block
    constexpr int NXB = NKB < 2 ? NKB : 2;         // x buffers per wave
    constexpr int WL = NBLK * 3;                   // weight, scale and zero-point loads per k block
    constexpr int XS = WAVES * XBUF;
    constexpr int RED = WAVES * RB * NBLK * kWave * 16;
    static_assert(RED <= XS, "the partials reuse the first x buffer");
    // Two distinct LDS objects, so the compiler's wait before a fragment read
    // covers only the direct loads into that buffer.
    __shared__ __attribute__((aligned(1024))) uint8_t xbuf0[XS];
    __shared__ __attribute__((aligned(1024))) uint8_t xbuf1[NXB > 1 ? XS : 16];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t row0 = (int64_t)blockIdx.y * 16 * RB;
    const int64_t nblocks = n / 16, kblocks = k / 128, groups = k / group_size;
    const int fr = lane % 16, q = lane / 16;
    const int64_t z = blockIdx.z;
    x += z * m * k;
    packed_w += z * (n * k / 8);
    scales += z * n * groups;
    packed_z += z * groups * (n / 8);
    if (bias) bias += z * n;
    const int64_t obase = z * m * n;

    // Global source of each direct load of a k block (k block 0); rows past
    // m read row 0 (their outputs are never stored).
    const uint16_t *xsrc[XL];
#pragma unroll
    for (int i = 0; i < XL; i++) {
        const int r = 4 * i + lane / 16;
        const int64_t row = row0 + r;
        xsrc[i] = x + (row < m ? row : 0) * k + 8 * ((lane % 16) ^ (r % 16));
    }
    auto kb_of = [&](int u) { return (int64_t)wave + (int64_t)u * WAVES; };
    auto load_x = [&](int u) {
        const int64_t kb = kb_of(u), kbc = kb < kblocks ? kb : kblocks - 1;
        uint8_t *buf = (u % 2 == 0 ? xbuf0 : xbuf1) + wave * XBUF;
#pragma unroll
        for (int i = 0; i < XL; i++) lds_load16_hidden(xsrc[i] + kbc * 128, buf + 1024 * i);
    };

    uint4 w[NKB][NBLK];
    uint32_t sc[NKB][NBLK][1], zr[NKB][NBLK];
    auto load_w = [&](int u) {
        const int64_t kb = kb_of(u), kbc = kb < kblocks ? kb : kblocks - 1;
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            const int64_t col = nbc * 16 + fr;
            w[u][j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
            if constexpr (SUB) {
                int64_t gt[4];
                subblock_groups(kbc, group_size / 32, gt);
                sc[u][j][0] = lane_scale_zero(scales, packed_z, col, gt, groups, n, lane);
                zr[u][j] = 0;
            } else {
                const int64_t g = kbc * 128 / group_size;
                sc[u][j][0] = scales[col * groups + g];
                zr[u][j] = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
            }
        }
    };
    // Issue order: weights of block 0, x(0), x(1), weights of blocks 1 ..
    // NKB - 1, then x(u) for u >= 2 after block u - 2 (scheduling barriers
    // keep it).
    load_w(0);
    __builtin_amdgcn_sched_barrier(0);
    load_x(0);
    if constexpr (NKB > 1) load_x(1);
    __builtin_amdgcn_sched_barrier(0);
    static_for<1, NKB>([&](auto uc) {
        load_w(decltype(uc)::value);
        __builtin_amdgcn_sched_barrier(0);
    });

    v4f acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4f{0.f, 0.f, 0.f, 0.f};

    static_for<0, NKB>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        // Issue order: x(0), x(1), every weight load, then x(u) for u >= 2
        // after block u - 2.  Wait until x(u) has landed (the weights are
        // registers: the compiler waits for those itself).
        // loads after x(0): x(1) and the weights of blocks 1 ..; after x(1):
        // those weights and x(2)
        constexpr int after0 = (NKB > 1 ? XL : 0) + (NKB - 1) * WL;
        constexpr int after1 = (NKB - 1) * WL + (NKB > 2 ? XL : 0);
        if constexpr (u == 0) wait_vmcnt<after0 < 63 ? after0 : 63>();
        else if constexpr (u == 1) wait_vmcnt<after1 < 63 ? after1 : 63>();
        else if constexpr (u + 1 < NKB) wait_vmcnt<XL>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint8_t *buf = (u % 2 == 0 ? xbuf0 : xbuf1) + wave * XBUF;
        v8h a[RB][4];
#pragma unroll
        for (int b = 0; b < RB; b++) {
            uint32_t ad[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int piece = SUB ? 4 * t + q : 4 * q + t;
                ad[t] = (uint32_t)(uintptr_t)(buf + (16 * b + fr) * 256 + 16 * (piece ^ fr));
            }
            // The compiler cannot tell which direct loads wrote this buffer
            // and would wait for every outstanding load; the explicit vmcnt
            // wait above covers them, and the reads wait for themselves.
            asm volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %5\n\t"
                "ds_read_b128 %2, %6\n\t"
                "ds_read_b128 %3, %7\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=v"(a[b][0]), "=v"(a[b][1]), "=v"(a[b][2]), "=v"(a[b][3])
                : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                : "memory");
        }
        block_mma<NBLK, RB, SUB>(a, w[u], sc[u], zr[u], acc, kb_of(u) < kblocks, nb0, nblocks, lane);
        if constexpr (u + 2 < NKB) {
            // every fragment of this buffer was read into registers above
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            load_x(u + 2);
        }
    });

    __syncthreads();   // every wave is done with its x buffers: the same LDS holds the partials
    v4f *red = reinterpret_cast<v4f *>(xbuf0);
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[(wave * RB * NBLK + b * NBLK + j) * kWave + lane] = acc[b][j];
    __syncthreads();
    for (int e = wave; e < RB * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t nb = nb0 + j;
        if (nb >= nblocks) continue;
        v4f sum = red[e * kWave + lane];
#pragma unroll
        for (int wv = 1; wv < WAVES; wv++) sum += red[(wv * RB * NBLK + e) * kWave + lane];
        const int64_t col = nb * 16 + fr;
        const float cb = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = row0 + b * 16 + 4 * (lane / 16) + r;
            if (row < m) store_out<OUT>(out, obase + row * n + col, bias ? __fadd_rn(sum[r], cb) : sum[r]);
        }
    }
}

// Waves with at most this many k blocks issue all their loads at once.
constexpr int kAllIn = 4;

template <int NBLK, int WAVES, int RB, int OUT, bool SUB>
hipError_t launch_cfg(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                      const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k,
                      void *out, hipStream_t st, int64_t batch) {
    const int64_t nblocks = n / 16;
    dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), (unsigned)((m + 16 * RB - 1) / (16 * RB)), (unsigned)batch);
    // Two row blocks with at most four k blocks per wave: the direct-load
    // form (all weight loads at the start, x straight into LDS).
    if constexpr (RB == 2) {
        const int64_t per_wave = (k / 128 + WAVES - 1) / WAVES;
        if (per_wave <= 2) {
            hipLaunchKernelGGL((int4_grouped_dl_kernel<NBLK, WAVES, RB, OUT, 2, SUB>), grid, dim3(WAVES * 64), 0, st,
                               x, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
            return hipGetLastError();
        }
        if (per_wave <= 4) {
            hipLaunchKernelGGL((int4_grouped_dl_kernel<NBLK, WAVES, RB, OUT, 4, SUB>), grid, dim3(WAVES * 64), 0, st,
                               x, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
            return hipGetLastError();
        }
    }
    // With two row blocks, four stages of x fragments do not fit beside the
    // weights in registers; with per-step groups the all-in form fits but
    // measured slower (m = 16, g = 32: 13.9 against 12.9 us).  Those
    // launches keep the two-stage pipeline.
    if constexpr (RB == 1 && !SUB) {
        if (k / 128 <= (int64_t)WAVES * kAllIn) {
            hipLaunchKernelGGL((int4_grouped_kernel<NBLK, WAVES, RB, OUT, kAllIn, SUB>), grid, dim3(WAVES * 64), 0,
                               st, x, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((int4_grouped_kernel<NBLK, WAVES, RB, OUT, 0, SUB>), grid, dim3(WAVES * 64), 0, st, x,
                       packed_w, scales, packed_z, bias, group_size, m, n, k, out);
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_t(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                    const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k,
                    void *out, hipStream_t st, int64_t batch) {
    // m <= 16 needs one 16-row MFMA block; larger m takes 32-row slices so
    // every unpacked weight fragment serves two row blocks.  Groups smaller
    // than a 128-k block (or not aligned to one) take the per-step variant.
    if (group_size % 128 != 0) {
        if (m <= 16)
            return launch_cfg<3, 8, 1, OUT, true>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st,
                                                  batch);
        return launch_cfg<3, 8, 2, OUT, true>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st,
                                              batch);
    }
    if (m <= 16)
        return launch_cfg<3, 8, 1, OUT, false>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
    return launch_cfg<3, 8, 2, OUT, false>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
}

// ---------------------------------------------------------------------------
// int8 activation codes
// ---------------------------------------------------------------------------
// The same packed weights feed v_mfma_i32_16x16x64_i8.  Step s (0, 1) of a
// 128-k block gives lane l the 16 k from 32(l/16) + 16s: the activation codes
// are 16 contiguous bytes of its row, the weight operand is words 2s and
// 2s + 1 of its fragment with the nibbles (codes 0..15) restored to k order
// by two byte permutes per word.  The zero-point is applied afterwards:
// sum x (q - z) = sum x q - z sum x, with sum x from one more MFMA against an
// all-ones operand.  The block's exact int32 result is scaled by the group
// scale in fp32; the per-token scale multiplies the final sum.

// Natural-order int8 codes of the 8 k of one packed word.
__device__ __forceinline__ void nibbles_to_bytes(uint32_t w, int &lo_k, int &hi_k) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    lo_k = (int)__builtin_amdgcn_perm(hi, lo, 0x06040200u);   // k0 .. k0+3
    hi_k = (int)__builtin_amdgcn_perm(hi, lo, 0x07050301u);   // k0+4 .. k0+7
}

__device__ __forceinline__ v4i weight_step(const uint4 &w, int s) {
    int b0, b1, b2, b3;
    nibbles_to_bytes(s == 0 ? w.x : w.z, b0, b1);
    nibbles_to_bytes(s == 0 ? w.y : w.w, b2, b3);
    return v4i{b0, b1, b2, b3};
}

template <int NBLK, int RB, bool SUB>
struct StageI8 {
    uint4 w[NBLK];
    // SUB: the scale's fp16 bits | zero-point << 16 of this lane's 32-k
    // step lane / 16 (sub_scale_zero hands each lane the other steps').
    uint32_t s[NBLK][1], z[NBLK];
    v4i a[RB][2];
};

template <int NBLK, int RB, bool SUB>
__device__ __forceinline__ void load_stage_i8(StageI8<NBLK, RB, SUB> &st, const int8_t *__restrict__ xq,
                                              int64_t row0, int64_t m, int64_t k,
                                              const uint32_t *__restrict__ packed_w,
                                              const uint16_t *__restrict__ scales,
                                              const uint32_t *__restrict__ packed_z, int64_t kb, int64_t nb0,
                                              int64_t nblocks, int64_t kblocks, int64_t group_size,
                                              int64_t groups, int64_t n, int lane) {
    const int fr = lane % 16;
    const int64_t kbc = kb < kblocks ? kb : kblocks - 1;
    if constexpr (SUB) {
        int64_t gt[4];
        subblock_groups(kbc, group_size / 32, gt);
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            const int64_t col = nbc * 16 + fr;
            st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
            st.s[j][0] = lane_scale_zero(scales, packed_z, col, gt, groups, n, lane);
        }
    } else {
        const int64_t g = kbc * 128 / group_size;
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
            const int64_t col = nbc * 16 + fr;
            st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
            st.s[j][0] = scales[col * groups + g];
            st.z[j] = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
        }
    }
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int s = 0; s < 2; s++) {
            // Load s of row block b covers rows 16b + 8s + lane/8; rows past
            // m read row 0 (their outputs are never stored).
            const int64_t r = row0 + 16 * b + 8 * s + lane / 8;
            st.a[b][s] = *reinterpret_cast<const v4i *>(xq + (r < m ? r : 0) * k + kbc * 128 + 16 * (lane % 8));
        }
}

// As x_fragments for int8 codes: 128-byte rows, load s of row block b
// covers rows 16b + 8s + lane/8.
constexpr int kXPitchI8 = 144;

template <int RB>
__device__ __forceinline__ void x_fragments_i8(const v4i (&in)[RB][2], v4i (&frag)[RB][2], uint8_t *xb, int lane) {
    const int fr = lane % 16, q = lane / 16;
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<v4i *>(xb + (16 * b + 8 * s + lane / 8) * kXPitchI8 + 16 * (lane % 8)) = in[b][s];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int s = 0; s < 2; s++)
            frag[b][s] = *reinterpret_cast<const v4i *>(xb + (16 * b + fr) * kXPitchI8 + 32 * q + 16 * s);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sub-block fragments of the int8 codes: fragment t of lane (r, q) is the
// 8 bytes at k 32t + 8q of row r (the same k as word t of the transposed
// weight fragment).  Writes as x_fragments_i8; 8-byte reads.
template <int RB>
__device__ __forceinline__ void x_subblock_fragments_i8(const v4i (&in)[RB][2], long (&frag)[RB][4], uint8_t *xb,
                                                        int lane) {
    const int fr = lane % 16, q = lane / 16;
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<v4i *>(xb + (16 * b + 8 * s + lane / 8) * kXPitchI8 + 16 * (lane % 8)) = in[b][s];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++)
            frag[b][t] = *reinterpret_cast<const long *>(xb + (16 * b + fr) * kXPitchI8 + 32 * t + 8 * q);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NBLK, int RB, bool SUB>
__device__ __forceinline__ void compute_stage_i8(const StageI8<NBLK, RB, SUB> &st, v4f (&acc)[RB][NBLK], int64_t nb0,
                                                 int64_t nblocks, uint8_t *xb, int lane) {
    if constexpr (SUB) {
        // Step t (v_mfma_i32_16x16x32_i8) covers the 32-k sub-block t, whose
        // exact int32 partial gets its own zero-point and scale.
        const long ones = 0x0101010101010101l;
        long a[RB][4];
        x_subblock_fragments_i8<RB>(st.a, a, xb, lane);
        v4i sx[RB][4];
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int t = 0; t < 4; t++)
                sx[b][t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[b][t], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const bool ok = nb0 + j < nblocks;
            const uint4 wt = quad_transpose(st.w[j]);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t sz = sub_scale_zero(st.s[j][0], t, lane);
                const float sc = ok ? f16_bits_to_f32(sz & 0xffffu) : 0.0f;
                const int z = (int)((sz >> 16) & 15u);
                int lo, hi;
                nibbles_to_bytes(word_of(wt, t), lo, hi);
                const long wv = (long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
#pragma unroll
                for (int b = 0; b < RB; b++) {
                    const v4i p = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[b][t], wv, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[b][j][r] = __builtin_fmaf(sc, (float)(p[r] - z * sx[b][t][r]), acc[b][j][r]);
                }
            }
        }
        return;
    }
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    v4i a[RB][2];
    x_fragments_i8<RB>(st.a, a, xb, lane);
    v4i sx[RB];
#pragma unroll
    for (int b = 0; b < RB; b++) {
        sx[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[b][0], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
        sx[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[b][1], ones, sx[b], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const float sc = nb0 + j < nblocks ? f16_bits_to_f32(st.s[j][0]) : 0.0f;
        const int z = (int)(st.z[j] & 15u);
        const v4i w0 = weight_step(st.w[j], 0), w1 = weight_step(st.w[j], 1);
#pragma unroll
        for (int b = 0; b < RB; b++) {
            v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[b][0], w0, v4i{0, 0, 0, 0}, 0, 0, 0);
            p = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[b][1], w1, p, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[b][j][r] = __builtin_fmaf(sc, (float)(p[r] - z * sx[b][r]), acc[b][j][r]);
        }
    }
}

template <int NBLK, int WAVES, int RB, int OUT, int NST, bool SUB>
__global__ __launch_bounds__(WAVES * 64) void int4_grouped_i8_kernel(const int8_t *__restrict__ xq,
                                                                     const float *__restrict__ pts,
                                                                     const uint32_t *__restrict__ packed_w,
                                                                     const uint16_t *__restrict__ scales,
                                                                     const uint32_t *__restrict__ packed_z,
                                                                     const float *__restrict__ bias,
                                                                     int64_t group_size, int64_t m, int64_t n,
                                                                     int64_t k, void *__restrict__ out) {
    __shared__ v4f red[WAVES][RB * NBLK][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xlds[WAVES][16 * RB * kXPitchI8];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t row0 = (int64_t)blockIdx.y * 16 * RB;
    const int64_t nblocks = n / 16, kblocks = k / 128, groups = k / group_size;
    const int fr = lane % 16;
    uint8_t *xb = xlds[wave];
    // Batched launches: blockIdx.z selects one independent product.
    const int64_t z = blockIdx.z;
    xq += z * m * k;
    pts += z * m;
    packed_w += z * (n * k / 8);
    scales += z * n * groups;
    packed_z += z * groups * (n / 8);
    if (bias) bias += z * n;
    const int64_t obase = z * m * n;
    float prow[RB][4];
#pragma unroll
    for (int b = 0; b < RB; b++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int64_t orow = row0 + 16 * b + 4 * (lane / 16) + q;
            prow[b][q] = pts[orow < m ? orow : m - 1];
        }
    }

    v4f acc[RB][NBLK];
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // As in the fp16 kernel: NST > 0 issues the loads of NST k blocks
    // together; NST = 0 pipelines two register stages.  Same order, same bits.
    if constexpr (NST > 0) {
        for (int64_t kb0 = wave; kb0 < kblocks; kb0 += (int64_t)WAVES * NST) {
            StageI8<NBLK, RB, SUB> st[NST];
#pragma unroll
            for (int u = 0; u < NST; u++)
                load_stage_i8(st[u], xq, row0, m, k, packed_w, scales, packed_z, kb0 + (int64_t)u * WAVES, nb0, nblocks,
                              kblocks, group_size, groups, n, lane);
#pragma unroll
            for (int u = 0; u < NST; u++)
                if (kb0 + (int64_t)u * WAVES < kblocks) compute_stage_i8(st[u], acc, nb0, nblocks, xb, lane);
        }
    } else {
        StageI8<NBLK, RB, SUB> s0, s1;
        int64_t kb = wave;
        load_stage_i8(s0, xq, row0, m, k, packed_w, scales, packed_z, kb, nb0, nblocks, kblocks, group_size, groups, n, lane);
        while (kb < kblocks) {
            const int64_t kb1 = kb + WAVES;
            if (kb1 < kblocks)
                load_stage_i8(s1, xq, row0, m, k, packed_w, scales, packed_z, kb1, nb0, nblocks, kblocks, group_size, groups,
                              n, lane);
            compute_stage_i8(s0, acc, nb0, nblocks, xb, lane);
            if (kb1 >= kblocks) break;
            const int64_t kb2 = kb1 + WAVES;
            if (kb2 < kblocks)
                load_stage_i8(s0, xq, row0, m, k, packed_w, scales, packed_z, kb2, nb0, nblocks, kblocks, group_size, groups,
                              n, lane);
            compute_stage_i8(s1, acc, nb0, nblocks, xb, lane);
            kb = kb2;
        }
    }

#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[wave][b * NBLK + j][lane] = acc[b][j];
    __syncthreads();
    for (int e = wave; e < RB * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t nb = nb0 + j;
        if (nb >= nblocks) continue;
        v4f s = red[0][e][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) s += red[w][e][lane];
        const int64_t col = nb * 16 + fr;
        const float cb = bias ? bias[col] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = row0 + b * 16 + 4 * (lane / 16) + r;
            const float y = __fmul_rn(s[r], prow[b][r]);
            if (row < m) store_out<OUT>(out, obase + row * n + col, bias ? __fadd_rn(y, cb) : y);
        }
    }
}

template <int NBLK, int WAVES, int RB, int OUT, bool SUB>
hipError_t launch_cfg_i8(const int8_t *xq, const float *pts, const uint32_t *packed_w, const uint16_t *scales,
                         const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k, void *out,
                         hipStream_t st, int64_t batch) {
    const int64_t nblocks = n / 16;
    dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), (unsigned)((m + 16 * RB - 1) / (16 * RB)), (unsigned)batch);
    // Per-step groups with two row blocks keep the two-stage pipeline: the
    // all-in form fits (248 registers) but measured no faster.
    if (k / 128 <= (int64_t)WAVES * kAllIn && !(SUB && RB == 2))
        hipLaunchKernelGGL((int4_grouped_i8_kernel<NBLK, WAVES, RB, OUT, (SUB && RB == 2) ? 0 : kAllIn, SUB>), grid,
                           dim3(WAVES * 64), 0, st, xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k,
                           out);
    else
        hipLaunchKernelGGL((int4_grouped_i8_kernel<NBLK, WAVES, RB, OUT, 0, SUB>), grid, dim3(WAVES * 64), 0, st, xq,
                           pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_i8_t(const int8_t *xq, const float *pts, const uint32_t *packed_w, const uint16_t *scales,
                       const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k, void *out,
                       hipStream_t st, int64_t batch) {
    if (group_size % 128 != 0) {
        if (m <= 16)
            return launch_cfg_i8<3, 8, 1, OUT, true>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out,
                                                     st, batch);
        return launch_cfg_i8<3, 8, 2, OUT, true>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st,
                                                 batch);
    }
    if (m <= 16)
        return launch_cfg_i8<3, 8, 1, OUT, false>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st,
                                                  batch);
    return launch_cfg_i8<3, 8, 2, OUT, false>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st,
                                              batch);
}

}  // namespace

hipError_t launch_gemm_int4_grouped(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                                    const uint32_t *packed_zeros, const float *bias, int64_t group_size,
                                    int64_t m, int64_t n, int64_t k, int out_kind, void *out, hipStream_t st, int64_t batch) {
    if ((m + 31) / 32 > 65535 || batch < 1 || batch > 65535) return hipErrorInvalidValue;
    if (out_kind == OUT_F32)
        return launch_t<OUT_F32>(x, packed_w, scales, packed_zeros, bias, group_size, m, n, k, out, st, batch);
    return launch_t<OUT_F16>(x, packed_w, scales, packed_zeros, bias, group_size, m, n, k, out, st, batch);
}

}  // namespace ql

namespace ql {

hipError_t launch_gemm_int4_grouped_i8(const int8_t *xq, const float *pts, const uint32_t *packed_w,
                                       const uint16_t *scales, const uint32_t *packed_zeros, const float *bias,
                                       int64_t group_size, int64_t m, int64_t n, int64_t k, int out_kind, void *out,
                                       hipStream_t st, int64_t batch) {
    if ((m + 31) / 32 > 65535 || batch < 1 || batch > 65535) return hipErrorInvalidValue;
    switch (out_kind) {
        case OUT_F32: return launch_i8_t<OUT_F32>(xq, pts, packed_w, scales, packed_zeros, bias, group_size, m, n, k, out, st, batch);
        case OUT_BF16: return launch_i8_t<OUT_BF16>(xq, pts, packed_w, scales, packed_zeros, bias, group_size, m, n, k, out, st, batch);
        default: return launch_i8_t<OUT_F16>(xq, pts, packed_w, scales, packed_zeros, bias, group_size, m, n, k, out, st, batch);
    }
}

}  // namespace ql
