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
// One 128-k block is four MFMA steps; its fp32 partial sum is closed before
// the group scale multiplies it once (group_size is a multiple of 128).
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
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int t) {
    return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}

// 8 exact fp16 (q - z) values from one packed word; zz is the pair (1024+z).
__device__ __forceinline__ v8h unpack_int4(uint32_t w, h2 zz) {
    v8h r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t pair = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        const h2 d = __builtin_bit_cast(h2, pair) - zz;
        r[2 * i] = d[0];
        r[2 * i + 1] = d[1];
    }
    return r;
}

// One k block's operands for the NBLK column blocks of a wave: packed
// weight fragments, raw fp16 scales, zero-point words and the x fragments of
// RB 16-row blocks.
template <int NBLK, int RB>
struct Stage {
    uint4 w[NBLK];
    uint32_t s[NBLK], z[NBLK];
    v8h a[RB][4];
};

// Issue every load of k block kb (clamped into range; the caller masks a
// block past the end).  All loads are unconditional, so none of them waits
// for another.
template <int NBLK, int RB>
__device__ __forceinline__ void load_stage(Stage<NBLK, RB> &st, const uint16_t *__restrict__ x, int64_t row0, int64_t m,
                                           int64_t k,
                                           const uint32_t *__restrict__ packed_w,
                                           const uint16_t *__restrict__ scales,
                                           const uint32_t *__restrict__ packed_z, int64_t kb,
                                           int64_t nb0, int64_t nblocks, int64_t kblocks,
                                           int64_t group_size, int64_t groups, int64_t n, int lane) {
    const int fr = lane % 16;
    const int64_t kbc = kb < kblocks ? kb : kblocks - 1;
    const int64_t g = kbc * 128 / group_size;
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
        const int64_t col = nbc * 16 + fr;
        st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
        st.s[j] = scales[col * groups + g];
        st.z[j] = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
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

// Accumulate one k block: per column block, four MFMA steps per row block
// into a fresh fp32 partial, then one multiply by the group scale.
template <int NBLK, int RB>
__device__ __forceinline__ void compute_stage(const Stage<NBLK, RB> &st, v4f (&acc)[RB][NBLK], bool kb_ok,
                                              int64_t nb0, int64_t nblocks, uint8_t *xb, int lane) {
    v8h a[RB][4];
    rows256_to_fragments<RB>(st.a, a, xb, lane);
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const bool ok = kb_ok && nb0 + j < nblocks;
        const float sc = ok ? f16_bits_to_f32(st.s[j]) : 0.0f;
        const h2 zz = __builtin_bit_cast(h2, (0x6400u | (st.z[j] & 15u)) * 0x00010001u);
        v4f p[RB];
#pragma unroll
        for (int b = 0; b < RB; b++) p[b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const v8h wv = unpack_int4(word_of(st.w[j], t), zz);
#pragma unroll
            for (int b = 0; b < RB; b++) p[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[b][t], wv, p[b], 0, 0, 0);
        }
#pragma unroll
        for (int b = 0; b < RB; b++)
#pragma unroll
            for (int r = 0; r < 4; r++) acc[b][j][r] = __builtin_fmaf(sc, p[b][r], acc[b][j][r]);
    }
}

template <int NBLK, int WAVES, int RB, int OUT, int NST>
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
            Stage<NBLK, RB> st[NST];
#pragma unroll
            for (int u = 0; u < NST; u++)
                load_stage(st[u], x, row0, m, k, packed_w, scales, packed_z, kb0 + (int64_t)u * WAVES, nb0, nblocks, kblocks,
                           group_size, groups, n, lane);
#pragma unroll
            for (int u = 0; u < NST; u++)
                compute_stage(st[u], acc, kb0 + (int64_t)u * WAVES < kblocks, nb0, nblocks, xb, lane);
        }
    } else {
        Stage<NBLK, RB> s0, s1;
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

// Waves with at most this many k blocks issue all their loads at once.
constexpr int kAllIn = 4;

template <int NBLK, int WAVES, int RB, int OUT>
hipError_t launch_cfg(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                      const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k,
                      void *out, hipStream_t st, int64_t batch) {
    const int64_t nblocks = n / 16;
    dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), (unsigned)((m + 16 * RB - 1) / (16 * RB)), (unsigned)batch);
    // With two row blocks, four stages of x fragments do not fit beside the
    // weights in registers: those launches keep the two-stage pipeline.
    if constexpr (RB == 1) {
        if (k / 128 <= (int64_t)WAVES * kAllIn) {
            hipLaunchKernelGGL((int4_grouped_kernel<NBLK, WAVES, RB, OUT, kAllIn>), grid, dim3(WAVES * 64), 0, st, x,
                               packed_w, scales, packed_z, bias, group_size, m, n, k, out);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((int4_grouped_kernel<NBLK, WAVES, RB, OUT, 0>), grid, dim3(WAVES * 64), 0, st, x, packed_w,
                       scales, packed_z, bias, group_size, m, n, k, out);
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_t(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                    const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k,
                    void *out, hipStream_t st, int64_t batch) {
    // m <= 16 needs one 16-row MFMA block; larger m takes 32-row slices so
    // every unpacked weight fragment serves two row blocks.
    if (m <= 16) return launch_cfg<3, 8, 1, OUT>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
    return launch_cfg<3, 8, 2, OUT>(x, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
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

template <int NBLK, int RB>
struct StageI8 {
    uint4 w[NBLK];
    uint32_t s[NBLK], z[NBLK];
    v4i a[RB][2];
};

template <int NBLK, int RB>
__device__ __forceinline__ void load_stage_i8(StageI8<NBLK, RB> &st, const int8_t *__restrict__ xq, int64_t row0,
                                              int64_t m, int64_t k,
                                              const uint32_t *__restrict__ packed_w,
                                              const uint16_t *__restrict__ scales,
                                              const uint32_t *__restrict__ packed_z, int64_t kb, int64_t nb0,
                                              int64_t nblocks, int64_t kblocks, int64_t group_size,
                                              int64_t groups, int64_t n, int lane) {
    const int fr = lane % 16;
    const int64_t kbc = kb < kblocks ? kb : kblocks - 1;
    const int64_t g = kbc * 128 / group_size;
#pragma unroll
    for (int j = 0; j < NBLK; j++) {
        const int64_t nbc = nb0 + j < nblocks ? nb0 + j : nblocks - 1;
        const int64_t col = nbc * 16 + fr;
        st.w[j] = load16_stream(packed_w + (nbc * kblocks + kbc) * 256 + 4 * lane);
        st.s[j] = scales[col * groups + g];
        st.z[j] = packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8));
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

template <int NBLK, int RB>
__device__ __forceinline__ void compute_stage_i8(const StageI8<NBLK, RB> &st, v4f (&acc)[RB][NBLK], int64_t nb0,
                                                 int64_t nblocks, uint8_t *xb, int lane) {
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
        const float sc = nb0 + j < nblocks ? f16_bits_to_f32(st.s[j]) : 0.0f;
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

template <int NBLK, int WAVES, int RB, int OUT, int NST>
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
            StageI8<NBLK, RB> st[NST];
#pragma unroll
            for (int u = 0; u < NST; u++)
                load_stage_i8(st[u], xq, row0, m, k, packed_w, scales, packed_z, kb0 + (int64_t)u * WAVES, nb0, nblocks,
                              kblocks, group_size, groups, n, lane);
#pragma unroll
            for (int u = 0; u < NST; u++)
                if (kb0 + (int64_t)u * WAVES < kblocks) compute_stage_i8(st[u], acc, nb0, nblocks, xb, lane);
        }
    } else {
        StageI8<NBLK, RB> s0, s1;
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

template <int NBLK, int WAVES, int RB, int OUT>
hipError_t launch_cfg_i8(const int8_t *xq, const float *pts, const uint32_t *packed_w, const uint16_t *scales,
                         const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k, void *out,
                         hipStream_t st, int64_t batch) {
    const int64_t nblocks = n / 16;
    dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), (unsigned)((m + 16 * RB - 1) / (16 * RB)), (unsigned)batch);
    if (k / 128 <= (int64_t)WAVES * kAllIn)
        hipLaunchKernelGGL((int4_grouped_i8_kernel<NBLK, WAVES, RB, OUT, kAllIn>), grid, dim3(WAVES * 64), 0, st, xq,
                           pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
    else
        hipLaunchKernelGGL((int4_grouped_i8_kernel<NBLK, WAVES, RB, OUT, 0>), grid, dim3(WAVES * 64), 0, st, xq,
                           pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out);
    return hipGetLastError();
}

template <int OUT>
hipError_t launch_i8_t(const int8_t *xq, const float *pts, const uint32_t *packed_w, const uint16_t *scales,
                       const uint32_t *packed_z, const float *bias, int64_t group_size, int64_t m, int64_t n, int64_t k, void *out,
                       hipStream_t st, int64_t batch) {
    if (m <= 16)
        return launch_cfg_i8<3, 8, 1, OUT>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
    return launch_cfg_i8<3, 8, 2, OUT>(xq, pts, packed_w, scales, packed_z, bias, group_size, m, n, k, out, st, batch);
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
