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
// Workgroup: WAVES waves split the k blocks of NBLK column blocks for one
// 32-row slice of x (two 16-row MFMA blocks share every unpacked weight
// fragment); fp32 partials are added in LDS in a fixed wave order.
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

template <int NBLK, int WAVES, int OUT>
__global__ __launch_bounds__(WAVES * 64) void int4_grouped_kernel(const uint16_t *__restrict__ x,
                                                                  const uint32_t *__restrict__ packed_w,
                                                                  const uint16_t *__restrict__ scales,
                                                                  const uint32_t *__restrict__ packed_z,
                                                                  int64_t group_size, int64_t m,
                                                                  int64_t n, int64_t k,
                                                                  void *__restrict__ out) {
    __shared__ v4f red[WAVES][2 * NBLK][kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int64_t nb0 = (int64_t)blockIdx.x * NBLK;
    const int64_t row0 = (int64_t)blockIdx.y * 32;
    const int64_t nblocks = n / 16, kblocks = k / 128, groups = k / group_size;
    const int fr = lane % 16;
    const int64_t r0 = row0 + fr, r1 = row0 + 16 + fr;
    const bool ok0 = r0 < m, ok1 = r1 < m;
    const int koff = 32 * (lane / 16);

    v4f acc[2][NBLK];
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) acc[b][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = wave; kb < kblocks; kb += WAVES) {
        const int64_t g = kb * 128 / group_size;
        uint4 bw[NBLK];
        float sc[NBLK];
        uint32_t zq[NBLK];
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const int64_t nb = nb0 + j;
            const bool ok = nb < nblocks;
            const int64_t col = nb * 16 + fr;
            bw[j] = ok ? load16_stream(packed_w + (nb * kblocks + kb) * 256 + 4 * lane) : make_uint4(0, 0, 0, 0);
            sc[j] = ok ? f16_bits_to_f32(scales[col * groups + g]) : 0.0f;
            zq[j] = ok ? (packed_z[g * (n / 8) + col / 8] >> (4 * (col % 8))) & 15u : 0u;
        }
        v8h a0[4], a1[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int64_t kk = kb * 128 + koff + 8 * t;
            a0[t] = ok0 ? *reinterpret_cast<const v8h *>(x + r0 * k + kk) : v8h{};
            a1[t] = ok1 ? *reinterpret_cast<const v8h *>(x + r1 * k + kk) : v8h{};
        }
#pragma unroll
        for (int j = 0; j < NBLK; j++) {
            const uint32_t zpair = (0x6400u | zq[j]) * 0x00010001u;
            const h2 zz = __builtin_bit_cast(h2, zpair);
            v4f p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const v8h b = unpack_int4(word_of(bw[j], t), zz);
                p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[t], b, p0, 0, 0, 0);
                p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[t], b, p1, 0, 0, 0);
            }
            acc[0][j] += sc[j] * p0;
            acc[1][j] += sc[j] * p1;
        }
    }

#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
        for (int j = 0; j < NBLK; j++) red[wave][b * NBLK + j][lane] = acc[b][j];
    __syncthreads();
    for (int e = wave; e < 2 * NBLK; e += WAVES) {
        const int b = e / NBLK, j = e % NBLK;
        const int64_t nb = nb0 + j;
        if (nb >= nblocks) continue;
        v4f s = red[0][e][lane];
#pragma unroll
        for (int w = 1; w < WAVES; w++) s += red[w][e][lane];
        const int64_t col = nb * 16 + fr;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int64_t row = row0 + b * 16 + 4 * (lane / 16) + r;
            if (row < m) store_out<OUT>(out, row * n + col, s[r]);
        }
    }
}

template <int OUT>
hipError_t launch_t(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                    const uint32_t *packed_z, int64_t group_size, int64_t m, int64_t n, int64_t k,
                    void *out, hipStream_t st) {
    constexpr int NBLK = 4, WAVES = 8;
    const int64_t nblocks = n / 16;
    dim3 grid((unsigned)((nblocks + NBLK - 1) / NBLK), (unsigned)((m + 31) / 32));
    hipLaunchKernelGGL((int4_grouped_kernel<NBLK, WAVES, OUT>), grid, dim3(WAVES * 64), 0, st, x, packed_w,
                       scales, packed_z, group_size, m, n, k, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_int4_grouped(const uint16_t *x, const uint32_t *packed_w, const uint16_t *scales,
                                    const uint32_t *packed_zeros, int64_t group_size, int64_t m,
                                    int64_t n, int64_t k, int out_kind, void *out, hipStream_t st) {
    if ((m + 31) / 32 > 65535) return hipErrorInvalidValue;
    if (out_kind == OUT_F32)
        return launch_t<OUT_F32>(x, packed_w, scales, packed_zeros, group_size, m, n, k, out, st);
    return launch_t<OUT_F16>(x, packed_w, scales, packed_zeros, group_size, m, n, k, out, st);
}

}  // namespace ql
