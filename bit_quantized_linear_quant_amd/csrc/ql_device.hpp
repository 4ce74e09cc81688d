// Device helpers shared by the gfx950 kernels of libqlinear: vector types,
// element conversions, wave64 reductions and the rounding stores of the
// dequant epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ql {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l of the wave writes lds_base + 16 l.
// lds_base must be the same for every lane of the wave.
__device__ __forceinline__ void lds_load16(const void *src, void *lds_base) {
    typedef __attribute__((address_space(1))) void gvoid;
    typedef __attribute__((address_space(3))) void lvoid;
    __builtin_amdgcn_global_load_lds((gvoid *)src, (lvoid *)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N), leaving expcnt and lgkmcnt at their maximum: waits until
// at most N of this wave's vector-memory operations (LDS-DMA loads included)
// are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (N & 15) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the full memory wait __syncthreads() implies
// (which drains every outstanding LDS-DMA load); callers wait explicitly.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value, so that arithmetic on it runs on the scalar unit.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// 16-byte streaming load (non-temporal: the data is read once and should not
// displace reused lines from the caches).  p must be 16-byte aligned.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
}

// Operand rows of 256 bytes (one k block), 16 bytes per lane per load.  A
// matrix-core fragment gives lane (r, q) = (lane % 16, lane / 16) the 16-byte
// pieces 4q + t (t = 0..3) of row r, so loading fragments directly makes one
// load instruction touch 32 cache lines and use a quarter of each.  Instead
// load t of row block b gives lane (r, q) piece r of row 16b + 4t + q (whole
// lines), and this turns those pieces into fragments through the wave's own
// LDS block xb (16 RB rows at kRow256Pitch bytes, 16 more than a row so that
// the fragment reads of 16 rows fall in distinct banks).  Only the wave
// touches its block and LDS operations of one wave complete in issue order,
// so wave-scope fences (which keep the compiler from moving the reads above
// the writes, or the next call's writes above these reads) are all the
// ordering needed.
constexpr int kRow256Pitch = 272;

template <int RB, typename T>
__device__ __forceinline__ void rows256_to_fragments(const T (&in)[RB][4], T (&frag)[RB][4], uint8_t *xb, int lane) {
    static_assert(sizeof(T) == 16, "16-byte pieces");
    const int fr = lane % 16, q = lane / 16;
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++)
            *reinterpret_cast<T *>(xb + (16 * b + 4 * t + q) * kRow256Pitch + 16 * fr) = in[b][t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++)
            frag[b][t] = *reinterpret_cast<const T *>(xb + (16 * b + fr) * kRow256Pitch + 64 * q + 16 * t);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// As rows256_to_fragments, with the fragments of 32-k sub-blocks: fragment t
// of lane (r, q) is the 16-byte piece t * 4 + q of row r (k 32t + 8q of the
// 128-k block for 16-bit elements), so that one matrix-core step covers one
// contiguous 32-k range.  Same LDS block, same ordering.
template <int RB, typename T>
__device__ __forceinline__ void rows256_to_subblock_fragments(const T (&in)[RB][4], T (&frag)[RB][4], uint8_t *xb,
                                                              int lane) {
    static_assert(sizeof(T) == 16, "16-byte pieces");
    const int fr = lane % 16, q = lane / 16;
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++)
            *reinterpret_cast<T *>(xb + (16 * b + 4 * t + q) * kRow256Pitch + 16 * fr) = in[b][t];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int b = 0; b < RB; b++)
#pragma unroll
        for (int t = 0; t < 4; t++)
            frag[b][t] = *reinterpret_cast<const T *>(xb + (16 * b + fr) * kRow256Pitch + 64 * t + 16 * q);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Transpose of four 32-bit words across the four 16-lane rows of a wave: on
// return, word t of the lane in row q holds what word q of the lane in the
// same column of row t held.  Two v_permlane32_swap (rows 0-1 with rows 2-3)
// and two v_permlane16_swap (even rows with odd rows).
__device__ __forceinline__ uint4 quad_transpose(uint4 v) {
    const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return make_uint4(c[0], c[1], d[0], d[1]);
}

// Workgroup id -> (tile row, tile column) for a grid of tiles_m x tiles_n
// output tiles.  The hardware hands consecutive workgroup ids to the 8 XCDs in
// turn; ids are first regrouped so each XCD receives a contiguous range of
// tiles, then each range is walked group_m tile rows at a time, column by
// column, so tiles running together on one XCD share A and B slices in its L2.
__device__ __forceinline__ void xcd_tile(int b, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
    const int total = tiles_m * tiles_n;
    int t = b;
    if (total % 8 == 0) t = (b % 8) * (total / 8) + b / 8;
    const int group = t / (group_m * tiles_n);
    const int first = group * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int within = t - group * group_m * tiles_n;
    tm = first + within % rows;
    tn = within / rows;
}

// Output element kinds of the epilogue.
enum OutKind : int { OUT_F16 = 0, OUT_BF16 = 1, OUT_I32 = 2, OUT_F32 = 3 };

// Input element kinds of the quantizers.
enum InKind : int { IN_F32 = 0, IN_F16 = 1, IN_BF16 = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
    return (float)h;
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN and
// values past the largest finite bf16 become +-inf.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// fp32 -> fp16, round to nearest, ties to even (v_cvt_f16_f32 under the
// default rounding mode); overflow gives +-inf.  The empty asm makes `f` an
// fp32 value in a register first, so the compiler cannot fold the product
// that produced it into a mixed-precision multiply that rounds once to fp16:
// the output is exactly the fp32 result rounded once more.
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
    asm volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Load element i of a row of kind K as fp32 (exact for all three kinds).
template <int K>
__device__ __forceinline__ float load_elem(const void *p, int64_t i) {
    if constexpr (K == IN_F32) return static_cast<const float *>(p)[i];
    else if constexpr (K == IN_F16) return f16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
}

// Load 8 consecutive elements starting at element i (16-byte aligned for
// 16-bit kinds, 32-byte aligned for fp32) as fp32.
template <int K>
__device__ __forceinline__ void load8_vec(const void *p, int64_t i, float v[8]) {
    if constexpr (K == IN_F32) {
        const float4 *q = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + i);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if constexpr (K == IN_F16) {
                v[2 * j] = f16_bits_to_f32(w[j] & 0xffffu);
                v[2 * j + 1] = f16_bits_to_f32(w[j] >> 16);
            } else {
                v[2 * j] = __uint_as_float(w[j] << 16);
                v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        T u = __shfl_xor(v, o, kWave);
        v = u > v ? u : v;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Store one epilogue value.  For OUT_I32 the caller passes the integer.
template <int OUT>
__device__ __forceinline__ void store_out(void *out, int64_t idx, float y) {
    if constexpr (OUT == OUT_F16) static_cast<uint16_t *>(out)[idx] = f32_to_f16_rne(y);
    else if constexpr (OUT == OUT_BF16) static_cast<uint16_t *>(out)[idx] = f32_to_bf16_rne(y);
    else static_cast<float *>(out)[idx] = y;
}

// fl32(v / sp) from the reciprocal r = fl32(1 / sp) in three operations
// instead of a full IEEE division: y = fl32(v * r) is within an ulp of v / sp,
// e = v - y * sp is exact in one FMA, and fl32(y + e * r) is the correctly
// rounded quotient (Markstein's correction; r must itself be correctly
// rounded).  Where |y| > 16 the 4-bit code saturates whatever the last bits
// are, so y is returned as it is: this keeps an overflowing y from turning
// into inf - inf.
__device__ __forceinline__ float q4_quotient(float v, float sp, float r) {
    const float y = __fmul_rn(v, r);
    const float e = __builtin_fmaf(-y, sp, v);
    const float q = __builtin_fmaf(e, r, y);
    return fabsf(y) <= 16.0f ? q : y;
}

// The 4-bit code clamp(rne(q), -8, 7) of a quotient, as a float.  + 0 turns
// the -0 of a small negative quotient into +0, the code 0.
__device__ __forceinline__ float q4_code(float q) {
    return fminf(fmaxf(__builtin_rintf(q), -8.0f), 7.0f) + 0.0f;
}

__device__ __forceinline__ float code_i4_f(float v, float sp, float r) { return q4_code(q4_quotient(v, sp, r)); }

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

}  // namespace ql
