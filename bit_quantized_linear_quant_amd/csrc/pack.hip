// One-time weight packing kernels for gfx950.
//
// Ternary ("Class BitLinear" forward step 3; "Common Attention Utilities"
// weight_quant and bake_ternary_weights): gamma' = max(mean|W|, eps) is an
// fp64 sum over fixed 16384-element chunks (one workgroup each, fixed
// per-thread order and a fixed shuffle tree), then one 1024-thread workgroup
// sums the chunk partials in a fixed order, so gamma' is identical on every
// call.
// The pack kernel compares |W| with gamma'/2 exactly in fp64 and writes one
// 16-byte lane slice (four words) of the 2-bit layout per thread.
//
// 4-bit ("linear_4bit/mod.rs" module doc: eight nibbles per u32): weights
// into the fragment-ordered layout, zero-points group-major.
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

constexpr int kPThreads = 256;
constexpr int kChunkIters = 16;
constexpr int64_t kChunk = (int64_t)kPThreads * 4 * kChunkIters;  // 16384 elements

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) lds[w] = v;
    __syncthreads();
    double r = lds[0];
#pragma unroll
    for (int i = 1; i < kPThreads / kWave; i++) r += lds[i];
    return r;
}

__global__ __launch_bounds__(kPThreads) void absmean_partial_kernel(const float *__restrict__ w,
                                                                    int64_t count,
                                                                    double *__restrict__ partial) {
    __shared__ double red[kPThreads / kWave];
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    double acc = 0.0;
    if (base + kChunk <= count) {
        // whole chunk: every load first (non-temporal: read once), then the
        // adds in the same order as the ragged path below
        float4 v[kChunkIters];
#pragma unroll
        for (int it = 0; it < kChunkIters; it++) {
            const v4u t = __builtin_nontemporal_load(
                reinterpret_cast<const v4u *>(w + base + ((int64_t)it * kPThreads + threadIdx.x) * 4));
            v[it] = make_float4(__uint_as_float(t[0]), __uint_as_float(t[1]), __uint_as_float(t[2]),
                                __uint_as_float(t[3]));
        }
#pragma unroll
        for (int it = 0; it < kChunkIters; it++) {
            acc += fabs((double)v[it].x);
            acc += fabs((double)v[it].y);
            acc += fabs((double)v[it].z);
            acc += fabs((double)v[it].w);
        }
        const double s = block_sum_f64(acc, red);
        if (threadIdx.x == 0) partial[blockIdx.x] = s;
        return;
    }
#pragma unroll 4
    for (int it = 0; it < kChunkIters; it++) {
        const int64_t idx = base + ((int64_t)it * kPThreads + threadIdx.x) * 4;
        if (idx + 4 <= count) {
            const float4 v = *reinterpret_cast<const float4 *>(w + idx);
            acc += fabs((double)v.x);
            acc += fabs((double)v.y);
            acc += fabs((double)v.z);
            acc += fabs((double)v.w);
        } else {
            for (int j = 0; j < 4; j++)
                if (idx + j < count) acc += fabs((double)w[idx + j]);
        }
    }
    const double s = block_sum_f64(acc, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// Sum of the chunk partials by one 1024-thread workgroup: thread t adds
// partials t, t + 1024, ... in order (loaded 16 at a time, so the loads are in
// flight together), then the 16 wave sums are added in wave order.
constexpr int kFThreads = 1024;
constexpr int kFBatch = 16;

__global__ __launch_bounds__(kFThreads) void absmean_final_kernel(const double *__restrict__ partial,
                                                                  int64_t nparts, int64_t count,
                                                                  double eps,
                                                                  double *__restrict__ gamma) {
    __shared__ double red[kFThreads / kWave];
    double acc = 0.0;
    for (int64_t base = threadIdx.x; base < nparts; base += (int64_t)kFThreads * kFBatch) {
        double v[kFBatch];
#pragma unroll
        for (int j = 0; j < kFBatch; j++) {
            const int64_t i = base + (int64_t)j * kFThreads;
            v[j] = i < nparts ? partial[i] : 0.0;
        }
#pragma unroll
        for (int j = 0; j < kFBatch; j++) acc += v[j];
    }
    acc = wave_sum(acc);
    if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = red[0];
#pragma unroll
        for (int i = 1; i < kFThreads / kWave; i++) s += red[i];
        const double g = s / (double)count;
        gamma[0] = g < eps ? eps : g;
    }
}

// 2-bit field of one weight: code + 1 in {0, 1, 2}.
__device__ __forceinline__ uint32_t tern_field(float v, double half) {
    const double a = fabs((double)v);
    return a > half ? (v > 0.0f ? 2u : 0u) : 1u;
}

// One thread = one lane slice (4 words, 64 consecutive k of one column) of a
// 16-column x 256-k block.
template <bool NK>
__global__ __launch_bounds__(kPThreads) void pack_ternary_kernel(const float *__restrict__ w,
                                                                 int64_t n, int64_t k,
                                                                 const double *__restrict__ gamma,
                                                                 uint32_t *__restrict__ packed,
                                                                 int64_t nslices) {
    const int64_t g = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
    if (g >= nslices) return;
    const int64_t bi = g / 64;
    const int l = (int)(g % 64);
    const int64_t kblocks = k / 256;
    const int64_t nb = bi / kblocks, kb = bi % kblocks;
    const int64_t col = nb * 16 + (l % 16);
    const int64_t kbase = kb * 256 + 64 * (l / 16);
    const double half = gamma[0] * 0.5;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; t++) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            float v[4];
            const int64_t k0 = kbase + 16 * t + 4 * q4;
            if (NK) {
                const float4 f = *reinterpret_cast<const float4 *>(w + col * k + k0);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) v[j] = w[(k0 + j) * n + col];
            }
            // element e = 4*q4 + j of the word: a = q4, b = j -> bits 8b + 2a
#pragma unroll
            for (int j = 0; j < 4; j++) words[t] |= tern_field(v[j], half) << (8 * j + 2 * q4);
        }
    }
    *reinterpret_cast<uint4 *>(packed + bi * 256 + 4 * l) =
        make_uint4(words[0], words[1], words[2], words[3]);
}

// One thread = one lane slice (4 words, 32 consecutive k of one column) of a
// 16-column x 128-k block.  Nibble p holds k-offset 2p (p < 4) or 2(p-4)+1.
__global__ __launch_bounds__(kPThreads) void pack_int4_weight_kernel(const uint8_t *__restrict__ codes,
                                                                     int64_t k,
                                                                     uint32_t *__restrict__ packed,
                                                                     int64_t nslices) {
    const int64_t g = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
    if (g >= nslices) return;
    const int64_t bi = g / 64;
    const int l = (int)(g % 64);
    const int64_t kblocks = k / 128;
    const int64_t nb = bi / kblocks, kb = bi % kblocks;
    const int64_t col = nb * 16 + (l % 16);
    const int64_t kbase = kb * 128 + 32 * (l / 16);
    const uint4 *src = reinterpret_cast<const uint4 *>(codes + col * k + kbase);
    const uint4 a = src[0], b = src[1];
    const uint32_t in[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t words[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        uint32_t wd = 0;
#pragma unroll
        for (int off = 0; off < 8; off++) {
            const uint32_t c = (in[2 * t + off / 4] >> (8 * (off % 4))) & 15u;
            const int p = (off % 2 == 0) ? off / 2 : off / 2 + 4;
            wd |= c << (4 * p);
        }
        words[t] = wd;
    }
    *reinterpret_cast<uint4 *>(packed + bi * 256 + 4 * l) =
        make_uint4(words[0], words[1], words[2], words[3]);
}

__global__ __launch_bounds__(kPThreads) void pack_int4_zeros_kernel(const uint8_t *__restrict__ z,
                                                                    int64_t n, int64_t groups,
                                                                    uint32_t *__restrict__ packed) {
    const int64_t g = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
    const int64_t words_per_group = n / 8;
    if (g >= groups * words_per_group) return;
    const int64_t gi = g / words_per_group, w8 = g % words_per_group;
    uint32_t wd = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) wd |= ((uint32_t)z[(8 * w8 + j) * groups + gi] & 15u) << (4 * j);
    packed[g] = wd;
}

unsigned blocks_for(int64_t threads) {
    return (unsigned)((threads + kPThreads - 1) / kPThreads);
}

}  // namespace

size_t absmean_partial_count(int64_t count) {
    return (size_t)((count + kChunk - 1) / kChunk);
}

hipError_t launch_pack_ternary(const float *w, bool layout_nk, int64_t n, int64_t k, double eps,
                               uint32_t *packed, double *gamma, double *partials, hipStream_t st) {
    const int64_t count = n * k;
    const int64_t nparts = (int64_t)absmean_partial_count(count);
    hipLaunchKernelGGL(absmean_partial_kernel, dim3((unsigned)nparts), dim3(kPThreads), 0, st, w,
                       count, partials);
    hipLaunchKernelGGL(absmean_final_kernel, dim3(1), dim3(kFThreads), 0, st, partials, nparts,
                       count, eps, gamma);
    const int64_t nslices = (n / 16) * (k / 256) * 64;
    if (layout_nk)
        hipLaunchKernelGGL((pack_ternary_kernel<true>), dim3(blocks_for(nslices)), dim3(kPThreads),
                           0, st, w, n, k, gamma, packed, nslices);
    else
        hipLaunchKernelGGL((pack_ternary_kernel<false>), dim3(blocks_for(nslices)), dim3(kPThreads),
                           0, st, w, n, k, gamma, packed, nslices);
    return hipGetLastError();
}

hipError_t launch_pack_int4_weight(const uint8_t *codes, int64_t n, int64_t k, uint32_t *packed,
                                   hipStream_t st) {
    const int64_t nslices = (n / 16) * (k / 128) * 64;
    hipLaunchKernelGGL(pack_int4_weight_kernel, dim3(blocks_for(nslices)), dim3(kPThreads), 0, st,
                       codes, k, packed, nslices);
    return hipGetLastError();
}

hipError_t launch_pack_int4_zeros(const uint8_t *z, int64_t n, int64_t groups, uint32_t *packed,
                                  hipStream_t st) {
    hipLaunchKernelGGL(pack_int4_zeros_kernel, dim3(blocks_for(groups * (n / 8))), dim3(kPThreads),
                       0, st, z, n, groups, packed);
    return hipGetLastError();
}

}  // namespace ql
