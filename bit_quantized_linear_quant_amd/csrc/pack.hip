// One-time weight packing kernels for gfx950.
//
// Ternary ("Class BitLinear" forward step 3; "Common Attention Utilities"
// weight_quant and bake_ternary_weights): gamma' = max(mean|W|, eps) is an
// fp64 sum over fixed 16384-element chunks (one workgroup each, fixed
// per-thread order and a fixed shuffle tree), then one 1024-thread workgroup
// sums the chunk partials in a fixed order, so gamma' is identical on every
// call.
// The pack kernels compare |W| with gamma'/2 exactly in fp64.  For [n][k]
// weights one wave builds a 1 KB block of the 2-bit layout from 16 whole
// 1 KB row segments (coalesced loads); for [k][n] weights one thread builds
// one 16-byte lane slice (four words) from four-byte column gathers.
//
// 4-bit ("linear_4bit/mod.rs" module doc: eight nibbles per u32): weights
// into the fragment-ordered layout, zero-points group-major.
#include <atomic>

#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

// Scratch of the allocation-free ternary pack: the fp64 chunk partials of
// the absmean, one per 16384 weights, for at most kPackScratchPartials
// chunks (1 MiB of device memory per GPU, held until the process ends).  In
// host code `scratch` is a host-side stand-in, not a device address: host
// code uses only the per-device pointer from hipGetSymbolAddress below.
static __device__ __align__(256) double scratch[kPackScratchPartials];

// Per-device address of `scratch`, found once per device.
constexpr int kMaxDevices = 64;
std::atomic<double *> g_scratch_ptr[kMaxDevices];

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

// [k][n] weights: one thread = one lane slice (4 words, 64 consecutive k of
// one column) of a 16-column x 256-k block.
__global__ __launch_bounds__(kPThreads) void pack_ternary_kn_kernel(const float *__restrict__ w,
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
#pragma unroll
            for (int j = 0; j < 4; j++) v[j] = w[(k0 + j) * n + col];
            // element e = 4*q4 + j of the word: a = q4, b = j -> bits 8b + 2a
#pragma unroll
            for (int j = 0; j < 4; j++) words[t] |= tern_field(v[j], half) << (8 * j + 2 * q4);
        }
    }
    *reinterpret_cast<uint4 *>(packed + bi * 256 + 4 * l) =
        make_uint4(words[0], words[1], words[2], words[3]);
}

// [n][k] weights: one wave per 16-column x 256-k block (1 KB of output).
// Lane l loads the floats 4 l .. 4 l + 3 of each of the block's 16 weight
// rows (one coalesced 1 KB load per row), so it holds element e = 4 (l % 4)
// + j of word (l % 16) / 4 of k group l / 16 of every column; its four 2-bit
// fields go to bits 8 j + 2 (l % 4), the four lanes of a quad OR their
// parts into the whole word, and the words go through a wave-private LDS
// block to one 16-byte store per lane.  Same comparison as the [k][n] form.
constexpr int kTWaves = kPThreads / kWave;

__global__ __launch_bounds__(kPThreads) void pack_ternary_rows_kernel(const float *__restrict__ w, int64_t k,
                                                                      const double *__restrict__ gamma,
                                                                      uint32_t *__restrict__ packed,
                                                                      int64_t nblocks) {
    __shared__ uint32_t blk[kTWaves][256];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int64_t bi = (int64_t)blockIdx.x * kTWaves + wave;
    if (bi >= nblocks) return;
    const int64_t kblocks = k / 256;
    const int64_t nb = bi / kblocks, kb = bi % kblocks;
    const float *src = w + nb * 16 * k + kb * 256 + 4 * lane;
    uint4 v[16];
#pragma unroll
    for (int r = 0; r < 16; r++) v[r] = load16_stream(src + r * k);
    const double half = gamma[0] * 0.5;
    const int q4 = lane % 4;
    uint32_t word[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const float e[4] = {__uint_as_float(v[r].x), __uint_as_float(v[r].y), __uint_as_float(v[r].z),
                            __uint_as_float(v[r].w)};
        uint32_t part = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) part |= tern_field(e[j], half) << (8 * j + 2 * q4);
        part |= (uint32_t)__shfl_xor((int)part, 1);
        part |= (uint32_t)__shfl_xor((int)part, 2);
        word[r] = part;
    }
    // lane 4 m (m = 4 g + t) holds word t of packed lane r + 16 g for every row r
    uint32_t *b = blk[wave];
    if (q4 == 0) {
        const int g = lane / 16, t = (lane % 16) / 4;
#pragma unroll
        for (int r = 0; r < 16; r++) b[4 * (r + 16 * g) + t] = word[r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint4 o = *reinterpret_cast<const uint4 *>(b + 4 * lane);
    *reinterpret_cast<uint4 *>(packed + bi * 256 + 4 * lane) = o;
}

// One wave per 16-column x 128-k block (2 KB of codes, 1 KB of words).
// Lane L loads 16 codes of column 8 i + L / 8 (i = 0, 1) at k 16 (L % 8)
// of the block, so each load takes whole 128-byte row segments; those 16
// codes are exactly words 2 (q % 2) and 2 (q % 2) + 1 (q = L % 8) of lane
// slice column + 16 (q / 2), whose nibble p holds k-offset 2p (p < 4) or
// 2(p-4)+1 within its 8 codes.  The words go through a wave-private LDS
// block to one 16-byte store per lane.
__global__ __launch_bounds__(kPThreads) void pack_int4_weight_kernel(const uint8_t *__restrict__ codes,
                                                                     int64_t k,
                                                                     uint32_t *__restrict__ packed,
                                                                     int64_t nblocks) {
    __shared__ uint32_t blk[kPThreads / kWave][256];
    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int64_t bi = (int64_t)blockIdx.x * (kPThreads / kWave) + wave;
    if (bi >= nblocks) return;
    const int64_t kblocks = k / 128;
    const int64_t nb = bi / kblocks, kb = bi % kblocks;
    const int q = lane % 8;
    uint4 v[2];
#pragma unroll
    for (int i = 0; i < 2; i++)
        v[i] = *reinterpret_cast<const uint4 *>(codes + (nb * 16 + 8 * i + lane / 8) * k + kb * 128 + 16 * q);
    uint32_t *b = blk[wave];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const uint32_t in[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t words[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t wd = 0;
#pragma unroll
            for (int off = 0; off < 8; off++) {
                const uint32_t c = (in[2 * h + off / 4] >> (8 * (off % 4))) & 15u;
                const int p = (off % 2 == 0) ? off / 2 : off / 2 + 4;
                wd |= c << (4 * p);
            }
            words[h] = wd;
        }
        const int col = 8 * i + lane / 8;
        *reinterpret_cast<uint2 *>(b + 4 * (col + 16 * (q / 2)) + 2 * (q % 2)) = make_uint2(words[0], words[1]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    *reinterpret_cast<uint4 *>(packed + bi * 256 + 4 * lane) = *reinterpret_cast<const uint4 *>(b + 4 * lane);
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
    if (layout_nk) {
        const int64_t nblocks = nslices / 64;
        hipLaunchKernelGGL(pack_ternary_rows_kernel, dim3((unsigned)((nblocks + kTWaves - 1) / kTWaves)),
                           dim3(kPThreads), 0, st, w, k, gamma, packed, nblocks);
    } else
        hipLaunchKernelGGL(pack_ternary_kn_kernel, dim3(blocks_for(nslices)), dim3(kPThreads), 0, st, w, n,
                           k, gamma, packed, nslices);
    return hipGetLastError();
}

hipError_t pack_ternary_scratch(double **partials) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    double *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // Idempotent: threads racing here all store the same address.
        e = hipGetSymbolAddress(reinterpret_cast<void **>(&p), HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *partials = p;
    return hipSuccess;
}

hipError_t launch_pack_int4_weight(const uint8_t *codes, int64_t n, int64_t k, uint32_t *packed,
                                   hipStream_t st) {
    const int64_t nblocks = (n / 16) * (k / 128);
    constexpr int64_t per = kPThreads / kWave;
    hipLaunchKernelGGL(pack_int4_weight_kernel, dim3((unsigned)((nblocks + per - 1) / per)), dim3(kPThreads), 0,
                       st, codes, k, packed, nblocks);
    return hipGetLastError();
}

hipError_t launch_pack_int4_zeros(const uint8_t *z, int64_t n, int64_t groups, uint32_t *packed,
                                  hipStream_t st) {
    hipLaunchKernelGGL(pack_int4_zeros_kernel, dim3(blocks_for(groups * (n / 8))), dim3(kPThreads),
                       0, st, z, n, groups, packed);
    return hipGetLastError();
}

}  // namespace ql
