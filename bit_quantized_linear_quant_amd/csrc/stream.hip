// HBM read stream for gfx950: the rate at which the device reads a buffer
// once.  It is the ceiling of every kernel whose cost is streaming its
// operand bytes from HBM (the decode product reads each packed weight byte
// exactly once), measured with the same load form those kernels use:
// 16-byte non-temporal loads, eight in flight per thread, 512 threads per
// workgroup, spread over a grid that covers every CU several times.  The bytes are folded into one XOR per
// wave, which the wave XORs into its own word of the sink array (no atomics:
// one address taken by every wave would serialize them), so no load can be
// dropped.
#include "qlinear.h"
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

constexpr int kStThreads = 512;   // with 8 loads in flight per thread: 10.2 us per 58.7 MB launch,
                                   // against 10.2-11.4 for 256 / 1024 threads and 2, 4 or 16 loads
constexpr int kStUnroll = 8;
constexpr int64_t kStMaxGroups = QL_HBM_STREAM_SINK_WORDS / (kStThreads / kWave);

__global__ __launch_bounds__(kStThreads) void hbm_read_stream_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                                     uint64_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kStThreads;
    int64_t i = (int64_t)blockIdx.x * kStThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kStUnroll - 1) * stride < n16; i += kStUnroll * stride) {
        uint4 v[kStUnroll];
#pragma unroll
        for (int u = 0; u < kStUnroll; u++) v[u] = load16_stream(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = load16_stream(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if (threadIdx.x % kWave == 0) sink[(int64_t)blockIdx.x * (kStThreads / kWave) + wave_id()] ^= acc;
}

}  // namespace

hipError_t launch_hbm_read_stream(const void *buf, int64_t bytes, uint64_t *sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    int64_t groups = (n16 + (int64_t)kStThreads * kStUnroll - 1) / ((int64_t)kStThreads * kStUnroll);
    groups = groups < 1 ? 1 : (groups > kStMaxGroups ? kStMaxGroups : groups);
    hipLaunchKernelGGL(hbm_read_stream_kernel, dim3((unsigned)groups), dim3(kStThreads), 0, st,
                       static_cast<const uint4 *>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace ql
