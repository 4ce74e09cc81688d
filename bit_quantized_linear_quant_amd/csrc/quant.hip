// Activation quantizers for gfx950.
//
// quant_act: per-token absmax int8 codes with an optional parameter-free
// RMSNorm folded into the per-token scale ("Class BitLinear" forward steps
// 1-2 and 5; "Common Attention Utilities" activation_quant).  Rows of up to
// 8192 elements in whole 8-element chunks: rows of more than 3584 elements
// take two or four waves per row while a launch has at most 16384 waves,
// others one, the row held in registers, all
// of a lane's loads in flight at once, wave64 shuffle reductions (the wave
// results of a split row combined through LDS).  Other rows: one 256-thread
// workgroup per row, the row read from HBM once and kept in registers (up
// to 8192 elements), wave reductions combined through LDS.  Codes are
// written with 8-byte stores.
//
// quant_int4_tensor: per-tensor 4-bit codes of "Q4LinearFunction" forward,
// q = clamp(rne(x / max(scale, eps)), -8, 7) with IEEE division.
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

constexpr int kQThreads = 256;
constexpr int kQCache = 4;  // chunks of 8 elements per thread held in registers

template <int K, bool VEC>
__device__ __forceinline__ void load_chunk(const void *row, int64_t ch, int64_t k, float v[8]) {
    const int64_t base = ch * 8;
    if (VEC && base + 8 <= k) {
        load8_vec<K>(row, base, v);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = (base + j < k) ? load_elem<K>(row, base + j) : 0.0f;
    }
}

__device__ __forceinline__ int code_i8(float v, float s) {
    float t = __builtin_rintf(__fmul_rn(v, s));
    t = fminf(fmaxf(t, -128.0f), 127.0f);
    return (int)t;
}

template <bool VEC>
__device__ __forceinline__ int store_chunk(int8_t *qrow, int64_t ch, int64_t k, const float v[8], float s) {
    const int64_t base = ch * 8;
    int sum = 0;
    if (VEC && base + 8 <= k) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int c0 = code_i8(v[j], s), c1 = code_i8(v[j + 4], s);
            sum += c0 + c1;
            lo |= (uint32_t)(c0 & 0xff) << (8 * j);
            hi |= (uint32_t)(c1 & 0xff) << (8 * j);
        }
        *reinterpret_cast<uint2 *>(qrow + base) = make_uint2(lo, hi);
    } else {
#pragma unroll
        for (int j = 0; j < 8; j++) {
            if (base + j < k) {
                int c = code_i8(v[j], s);
                sum += c;
                qrow[base + j] = (int8_t)c;
            }
        }
    }
    return sum;
}

// The RMSNorm factor r = 1 / sqrt(ss / k + eps_norm) (1 without RMSNorm) and
// the guarded absmax a' = max(a, eps_q / r).  The quantizer sees the
// normalized row r x, whose absmax r a is guarded by eps_q; in the units of x
// that guard is eps_q / r = eps_q * sqrt(ss / k + eps_norm).  Without RMSNorm
// a' = max(a, eps_q) exactly.
template <bool RMS>
__device__ __forceinline__ void guarded_absmax(float amax, float ss, int64_t k, float eps_norm, float eps_q,
                                               float &r, float &ap) {
    float t = eps_q;
    r = 1.0f;
    if (RMS) {
        const float d = sqrtf(__fadd_rn(__fdiv_rn(ss, (float)k), eps_norm));
        r = __fdiv_rn(1.0f, d);
        t = __fmul_rn(eps_q, d);
    }
    ap = amax > t ? amax : t;
}

// Block-wide reduction of one value through LDS after a wave reduction; the
// four wave results are combined in a fixed order, so the result does not
// depend on scheduling.
template <typename T, bool MAX>
__device__ __forceinline__ T block_reduce(T v, T *lds) {
    v = MAX ? wave_max(v) : wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) lds[w] = v;
    __syncthreads();
    T r = lds[0];
#pragma unroll
    for (int i = 1; i < kQThreads / kWave; i++) r = MAX ? (lds[i] > r ? lds[i] : r) : r + lds[i];
    __syncthreads();
    return r;
}

template <int K, bool VEC, bool RMS>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(const void *__restrict__ x, int64_t k,
                                                              float eps_norm, float eps_q,
                                                              int8_t *__restrict__ q,
                                                              float *__restrict__ pts,
                                                              int32_t *__restrict__ rowsum) {
    __shared__ float red_f[kQThreads / kWave];
    __shared__ int red_i[kQThreads / kWave];
    const int64_t row = blockIdx.x;
    const int esz = K == IN_F32 ? 4 : 2;
    const void *xr = static_cast<const char *>(x) + row * k * esz;
    int8_t *qr = q + row * k;
    const int64_t nchunk = (k + 7) / 8;
    const int tid = threadIdx.x;

    float cache[kQCache][8];
    float amax = 0.0f, ss = 0.0f;
#pragma unroll
    for (int c = 0; c < kQCache; c++) {
        const int64_t ch = (int64_t)c * kQThreads + tid;
        if (ch < nchunk) {
            load_chunk<K, VEC>(xr, ch, k, cache[c]);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                amax = fmaxf(amax, fabsf(cache[c][j]));
                if (RMS) ss += cache[c][j] * cache[c][j];
            }
        }
    }
    for (int64_t ch = (int64_t)kQCache * kQThreads + tid; ch < nchunk; ch += kQThreads) {
        float v[8];
        load_chunk<K, VEC>(xr, ch, k, v);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            amax = fmaxf(amax, fabsf(v[j]));
            if (RMS) ss += v[j] * v[j];
        }
    }
    amax = block_reduce<float, true>(amax, red_f);
    if (RMS) ss = block_reduce<float, false>(ss, red_f);

    float r, ap;
    guarded_absmax<RMS>(amax, ss, k, eps_norm, eps_q, r, ap);
    const float s = __fdiv_rn(127.0f, ap);

    int rs = 0;
#pragma unroll
    for (int c = 0; c < kQCache; c++) {
        const int64_t ch = (int64_t)c * kQThreads + tid;
        if (ch < nchunk) rs += store_chunk<VEC>(qr, ch, k, cache[c], s);
    }
    for (int64_t ch = (int64_t)kQCache * kQThreads + tid; ch < nchunk; ch += kQThreads) {
        float v[8];
        load_chunk<K, VEC>(xr, ch, k, v);
        rs += store_chunk<VEC>(qr, ch, k, v, s);
    }
    rs = block_reduce<int, false>(rs, red_i);

    if (tid == 0) {
        pts[row] = RMS ? __fdiv_rn(__fmul_rn(ap, r), 127.0f) : __fdiv_rn(ap, 127.0f);
        if (rowsum) rowsum[row] = rs;
    }
}

// One 8-element chunk as raw words (16 bytes for 16-bit kinds, 32 for fp32)
// and its conversion to fp32, apart, so that a kernel can issue every chunk
// load before it converts any: the scheduler would otherwise place the
// first conversions, and the wait for their load, among the later loads.
template <int K>
__device__ __forceinline__ void load_chunk_raw(const void *row, int64_t ch, uint4 (&r)[2]) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const char *>(row) + ch * 8 * (K == IN_F32 ? 4 : 2));
    r[0] = p[0];
    if constexpr (K == IN_F32) r[1] = p[1];
}

template <int K>
__device__ __forceinline__ void chunk_to_f32(const uint4 (&r)[2], float v[8]) {
    if constexpr (K == IN_F32) {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = __uint_as_float(w[j]);
    } else {
        const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
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

// The int8 codes of eight values packed into two words (element j in byte
// j % 4 of lo (j < 4) or hi), and rs plus their sum.  The code of v is
// clamp(rint(fl(v * s)), -128, 127): clamping first (the bounds are
// integers) and adding 1.5 * 2^23 rounds the value to an integer, ties to
// even, in the low mantissa bits, so the word is 0x4B400000 + code, whose low
// byte is the code's byte.  The sum is a 4-way signed byte dot product of the
// packed codes with ones.
__device__ __forceinline__ int pack_codes8(const float (&v)[8], float s, int rs, uint32_t &lo, uint32_t &hi) {
    constexpr float kRound = 12582912.0f;
    uint32_t y[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const float t = fminf(fmaxf(__fmul_rn(v[j], s), -128.0f), 127.0f);
        y[j] = __float_as_uint(__fadd_rn(t, kRound));
    }
    lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[3], y[2], 0x0c0c0400u),
                               __builtin_amdgcn_perm(y[1], y[0], 0x0c0c0400u), 0x05040100u);
    hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(y[7], y[6], 0x0c0c0400u),
                               __builtin_amdgcn_perm(y[5], y[4], 0x0c0c0400u), 0x05040100u);
    rs = __builtin_amdgcn_sdot4((int)lo, 0x01010101, rs, false);
    return __builtin_amdgcn_sdot4((int)hi, 0x01010101, rs, false);
}

// One wave per token row for rows of at most 64 * NCH whole 8-element
// chunks: lane l holds chunks l, l + 64, ... in registers.  Every load is
// unconditional (a chunk index past the row is clamped to the last chunk and
// its values are masked to zero), so all of a lane's loads are in flight
// together; absmax, sum of squares and the code sum are wave64 shuffle
// reductions, with no LDS and no barrier.
constexpr int kQWaveRows = 4;  // rows (waves) per workgroup

template <int K, int NCH, bool RMS, bool FULL>
__global__ __launch_bounds__(kQWaveRows * kWave) void quant_act_wave_kernel(const void *__restrict__ x,
                                                                            int64_t m, int64_t k,
                                                                            float eps_norm, float eps_q,
                                                                            int8_t *__restrict__ q,
                                                                            float *__restrict__ pts,
                                                                            int32_t *__restrict__ rowsum) {
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * kQWaveRows + wave_id();
    if (row >= m) return;
    const int esz = K == IN_F32 ? 4 : 2;
    const void *xr = static_cast<const char *>(x) + row * k * esz;
    int8_t *qr = q + row * k;
    const int64_t nchunk = k / 8;

    float v[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int64_t ch = (int64_t)c * kWave + lane;
        load8_vec<K>(xr, (ch < nchunk ? ch : nchunk - 1) * 8, v[c]);
    }
    float amax = 0.0f, ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const bool in = FULL || (int64_t)c * kWave + lane < nchunk;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float e = in ? v[c][j] : 0.0f;
            v[c][j] = e;
            amax = fmaxf(amax, fabsf(e));
            if (RMS) ss += e * e;
        }
    }
    amax = wave_max(amax);
    if (RMS) ss = wave_sum(ss);

    float r, ap;
    guarded_absmax<RMS>(amax, ss, k, eps_norm, eps_q, r, ap);
    const float s = __fdiv_rn(127.0f, ap);
    int rs = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int64_t ch = (int64_t)c * kWave + lane;
        uint32_t lo, hi;
        rs = pack_codes8(v[c], s, rs, lo, hi);
        if (FULL || ch < nchunk) *reinterpret_cast<uint2 *>(qr + ch * 8) = make_uint2(lo, hi);
    }
    rs = wave_sum(rs);
    if (lane == 0) {
        pts[row] = RMS ? __fdiv_rn(__fmul_rn(ap, r), 127.0f) : __fdiv_rn(ap, 127.0f);
        if (rowsum) rowsum[row] = rs;
    }
}

// W waves per token row (W = 2 or 4), for rows the wave kernel would hold
// as at least eight chunks per lane when a launch leaves room for more
// waves: wave w holds chunks
// 64 (w NCH + c) + l, c < NCH, so a row's loads are spread over W waves and
// each wave's share of the code step, which follows the last of its loads,
// is 1 / W of the row's.  The W wave results of absmax and the sum of
// squares are combined through LDS in wave order, the code sums likewise;
// codes and code sums are those of the one-wave kernel (absmax is exact),
// the sum of squares is added in another order.
template <int K, int NCH, int W, bool RMS, bool FULL>
__global__ __launch_bounds__(W * kWave) void quant_act_split_kernel(const void *__restrict__ x, int64_t k,
                                                                    float eps_norm, float eps_q,
                                                                    int8_t *__restrict__ q,
                                                                    float *__restrict__ pts,
                                                                    int32_t *__restrict__ rowsum) {
    __shared__ float red_a[W], red_s[W];
    __shared__ int red_r[W];
    const int lane = threadIdx.x % kWave, w = wave_id();
    const int64_t row = blockIdx.x;
    const int esz = K == IN_F32 ? 4 : 2;
    const void *xr = static_cast<const char *>(x) + row * k * esz;
    int8_t *qr = q + row * k;
    const int64_t nchunk = k / 8;

    uint4 raw[NCH][2];
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int64_t ch = (int64_t)(w * NCH + c) * kWave + lane;
        load_chunk_raw<K>(xr, FULL || ch < nchunk ? ch : nchunk - 1, raw[c]);
    }
    __builtin_amdgcn_sched_barrier(0);
    float v[NCH][8];
#pragma unroll
    for (int c = 0; c < NCH; c++) chunk_to_f32<K>(raw[c], v[c]);
    float amax = 0.0f, ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const bool in = FULL || (int64_t)(w * NCH + c) * kWave + lane < nchunk;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const float e = in ? v[c][j] : 0.0f;
            v[c][j] = e;
            amax = fmaxf(amax, fabsf(e));
            if (RMS) ss += e * e;
        }
    }
    amax = wave_max(amax);
    if (RMS) ss = wave_sum(ss);
    if (lane == 0) {
        red_a[w] = amax;
        red_s[w] = ss;
    }
    __syncthreads();
    amax = red_a[0];
    ss = red_s[0];
#pragma unroll
    for (int i = 1; i < W; i++) {
        amax = fmaxf(amax, red_a[i]);
        ss += red_s[i];
    }

    float r, ap;
    guarded_absmax<RMS>(amax, ss, k, eps_norm, eps_q, r, ap);
    const float s = __fdiv_rn(127.0f, ap);
    int rs = 0;
#pragma unroll
    for (int c = 0; c < NCH; c++) {
        const int64_t ch = (int64_t)(w * NCH + c) * kWave + lane;
        uint32_t lo, hi;
        rs = pack_codes8(v[c], s, rs, lo, hi);
        if (FULL || ch < nchunk) *reinterpret_cast<uint2 *>(qr + ch * 8) = make_uint2(lo, hi);
    }
    rs = wave_sum(rs);
    if (lane == 0) red_r[w] = rs;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = red_r[0];
#pragma unroll
        for (int i = 1; i < W; i++) t += red_r[i];
        pts[row] = RMS ? __fdiv_rn(__fmul_rn(ap, r), 127.0f) : __fdiv_rn(ap, 127.0f);
        if (rowsum) rowsum[row] = t;
    }
}

template <int K, int NCH>
hipError_t launch_wave_rows(bool rms, const void *x, int64_t m, int64_t k, float eps_norm, float eps_q,
                            int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    const unsigned grid = (unsigned)((m + kQWaveRows - 1) / kQWaveRows);
    // rows of exactly 64 NCH chunks need no per-lane masking
    const bool full = k == (int64_t)NCH * kWave * 8;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kQWaveRows * kWave), 0, st, x, m, k, eps_norm, eps_q, q, pts,
                           rowsum);
    };
    if (rms) full ? go(quant_act_wave_kernel<K, NCH, true, true>) : go(quant_act_wave_kernel<K, NCH, true, false>);
    else full ? go(quant_act_wave_kernel<K, NCH, false, true>) : go(quant_act_wave_kernel<K, NCH, false, false>);
    return hipGetLastError();
}

// Rows of whole 8-element chunks up to 8192 elements take the wave-per-row
// kernel, sized to the row; anything else the workgroup-per-row kernel.
template <int K, int W, int NCH>
hipError_t launch_split_rows(bool rms, const void *x, int64_t m, int64_t k, float eps_norm, float eps_q,
                             int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    const bool full = k == (int64_t)W * NCH * kWave * 8;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)m), dim3(W * kWave), 0, st, x, k, eps_norm, eps_q, q, pts, rowsum);
    };
    if (rms) full ? go(quant_act_split_kernel<K, NCH, W, true, true>) : go(quant_act_split_kernel<K, NCH, W, true, false>);
    else full ? go(quant_act_split_kernel<K, NCH, W, false, true>) : go(quant_act_split_kernel<K, NCH, W, false, false>);
    return hipGetLastError();
}

// W waves per row for rows of more than 3584 elements (at least eight chunks
// per lane with one wave) while the launch has at most 16384 waves (16 per
// SIMD).  Measured on MI355X, bf16 with RMSNorm, us per graph-replayed
// launch for W = 1 / 2 / 4 / 8: rows of 4096: 512 rows 4.12 / 3.91 / 3.69
// / 3.95, 2048 rows 7.60-7.64 / 7.18-7.27 / 7.07-7.09 / 9.33, 8192 rows
// 19.1-19.3 / 18.6-18.8 / 19.8-20.1 / 27.7-28.0; rows of 8192 (W = 4): 1 /
// 16 / 256 / 2048 rows 3.6 / 4.1 / 5.2 / 12.4 -> 2.5 / 2.8 / 3.8 / 11.0.
// Shorter rows stay on one wave: 4096 rows of 2048 6.85 with W = 1 against
// 7.26 with W = 2 and 9.0 with W = 4; 1024 rows of 1024 2.99 against 3.27
// with W = 2.
template <int K, int W>
hipError_t launch_split_w(int64_t per_lane, bool rms, const void *x, int64_t m, int64_t k, float eps_norm,
                          float eps_q, int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    const int64_t nch = (per_lane + W - 1) / W;
    if (nch <= 1) return launch_split_rows<K, W, 1>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    if (nch <= 2) return launch_split_rows<K, W, 2>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    if (nch <= 4) return launch_split_rows<K, W, 4>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    return launch_split_rows<K, W, 8>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
}

template <int K>
bool try_wave_rows(hipError_t &err, bool rms, const void *x, int64_t m, int64_t k, float eps_norm,
                   float eps_q, int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    if (k % 8 != 0 || k > 8192) return false;
    const int64_t per_lane = (k / 8 + kWave - 1) / kWave;
    if (per_lane >= 8 && m <= 16384 / 4) {
        err = launch_split_w<K, 4>(per_lane, rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
        return true;
    }
    if (per_lane >= 8 && m <= 16384 / 2) {
        err = launch_split_w<K, 2>(per_lane, rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
        return true;
    }
    if (per_lane <= 2) err = launch_wave_rows<K, 2>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    else if (per_lane <= 4) err = launch_wave_rows<K, 4>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    else if (per_lane <= 8) err = launch_wave_rows<K, 8>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    else err = launch_wave_rows<K, 16>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    return true;
}

constexpr int kI4Threads = 256;

__device__ __forceinline__ uint32_t code_i4(float v, float sp, float r) {
    return (uint32_t)((int)code_i4_f(v, sp, r)) & 0xffu;
}

template <int K, bool VEC>
__global__ __launch_bounds__(kI4Threads) void quant_int4_tensor_kernel(const void *__restrict__ x,
                                                                       int64_t count,
                                                                       const float *__restrict__ scale,
                                                                       float eps,
                                                                       int8_t *__restrict__ q) {
    const float sc = *scale;
    const float sp = sc > eps ? sc : eps;
    const float r = __fdiv_rn(1.0f, sp);
    const int64_t nchunk = (count + 7) / 8;
    const int64_t stride = (int64_t)gridDim.x * kI4Threads;
    for (int64_t ch = (int64_t)blockIdx.x * kI4Threads + threadIdx.x; ch < nchunk; ch += stride) {
        const int64_t base = ch * 8;
        if (VEC && base + 8 <= count) {
            float v[8];
            load8_vec<K>(x, base, v);
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                lo |= code_i4(v[j], sp, r) << (8 * j);
                hi |= code_i4(v[j + 4], sp, r) << (8 * j);
            }
            *reinterpret_cast<uint2 *>(q + base) = make_uint2(lo, hi);
        } else {
            for (int j = 0; j < 8 && base + j < count; j++)
                q[base + j] = (int8_t)code_i4(load_elem<K>(x, base + j), sp, r);
        }
    }
}

// 4-bit codes as FP6 E3M2 operand tiles of the 4-bit product.  One thread
// per slot: slot l of tile (rb, ks) holds row 32rb + l%32, k 64ks + 32(l/32)
// .. +31; rows and k past the tensor are zero codes.  Every code in [-8, 7]
// is exact in E3M2, so the hardware conversion packs them without rounding;
// it interleaves its two 16-value sources (even element from the first), so
// the even and odd elements are passed apart.  The 6-dword image is written
// as 16 bytes at tile byte 16l and 8 bytes at 1024 + 8l: both stores of a
// wave are contiguous.
template <int K, bool VEC>
__global__ __launch_bounds__(kI4Threads) void quant_a4w4_tiles_kernel(const void *__restrict__ x, int64_t rows,
                                                                      int64_t k, const float *__restrict__ scale,
                                                                      float eps, int64_t ktiles, int64_t slots,
                                                                      uint8_t *__restrict__ tiles) {
    const int64_t t = (int64_t)blockIdx.x * kI4Threads + threadIdx.x;
    if (t >= slots) return;
    const float sc = *scale;
    const float sp = sc > eps ? sc : eps;
    const float r = __fdiv_rn(1.0f, sp);
    const int64_t tile = t / 64;
    const int l = (int)(t % 64);
    const int64_t row = 32 * (tile / ktiles) + l % 32;
    const int64_t k0 = 64 * (tile % ktiles) + 32 * (l / 32);
    float v[32];
    if (VEC && row < rows && k0 + 32 <= k) {
        const int64_t base = row * k + k0;
#pragma unroll
        for (int c = 0; c < 4; c++) load8_vec<K>(x, base + 8 * c, v + 8 * c);
    } else {
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] = (row < rows && k0 + j < k) ? load_elem<K>(x, row * k + k0 + j) : 0.0f;
    }
    v16f ev, od;
#pragma unroll
    for (int j = 0; j < 16; j++) {
        ev[j] = code_i4_f(v[2 * j], sp, r);
        od[j] = code_i4_f(v[2 * j + 1], sp, r);
    }
    const v6u img = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, 1.0f);
    uint8_t *dst = tiles + tile * 1536;
    *reinterpret_cast<uint4 *>(dst + 16 * l) = make_uint4(img[0], img[1], img[2], img[3]);
    *reinterpret_cast<uint2 *>(dst + 1024 + 8 * l) = make_uint2(img[4], img[5]);
}

// 4-bit codes as the packed two-per-byte operand: the tile grid of the FP6
// operand, 1024 bytes per tile, slot l (row 32rb + l%32, k 64ks + 32(l/32)
// .. +31) the 16 bytes at 16l.  Element j goes to word j/8, nibble j%8/2
// (even j) or 4 + j%8/2 (odd j), as code + 8, so that
// (word >> 4i) & 0x000F000F holds the elements 8w + 2i and 8w + 2i + 1 in
// its two halves.  One thread per slot; a wave writes 1 KB contiguously.
template <int K, bool VEC>
__global__ __launch_bounds__(kI4Threads) void quant_a4w4_packed_kernel(const void *__restrict__ x, int64_t rows,
                                                                       int64_t k, const float *__restrict__ scale,
                                                                       float eps, int64_t ktiles, int64_t slots,
                                                                       uint8_t *__restrict__ tiles) {
    const int64_t t = (int64_t)blockIdx.x * kI4Threads + threadIdx.x;
    if (t >= slots) return;
    const float sc = *scale;
    const float sp = sc > eps ? sc : eps;
    const float r = __fdiv_rn(1.0f, sp);
    const int64_t tile = t / 64;
    const int l = (int)(t % 64);
    const int64_t row = 32 * (tile / ktiles) + l % 32;
    const int64_t k0 = 64 * (tile % ktiles) + 32 * (l / 32);
    float v[32];
    if (VEC && row < rows && k0 + 32 <= k) {
        const int64_t base = row * k + k0;
#pragma unroll
        for (int c = 0; c < 4; c++) load8_vec<K>(x, base + 8 * c, v + 8 * c);
    } else {
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] = (row < rows && k0 + j < k) ? load_elem<K>(x, row * k + k0 + j) : 0.0f;
    }
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t nib = (uint32_t)((int)code_i4_f(v[8 * q + e], sp, r) + 8);
            word |= nib << (4 * ((e % 2 == 0) ? e / 2 : 4 + e / 2));
        }
        w[q] = word;
    }
    *reinterpret_cast<uint4 *>(tiles + tile * 1024 + 16 * l) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <int K, bool VEC, bool RMS>
hipError_t launch_quant_act_t(const void *x, int64_t m, int64_t k, float eps_norm, float eps_q,
                              int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    hipLaunchKernelGGL((quant_act_kernel<K, VEC, RMS>), dim3((unsigned)m), dim3(kQThreads), 0, st,
                       x, k, eps_norm, eps_q, q, pts, rowsum);
    return hipGetLastError();
}

template <int K, bool VEC>
hipError_t launch_quant_act_k(bool rms, const void *x, int64_t m, int64_t k, float eps_norm,
                              float eps_q, int8_t *q, float *pts, int32_t *rowsum, hipStream_t st) {
    return rms ? launch_quant_act_t<K, VEC, true>(x, m, k, eps_norm, eps_q, q, pts, rowsum, st)
               : launch_quant_act_t<K, VEC, false>(x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
}

template <int K>
hipError_t launch_quant_act_v(bool vec, bool rms, const void *x, int64_t m, int64_t k,
                              float eps_norm, float eps_q, int8_t *q, float *pts, int32_t *rowsum,
                              hipStream_t st) {
    return vec ? launch_quant_act_k<K, true>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st)
               : launch_quant_act_k<K, false>(rms, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
}

template <int K>
hipError_t launch_i4_v(bool vec, const void *x, int64_t count, const float *scale, float eps,
                       int8_t *q, hipStream_t st) {
    const int64_t nchunk = (count + 7) / 8;
    int64_t blocks = (nchunk + kI4Threads - 1) / kI4Threads;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (vec)
        hipLaunchKernelGGL((quant_int4_tensor_kernel<K, true>), dim3((unsigned)blocks),
                           dim3(kI4Threads), 0, st, x, count, scale, eps, q);
    else
        hipLaunchKernelGGL((quant_int4_tensor_kernel<K, false>), dim3((unsigned)blocks),
                           dim3(kI4Threads), 0, st, x, count, scale, eps, q);
    return hipGetLastError();
}

template <int K>
hipError_t launch_a4w4_tiles_k(bool vec, const void *x, int64_t rows, int64_t k, const float *scale, float eps,
                               uint8_t *tiles, hipStream_t st) {
    const int64_t ktiles = (k + 127) / 128 * 2, slots = (rows + 31) / 32 * ktiles * 64;
    const int64_t blocks = (slots + kI4Threads - 1) / kI4Threads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL((quant_a4w4_tiles_kernel<K, true>), dim3((unsigned)blocks), dim3(kI4Threads), 0, st, x,
                           rows, k, scale, eps, ktiles, slots, tiles);
    else
        hipLaunchKernelGGL((quant_a4w4_tiles_kernel<K, false>), dim3((unsigned)blocks), dim3(kI4Threads), 0, st, x,
                           rows, k, scale, eps, ktiles, slots, tiles);
    return hipGetLastError();
}

template <int K>
hipError_t launch_a4w4_packed_k(bool vec, const void *x, int64_t rows, int64_t k, const float *scale, float eps,
                                uint8_t *tiles, hipStream_t st) {
    const int64_t ktiles = (k + 127) / 128 * 2, slots = (rows + 31) / 32 * ktiles * 64;
    const int64_t blocks = (slots + kI4Threads - 1) / kI4Threads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (vec)
        hipLaunchKernelGGL((quant_a4w4_packed_kernel<K, true>), dim3((unsigned)blocks), dim3(kI4Threads), 0, st, x,
                           rows, k, scale, eps, ktiles, slots, tiles);
    else
        hipLaunchKernelGGL((quant_a4w4_packed_kernel<K, false>), dim3((unsigned)blocks), dim3(kI4Threads), 0, st, x,
                           rows, k, scale, eps, ktiles, slots, tiles);
    return hipGetLastError();
}

}  // namespace

size_t a4w4_packed_bytes(int64_t rows, int64_t k) {
    return (size_t)((rows + 31) / 32 * 32) * (size_t)((k + 127) / 128 * 128) / 2;
}

hipError_t launch_quant_a4w4_packed(int in_kind, const void *x, int64_t rows, int64_t k, const float *scale,
                                    float eps, uint8_t *tiles, hipStream_t st) {
    const bool vec = (k % 8) == 0;
    switch (in_kind) {
        case IN_F32: return launch_a4w4_packed_k<IN_F32>(vec, x, rows, k, scale, eps, tiles, st);
        case IN_F16: return launch_a4w4_packed_k<IN_F16>(vec, x, rows, k, scale, eps, tiles, st);
        default: return launch_a4w4_packed_k<IN_BF16>(vec, x, rows, k, scale, eps, tiles, st);
    }
}

size_t a4w4_operand_bytes(int64_t rows, int64_t k) {
    return (size_t)((rows + 31) / 32 * 32) * (size_t)((k + 127) / 128 * 128) * 3 / 4;
}

hipError_t launch_quant_a4w4_tiles(int in_kind, const void *x, int64_t rows, int64_t k, const float *scale,
                                   float eps, uint8_t *tiles, hipStream_t st) {
    // whole 8-element vector loads need every row 16-byte aligned
    const bool vec = (k % 8) == 0;
    switch (in_kind) {
        case IN_F32: return launch_a4w4_tiles_k<IN_F32>(vec, x, rows, k, scale, eps, tiles, st);
        case IN_F16: return launch_a4w4_tiles_k<IN_F16>(vec, x, rows, k, scale, eps, tiles, st);
        default: return launch_a4w4_tiles_k<IN_BF16>(vec, x, rows, k, scale, eps, tiles, st);
    }
}

hipError_t launch_quant_act(int in_kind, const void *x, int64_t m, int64_t k, bool rmsnorm,
                            float eps_norm, float eps_q, int8_t *q, float *pts, int32_t *rowsum,
                            hipStream_t st) {
    // Vector path: every row starts 16-byte aligned and holds whole 8-element
    // chunks, and the int8 code row is 8-byte aligned.
    const bool vec = (k % 8) == 0;
    hipError_t err = hipSuccess;
    const bool done = in_kind == IN_F32
                          ? try_wave_rows<IN_F32>(err, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st)
                          : in_kind == IN_F16
                                ? try_wave_rows<IN_F16>(err, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st)
                                : try_wave_rows<IN_BF16>(err, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    if (done) return err;
    switch (in_kind) {
        case IN_F32: return launch_quant_act_v<IN_F32>(vec, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
        case IN_F16: return launch_quant_act_v<IN_F16>(vec, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
        default: return launch_quant_act_v<IN_BF16>(vec, rmsnorm, x, m, k, eps_norm, eps_q, q, pts, rowsum, st);
    }
}

hipError_t launch_quant_int4_tensor(int in_kind, const void *x, int64_t count, const float *scale,
                                    float eps, int8_t *q, hipStream_t st) {
    // base pointers are 16-byte aligned; chunk starts are multiples of 8
    // elements, so the vector path is always aligned.
    const bool vec = true;
    switch (in_kind) {
        case IN_F32: return launch_i4_v<IN_F32>(vec, x, count, scale, eps, q, st);
        case IN_F16: return launch_i4_v<IN_F16>(vec, x, count, scale, eps, q, st);
        default: return launch_i4_v<IN_BF16>(vec, x, count, scale, eps, q, st);
    }
}

}  // namespace ql
