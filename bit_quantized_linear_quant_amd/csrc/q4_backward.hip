// Q4Linear backward on gfx950 ("Q4LinearFunction" backward: gradients for
// the input, the weight and the activation scale from the output gradient,
// adjusted to the quantization ranges; none for scale_w and eps).
//
// With the forward y = Xh Wh^T, Xh = s'_a q_a, Wh = s'_w q_w (4-bit codes
// q = clamp(rne(v), -8, 7) of the quotients v = fl32(X / s')), the
// straight-through reading is
//   grad_x = (G Wh) * [-8 <= v_a <= 7],  grad_w = (G^T Xh) * [-8 <= v_w <= 7],
//   grad_scale_a = sum (G Wh) * (q_a - v_a [-8 <= v_a <= 7])  if scale_a > eps.
//
// Both products contract over a dimension that is not contiguous in the
// forward's tensors, so the operands are first written k-contiguous in the
// workspace, zero-padded to a multiple of 32 along the contraction:
//   G  [m, n]  -> Gp  [m, n_p]  (only when n % 32 != 0)
//   G  [m, n]  -> Gt  [n, m_p]
//   W  [n, k]  -> Cwt [k, n_p]  4-bit codes of W, as exact 16-bit integers
//   X  [m, k]  -> Cxt [k, m_p]  4-bit codes of X
// Then grad_x = G Cwt^T (scaled by s'_w) and grad_w = Gt Cxt^T (scaled by
// s'_a) run on the 256 x 256 tile ring of gemm_ring.hpp with the fp16 or
// bf16 32x32x16 matrix-core product (codes are exact in both types, fp32
// accumulation).  The epilogue reads X (or W) at each output element,
// recomputes its quotient and code exactly as the forward did, applies the
// range mask and, for grad_x, accumulates the step-size term in fp64: one
// partial per wave, summed in a fixed order by a final kernel, so the scale
// gradient is deterministic.
#include "ql_device.hpp"
#include "ql_launch.hpp"
#include "gemm_ring.hpp"

namespace ql {

namespace {

constexpr int kTT = 64;          // transpose tile: 64 x 64 elements
constexpr int kTThreads = 256;

// 16-bit bits of a small integer (exact in fp16 and bf16).
template <int MK>
__device__ __forceinline__ uint16_t int_bits16(float c) {
    if constexpr (MK == MK_F16) return f32_to_f16_rne(c);
    else return f32_to_bf16_rne(c);
}

// dst[c][r] = f(src[r][c]) for r < rows, c < cols; dst rows are ld_dst
// (>= rows, a multiple of 32) elements long and dst[c][r] = 0 for
// rows <= r < ld_dst.  CODES: f = the 4-bit code of src / max(*scale, eps)
// as a 16-bit integer of the product type; otherwise f copies the 16-bit
// pattern (src already of the product type).  Each 256-thread workgroup
// moves a 64 x 64 tile through a padded LDS tile.
template <int IN, int MK, bool CODES, bool VEC>
__global__ __launch_bounds__(kTThreads) void bwd_transpose_kernel(const void *__restrict__ src, int64_t rows,
                                                                  int64_t cols, int64_t ld_dst,
                                                                  const float *__restrict__ scale, float eps,
                                                                  uint16_t *__restrict__ dst) {
    __shared__ uint16_t tile[kTT][kTT + 2];
    const int64_t r0 = (int64_t)blockIdx.y * kTT, c0 = (int64_t)blockIdx.x * kTT;
    const int t = threadIdx.x;
    float sp = 0.f, rcp = 0.f;
    if constexpr (CODES) {
        const float sc = *scale;
        sp = sc > eps ? sc : eps;
        rcp = __fdiv_rn(1.0f, sp);
    }
    {
        // load: thread t reads row t / 4, 16 columns from 16 (t % 4)
        const int lr = t / 4, lc = 16 * (t % 4);
        const int64_t r = r0 + lr, c = c0 + lc;
        float v[16];
        uint16_t raw[16];
        if (VEC && r < rows && c + 16 <= cols) {
            if constexpr (CODES) {
                load8_vec<IN>(src, r * cols + c, v);
                load8_vec<IN>(src, r * cols + c + 8, v + 8);
            } else {
                const uint4 a = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + r * cols + c);
                const uint4 b = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + r * cols + c + 8);
                const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    raw[2 * j] = (uint16_t)wv[j];
                    raw[2 * j + 1] = (uint16_t)(wv[j] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const bool ok = r < rows && c + j < cols;
                if constexpr (CODES) v[j] = ok ? load_elem<IN>(src, r * cols + c + j) : 0.0f;
                else raw[j] = ok ? static_cast<const uint16_t *>(src)[r * cols + c + j] : (uint16_t)0;
            }
        }
#pragma unroll
        for (int j = 0; j < 16; j++) {
            if constexpr (CODES) tile[lr][lc + j] = (r < rows && c + j < cols) ? int_bits16<MK>(code_i4_f(v[j], sp, rcp)) : 0;
            else tile[lr][lc + j] = raw[j];
        }
    }
    __syncthreads();
    {
        // store: thread t writes dst row c0 + t / 4, 16 elements from r0 + 16 (t % 4)
        const int lc = t / 4, lr = 16 * (t % 4);
        const int64_t c = c0 + lc, r = r0 + lr;
        if (c < cols && r < ld_dst) {
            uint32_t wv[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t lo = (r + 2 * j < rows) ? tile[lr + 2 * j][lc] : 0u;
                const uint32_t hi = (r + 2 * j + 1 < rows) ? tile[lr + 2 * j + 1][lc] : 0u;
                wv[j] = lo | (hi << 16);
            }
            uint16_t *d = dst + c * ld_dst + r;
            if (r + 16 <= ld_dst) {
                reinterpret_cast<uint4 *>(d)[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                reinterpret_cast<uint4 *>(d)[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
            } else {
#pragma unroll
                for (int j = 0; j < 16; j++)
                    if (r + j < ld_dst) d[j] = (uint16_t)(wv[j / 2] >> (16 * (j % 2)));
            }
        }
    }
}

// dst[r][c] = src[r][c] for c < cols, 0 for cols <= c < ld_dst (16-bit).
__global__ __launch_bounds__(kTThreads) void bwd_pad_kernel(const uint16_t *__restrict__ src, int64_t rows,
                                                            int64_t cols, int64_t ld_dst, uint16_t *__restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * kTThreads + threadIdx.x;
    if (i >= rows * ld_dst) return;
    const int64_t r = i / ld_dst, c = i % ld_dst;
    dst[i] = c < cols ? src[r * cols + c] : (uint16_t)0;
}

// Threads of a backward product's workgroup: eight waves on the
// phase-alternating ring (ring_gemm_pp).
constexpr int kBwdThreads = 2 * LThreads;

struct BwdParams {
    const int8_t *a;       // [rows_a][kc] 16-bit
    const int8_t *b;       // [rows_b][kc] 16-bit
    int64_t rows_a, rows_b, kbytes;
    const void *src;       // [rows_a][rows_b]: the tensor whose codes gate the gradient
    const float *src_scale;
    const float *val_scale; // the other tensor's scale: multiplies the product
    float eps;
    void *out;             // [rows_a][rows_b]
    double *partials;      // one per wave (step-size term), or NULL
};

// One 32-column block J of a wave's 128 x 64 sub-tile of the backward
// epilogue: the products d = acc * s'_v go to a padded LDS block (lane
// holds column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4 of register r
// of each 32x32 block), then each lane takes 8 runs of 8 columns of one
// row: one 16-byte load of the source values (all 8 issued before any is
// used), the mask and step-size term, and 8 outputs written together.  J is
// a template argument so the accumulators are indexed statically.
template <int J, int IN, int OUT, bool LSQ>
__device__ __forceinline__ void bwd_epi_block(const BwdParams &p, const v16f (&acc)[4][2], float *ep, bool vec,
                                              int64_t m0, int64_t n0, int wm, int wn, int lane, float sv, float sp,
                                              float rcp, double &part) {
    constexpr int j = J;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int lr = 32 * i + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
            ep[lr * 33 + lane % 32] = __fmul_rn(acc[i][j][r], sv);
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the block is in LDS
    __builtin_amdgcn_wave_barrier();
    const int64_t cb = n0 + wn * 64 + 32 * j;
    if (vec) {
        uint4 raw[8];
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int q = lane + 64 * t;
            const int64_t row = m0 + wm * 128 + q / 4, col = cb + 8 * (q % 4);
            const int64_t rc = row < p.rows_a ? row : p.rows_a - 1, cc = col < p.rows_b ? col : p.rows_b - 8;
            raw[t] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.src) + rc * p.rows_b + cc);
        }
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int q = lane + 64 * t, lr = q / 4, lc = 8 * (q % 4);
            const int64_t row = m0 + wm * 128 + lr, col = cb + lc;
            if (row >= p.rows_a || col >= p.rows_b) continue;
            const uint32_t wv[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t bits = (wv[e / 2] >> (16 * (e % 2))) & 0xffffu;
                const float xv = IN == IN_F16 ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
                const float d = ep[lr * 33 + lc + e];
                const float v = q4_quotient(xv, sp, rcp);
                const bool in = v >= -8.0f && v <= 7.0f;
                o[e] = in ? d : 0.0f;
                if constexpr (LSQ) {
                    const float qc = q4_code(v);
                    part += (double)d * (double)(in ? qc - v : qc);
                }
            }
            const int64_t idx = row * p.rows_b + col;
            if constexpr (OUT == OUT_F32) {
                float4 *dst = reinterpret_cast<float4 *>(static_cast<float *>(p.out) + idx);
                dst[0] = make_float4(o[0], o[1], o[2], o[3]);
                dst[1] = make_float4(o[4], o[5], o[6], o[7]);
            } else {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t lo = OUT == OUT_F16 ? f32_to_f16_rne(o[2 * e]) : f32_to_bf16_rne(o[2 * e]);
                    const uint32_t hi = OUT == OUT_F16 ? f32_to_f16_rne(o[2 * e + 1]) : f32_to_bf16_rne(o[2 * e + 1]);
                    h[e] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + idx) = make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; t++) {
            const int q = lane + 64 * t, lr = q / 4, lc = 8 * (q % 4);
            const int64_t row = m0 + wm * 128 + lr;
            const int64_t rc = row < p.rows_a ? row : p.rows_a - 1;
            float xs[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int64_t col = cb + lc + e;
                xs[e] = load_elem<IN>(p.src, rc * p.rows_b + (col < p.rows_b ? col : p.rows_b - 1));
            }
            if (row >= p.rows_a) continue;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int64_t col = cb + lc + e;
                if (col >= p.rows_b) continue;
                const float d = ep[lr * 33 + lc + e];
                const float v = q4_quotient(xs[e], sp, rcp);
                const bool in = v >= -8.0f && v <= 7.0f;
                store_out<OUT>(p.out, row * p.rows_b + col, in ? d : 0.0f);
                if constexpr (LSQ) {
                    const float qc = q4_code(v);
                    part += (double)d * (double)(in ? qc - v : qc);
                }
            }
        }
    }
    // every lane of the wave has read the block before the next one is written
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    }

template <int MK, int IN, int OUT, bool LSQ>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_gemm_kernel(BwdParams p, int tiles_m, int tiles_n) {
    constexpr int BK = 64, NBUF = 3;
    constexpr int STAGE = 2 * BigTile<BK>::TILE;
    // the ring, then per wave a padded 128 x 32 fp32 block of the epilogue
    constexpr int EPI_BYTES = kBwdThreads / kWave * 128 * 33 * 4;
    constexpr int SMEM = NBUF * STAGE > EPI_BYTES ? NBUF * STAGE : EPI_BYTES;
    __shared__ __attribute__((aligned(1024))) int8_t smem[SMEM];

    const int lane = threadIdx.x % kWave, wave = wave_id();
    const int wm = wave % 2, wn = (wave / 2) % 4;
    int tm, tn;
    xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
    const int64_t m0 = (int64_t)tm * LB, n0 = (int64_t)tn * LB;
    v16f acc[4][2];
    ring_gemm_pp<BK, NBUF, MK>(acc, smem, p.a, p.b, p.rows_a, p.rows_b, p.kbytes, m0, n0, wm, wn, lane, wave);

    const float ss = *p.src_scale, vs = *p.val_scale;
    const float sp = ss > p.eps ? ss : p.eps, rcp = __fdiv_rn(1.0f, sp);
    const float sv = vs > p.eps ? vs : p.eps;
    double part = 0.0;
    float *ep = reinterpret_cast<float *>(smem) + wave * (128 * 33);
    const bool vec = (p.rows_b % 8) == 0;
    bwd_epi_block<0, IN, OUT, LSQ>(p, acc, ep, vec, m0, n0, wm, wn, lane, sv, sp, rcp, part);
    bwd_epi_block<1, IN, OUT, LSQ>(p, acc, ep, vec, m0, n0, wm, wn, lane, sv, sp, rcp, part);
    if constexpr (LSQ) {
        // one partial per wave, no workgroup barrier: a barrier here would
        // make every wave wait for its output stores to drain
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if (lane == 0) p.partials[(int64_t)blockIdx.x * (kBwdThreads / kWave) + wave] = part;
    }
}

// grad_scale_a = sum of the partials in a fixed order, 0 when scale_a <= eps.
__global__ __launch_bounds__(256) void bwd_scale_grad_kernel(const double *__restrict__ partials, int64_t count,
                                                             const float *__restrict__ scale, float eps,
                                                             float *__restrict__ grad) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < count; i += 256) s += partials[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *grad = *scale > eps ? (float)red[0] : 0.0f;
}

template <int IN, int MK, bool CODES>
hipError_t launch_transpose(const void *src, int64_t rows, int64_t cols, int64_t ld_dst, const float *scale,
                            float eps, uint16_t *dst, hipStream_t st) {
    dim3 grid((unsigned)((cols + kTT - 1) / kTT), (unsigned)((ld_dst + kTT - 1) / kTT));
    if (grid.y > 65535) return hipErrorInvalidValue;
    if (cols % 16 == 0)
        hipLaunchKernelGGL((bwd_transpose_kernel<IN, MK, CODES, true>), grid, dim3(kTThreads), 0, st, src, rows, cols,
                           ld_dst, scale, eps, dst);
    else
        hipLaunchKernelGGL((bwd_transpose_kernel<IN, MK, CODES, false>), grid, dim3(kTThreads), 0, st, src, rows,
                           cols, ld_dst, scale, eps, dst);
    return hipGetLastError();
}

template <int MK, int IN, int OUT, bool LSQ>
hipError_t launch_bwd_gemm(const BwdParams &p, hipStream_t st) {
    const int64_t tm = (p.rows_a + LB - 1) / LB, tn = (p.rows_b + LB - 1) / LB;
    if (tm * tn > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_gemm_kernel<MK, IN, OUT, LSQ>), dim3((unsigned)(tm * tn)), dim3(kBwdThreads), 0, st, p,
                       (int)tm, (int)tn);
    return hipGetLastError();
}

template <int MK, int IN, bool LSQ>
hipError_t launch_bwd_out(int out_kind, const BwdParams &p, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_bwd_gemm<MK, IN, OUT_F16, LSQ>(p, st);
        case OUT_BF16: return launch_bwd_gemm<MK, IN, OUT_BF16, LSQ>(p, st);
        default: return launch_bwd_gemm<MK, IN, OUT_F32, LSQ>(p, st);
    }
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

template <int MK>
hipError_t backward_t(const Q4BackwardArgs &a, hipStream_t st) {
    constexpr int IN = MK == MK_F16 ? IN_F16 : IN_BF16;
    const int64_t m = a.m, n = a.n, k = a.k;
    const int64_t mp = (m + 31) / 32 * 32, np = (n + 31) / 32 * 32;
    uint8_t *ws = static_cast<uint8_t *>(a.workspace);
    uint16_t *gt = reinterpret_cast<uint16_t *>(ws);
    ws += round256((size_t)(n * mp) * 2);
    uint16_t *cwt = reinterpret_cast<uint16_t *>(ws);
    ws += round256((size_t)(k * np) * 2);
    uint16_t *cxt = reinterpret_cast<uint16_t *>(ws);
    ws += round256((size_t)(k * mp) * 2);
    double *partials = reinterpret_cast<double *>(ws);
    ws += round256(q4_backward_partials(m, k) * sizeof(double));
    const uint16_t *gp = static_cast<const uint16_t *>(a.grad_out);
    hipError_t e;
    if (n % 32 != 0) {
        uint16_t *pad = reinterpret_cast<uint16_t *>(ws);
        const int64_t blocks = (m * np + kTThreads - 1) / kTThreads;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(bwd_pad_kernel, dim3((unsigned)blocks), dim3(kTThreads), 0, st, gp, m, n, np, pad);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        gp = pad;
    }
    if ((e = launch_transpose<IN, MK, false>(a.grad_out, m, n, mp, nullptr, 0.0f, gt, st)) != hipSuccess) return e;
    if ((e = launch_transpose<IN, MK, true>(a.w, n, k, np, a.scale_w, a.eps, cwt, st)) != hipSuccess) return e;
    if ((e = launch_transpose<IN, MK, true>(a.x, m, k, mp, a.scale_a, a.eps, cxt, st)) != hipSuccess) return e;
    BwdParams px{reinterpret_cast<const int8_t *>(gp), reinterpret_cast<const int8_t *>(cwt), m, k, np * 2,
                 a.x, a.scale_a, a.scale_w, a.eps, a.grad_x, partials};
    if ((e = launch_bwd_out<MK, IN, true>(a.out_kind, px, st)) != hipSuccess) return e;
    BwdParams pw{reinterpret_cast<const int8_t *>(gt), reinterpret_cast<const int8_t *>(cxt), n, k, mp * 2,
                 a.w, a.scale_w, a.scale_a, a.eps, a.grad_w, nullptr};
    if ((e = launch_bwd_out<MK, IN, false>(a.out_kind, pw, st)) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_scale_grad_kernel, dim3(1), dim3(256), 0, st, partials, q4_backward_partials(m, k),
                       a.scale_a, a.eps, a.grad_scale_a);
    return hipGetLastError();
}

}  // namespace

size_t q4_backward_partials(int64_t m, int64_t k) {
    return (size_t)(((m + LB - 1) / LB) * ((k + LB - 1) / LB)) * (kBwdThreads / kWave);
}

size_t q4_backward_workspace(int64_t m, int64_t n, int64_t k) {
    const int64_t mp = (m + 31) / 32 * 32, np = (n + 31) / 32 * 32;
    size_t b = round256((size_t)(n * mp) * 2) + round256((size_t)(k * np) * 2) + round256((size_t)(k * mp) * 2) +
               round256(q4_backward_partials(m, k) * sizeof(double));
    if (n % 32 != 0) b += round256((size_t)(m * np) * 2);
    return b;
}

hipError_t launch_q4_backward(const Q4BackwardArgs &a, hipStream_t st) {
    return a.bf16 ? backward_t<MK_BF16>(a, st) : backward_t<MK_F16>(a, st);
}

}  // namespace ql
