// int8 x int8 -> int32 tiled GEMM on gfx950 matrix cores, with the dequant
// epilogue fused ("Per-token Quantization for Matmul": Input, Output and
// Example; "Q4LinearFunction" forward for the per-tensor scale pair).
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile as a 2 x 2
// grid of waves, each wave a 64 x 64 sub-tile of 4 x 4
// v_mfma_i32_16x16x64_i8 blocks (64 int32 accumulators per lane).  Each
// 64-byte k-step stages the A (activation rows) and B (weight columns) tiles
// in LDS with k contiguous; rows are padded to 80 bytes so the 16-byte
// fragment reads of 16 consecutive rows fall in distinct bank groups.  The
// next k-step's tiles are prefetched into registers while the matrix cores
// work on the current one.
//
// Weights stored [k][n] (the layout of the worked example) are transposed in
// registers, 4 k x 4 n bytes at a time, on their way into LDS.
// Edge tiles in m, n and k are zero-filled on load and masked on store, so
// any m, n, k >= 1 works; the 16-byte vector loads need k % 16 == 0 (rows of
// [n][k] and [m][k] operands) and fall back to byte loads otherwise.
#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace ql {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kLdsRow = BK + 16;  // padded row stride in bytes
constexpr int kThreads = 256;
constexpr int WM = 64, WN = 64;   // wave sub-tile
constexpr int TM = WM / 16, TN = WN / 16;

struct Params {
    const int8_t *x;
    const int8_t *w;
    const float *pts;
    const float *deq;
    const float *sa;
    const float *sw;
    float eps;
    int64_t m, n, k;
    void *out;
};

// 16 bytes of row `row` of a [rows][k] int8 matrix at column kk, zero-filled
// outside [0, rows) x [0, k).
template <bool VEC>
__device__ __forceinline__ uint4 load_row16(const int8_t *base, int64_t rows, int64_t k, int64_t row,
                                            int64_t kk) {
    if (row >= rows) return make_uint4(0, 0, 0, 0);
    const int8_t *p = base + row * k + kk;
    if (VEC && kk + 16 <= k) return *reinterpret_cast<const uint4 *>(p);
    uint32_t v[4] = {0, 0, 0, 0};
    for (int j = 0; j < 16; j++)
        if (kk + j < k) v[j / 4] |= (uint32_t)(uint8_t)p[j] << (8 * (j % 4));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 4 k-rows x 4 n-columns of a [k][n] int8 matrix, returned as 4 words, one
// per column, each holding the 4 consecutive k of that column.
__device__ __forceinline__ void load_kn_4x4(const int8_t *w, int64_t n, int64_t k, int64_t kk,
                                            int64_t nn, uint32_t col[4]) {
    uint32_t rowv[4];
    const bool full = (nn + 4 <= n) && (kk + 4 <= k) && ((n & 3) == 0);
    if (full) {
#pragma unroll
        for (int i = 0; i < 4; i++) rowv[i] = *reinterpret_cast<const uint32_t *>(w + (kk + i) * n + nn);
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t r = 0;
            for (int j = 0; j < 4; j++)
                if (kk + i < k && nn + j < n) r |= (uint32_t)(uint8_t)w[(kk + i) * n + nn + j] << (8 * j);
            rowv[i] = r;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) c |= ((rowv[i] >> (8 * j)) & 0xffu) << (8 * i);
        col[j] = c;
    }
}

template <bool NK, bool VEC, int EPI, int OUT>
__global__ __launch_bounds__(kThreads) void gemm_i8_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) int8_t As[BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t nk = (p.k + BK - 1) / BK;

    // Register staging of one k-step: A as 2 x 16 bytes, B likewise (NK) or
    // two 4x4 transposed blocks (KN).
    uint4 ra[2];
    uint4 rb[2];
    uint32_t rbt[2][4];

    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / 4, c16 = chunk % 4;
            ra[c] = load_row16<VEC>(p.x, p.m, p.k, m0 + row, k0 + 16 * c16);
            if (NK) {
                rb[c] = load_row16<VEC>(p.w, p.n, p.k, n0 + row, k0 + 16 * c16);
            } else {
                const int n4 = chunk % 32, k4 = chunk / 32;
                load_kn_4x4(p.w, p.n, p.k, k0 + 4 * k4, n0 + 4 * n4, rbt[c]);
            }
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / 4, c16 = chunk % 4;
            *reinterpret_cast<uint4 *>(As + row * kLdsRow + 16 * c16) = ra[c];
            if (NK) {
                *reinterpret_cast<uint4 *>(Bs + row * kLdsRow + 16 * c16) = rb[c];
            } else {
                const int n4 = chunk % 32, k4 = chunk / 32;
#pragma unroll
                for (int j = 0; j < 4; j++)
                    *reinterpret_cast<uint32_t *>(Bs + (4 * n4 + j) * kLdsRow + 4 * k4) = rbt[c][j];
            }
        }
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = v4i{0, 0, 0, 0};

    gload(0);
    sstore();
    __syncthreads();

    const int fr = lane % 16;           // fragment row / column
    const int fk = 16 * (lane / 16);    // fragment k offset (bytes)
    for (int64_t kt = 0; kt < nk; kt++) {
        if (kt + 1 < nk) gload((kt + 1) * BK);
        v4i a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; i++)
            a[i] = *reinterpret_cast<const v4i *>(As + (wm * WM + i * 16 + fr) * kLdsRow + fk);
#pragma unroll
        for (int j = 0; j < TN; j++)
            b[j] = *reinterpret_cast<const v4i *>(Bs + (wn * WN + j * 16 + fr) * kLdsRow + fk);
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int j = 0; j < TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        __syncthreads();
        if (kt + 1 < nk) {
            sstore();
            __syncthreads();
        }
    }

    // Epilogue: lane holds column fr of each 16x16 block and rows 4*(lane/16)+r.
    float s_scalar = 0.0f;
    if (EPI == EPI_SCALARS && OUT != OUT_I32) {
        const float sa = *p.sa, sw = *p.sw;
        const float a1 = sa > p.eps ? sa : p.eps;
        const float w1 = sw > p.eps ? sw : p.eps;
        s_scalar = a1;  // applied as (acc * s'_a) * s'_w
        (void)w1;
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int64_t col = n0 + wn * WN + j * 16 + fr;
        if (col >= p.n) continue;
        float cs = 1.0f;
        if (OUT != OUT_I32) {
            if (EPI == EPI_ROWCOL) cs = p.deq[col];
            else {
                const float sw = *p.sw;
                cs = sw > p.eps ? sw : p.eps;
            }
        }
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane / 16) + r;
                if (row >= p.m) continue;
                const int32_t v = acc[i][j][r];
                const int64_t idx = row * p.n + col;
                if (OUT == OUT_I32) {
                    static_cast<int32_t *>(p.out)[idx] = v;
                } else {
                    const float rs = EPI == EPI_ROWCOL ? p.pts[row] : s_scalar;
                    const float y = __fmul_rn(__fmul_rn((float)v, rs), cs);
                    store_out<OUT>(p.out, idx, y);
                }
            }
        }
    }
}

template <bool NK, bool VEC, int EPI, int OUT>
hipError_t launch_t(const Params &p, hipStream_t st) {
    dim3 grid((unsigned)((p.n + BN - 1) / BN), (unsigned)((p.m + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_i8_kernel<NK, VEC, EPI, OUT>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <bool NK, bool VEC, int EPI>
hipError_t launch_out(int out_kind, const Params &p, hipStream_t st) {
    switch (out_kind) {
        case OUT_F16: return launch_t<NK, VEC, EPI, OUT_F16>(p, st);
        case OUT_BF16: return launch_t<NK, VEC, EPI, OUT_BF16>(p, st);
        default: return launch_t<NK, VEC, EPI, OUT_I32>(p, st);
    }
}

template <bool NK, bool VEC>
hipError_t launch_epi(int epi, int out_kind, const Params &p, hipStream_t st) {
    return epi == EPI_ROWCOL ? launch_out<NK, VEC, EPI_ROWCOL>(out_kind, p, st)
                             : launch_out<NK, VEC, EPI_SCALARS>(out_kind, p, st);
}

}  // namespace

hipError_t launch_gemm_i8(const GemmI8Args &a, hipStream_t st) {
    Params p{a.x, a.w, a.pts, a.deq, a.sa, a.sw, a.eps, a.m, a.n, a.k, a.out};
    if (a.m > (int64_t)BM * 65535) return hipErrorInvalidValue;
    const bool vec = (a.k % 16) == 0;
    if (a.w_nk)
        return vec ? launch_epi<true, true>(a.epi, a.out_kind, p, st)
                   : launch_epi<true, false>(a.epi, a.out_kind, p, st);
    return vec ? launch_epi<false, true>(a.epi, a.out_kind, p, st)
               : launch_epi<false, false>(a.epi, a.out_kind, p, st);
}

}  // namespace ql
