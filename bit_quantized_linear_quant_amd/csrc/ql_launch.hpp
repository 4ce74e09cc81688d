// Internal launchers of libqlinear: one per kernel family.  The C ABI in
// api.hip validates arguments, then calls these; each enqueues its kernels
// on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

// quant.hip
// stream.hip: reads bytes (a multiple of 16) at buf once, XOR into *sink.
hipError_t launch_hbm_read_stream(const void *buf, int64_t bytes, uint64_t *sink, hipStream_t st);

hipError_t launch_quant_act(int in_kind, const void *x, int64_t m, int64_t k, bool rmsnorm,
                            float eps_norm, float eps_q, int8_t *q, float *pts, int32_t *rowsum,
                            hipStream_t st);
hipError_t launch_quant_int4_tensor(int in_kind, const void *x, int64_t count, const float *scale,
                                    float eps, int8_t *q, hipStream_t st);
// quant.hip: 4-bit codes of a [rows, k] tensor as FP6 E3M2 operand tiles
// (rows padded to 32 and k to 128 with zero codes; a4w4_operand_bytes).
size_t a4w4_operand_bytes(int64_t rows, int64_t k);
hipError_t launch_quant_a4w4_tiles(int in_kind, const void *x, int64_t rows, int64_t k, const float *scale,
                                   float eps, uint8_t *tiles, hipStream_t st);
// quant.hip: 4-bit codes of a [rows, k] tensor packed two per byte (code + 8)
// on the same tile grid, 1024 bytes per 32 x 64 tile (a4w4_packed_bytes).
size_t a4w4_packed_bytes(int64_t rows, int64_t k);
hipError_t launch_quant_a4w4_packed(int in_kind, const void *x, int64_t rows, int64_t k, const float *scale,
                                    float eps, uint8_t *tiles, hipStream_t st);

// pack.hip
size_t absmean_partial_count(int64_t count);
hipError_t launch_pack_ternary(const float *w, bool layout_nk, int64_t n, int64_t k, double eps,
                               uint32_t *packed, double *gamma, double *partials, hipStream_t st);
// Capacity of the static scratch of the allocation-free ternary pack, in
// fp64 chunk partials (absmean_partial_count of at most 2^31 weights).
constexpr int64_t kPackScratchPartials = 131072;
// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress; allocates nothing).
hipError_t pack_ternary_scratch(double **partials);
hipError_t launch_pack_int4_weight(const uint8_t *codes, int64_t n, int64_t k, uint32_t *packed,
                                   hipStream_t st);
hipError_t launch_pack_int4_zeros(const uint8_t *z, int64_t n, int64_t groups, uint32_t *packed,
                                  hipStream_t st);

// gemm_i8.hip: int8 x int8 -> int32 tiled MFMA GEMM with a fused epilogue.
enum EpiKind : int { EPI_ROWCOL = 0, EPI_SCALARS = 1 };
struct GemmI8Args {
    const int8_t *x;     // [m, k]
    const int8_t *w;     // [n, k] (nk) or [k, n]
    bool w_nk;
    int epi;             // EpiKind
    const float *pts;    // EPI_ROWCOL: [m]
    const float *deq;    // EPI_ROWCOL: [n]
    const float *sa;     // EPI_SCALARS: device scalar
    const float *sw;     // EPI_SCALARS: device scalar
    float eps;           // EPI_SCALARS: guard of both scalars
    int64_t m, n, k;
    int out_kind;        // OutKind
    void *out;           // [m, n]
    const float *bias;   // [n] added after the dequant, or NULL
    // Independent products over grid z: batch b reads x + b*m*k, w + b*n*k,
    // pts + b*m, deq + b*deq_stride (0: one [n] for every batch) and writes
    // out + b*m*n.  batch 0 is read as 1.
    int64_t batch;
    int64_t deq_stride;
};
hipError_t launch_gemm_i8(const GemmI8Args &a, hipStream_t st);
// 4-bit product on FP6 E3M2 operand tiles (launch_quant_a4w4_tiles):
// out = fl32(fl32(acc * max(*sa, eps)) * max(*sw, eps)), acc exact.
hipError_t launch_gemm_a4w4_tiles(const uint8_t *xa, const uint8_t *wb, const float *sa, const float *sw, float eps,
                                  int64_t m, int64_t n, int64_t k, int out_kind, void *out, hipStream_t st);
// The same product on packed two-per-byte operands (launch_quant_a4w4_packed),
// expanded to FP6 register images on their way into LDS.
hipError_t launch_gemm_a4w4_packed(const uint8_t *xa, const uint8_t *wb, const float *sa, const float *sw, float eps,
                                   int64_t m, int64_t n, int64_t k, int out_kind, void *out, hipStream_t st);
// True when the product runs on the 256 x 256 direct-to-LDS kernel.
bool gemm_i8_uses_big_tiles(bool w_nk, int64_t m, int64_t n, int64_t k, int64_t batch);

// q4_backward.hip: Q4Linear backward (grad_x, grad_w, grad of scale_a).
struct Q4BackwardArgs {
    const void *grad_out;  // [m][n]
    const void *x;         // [m][k]
    const void *w;         // [n][k]; all three fp16, or all three bf16
    bool bf16;
    const float *scale_a, *scale_w;
    float eps;
    int64_t m, n, k;
    int out_kind;          // OUT_F32 / OUT_F16 / OUT_BF16 for grad_x and grad_w
    void *grad_x;          // [m][k]
    void *grad_w;          // [n][k]
    float *grad_scale_a;   // device scalar
    void *workspace;       // q4_backward_workspace(m, n, k) bytes
};
size_t q4_backward_partials(int64_t m, int64_t k);
size_t q4_backward_workspace(int64_t m, int64_t n, int64_t k);
hipError_t launch_q4_backward(const Q4BackwardArgs &a, hipStream_t st);

// gemm_w2a8.hip: packed ternary weights.
hipError_t launch_gemm_w2a8(const int8_t *xq, const float *pts, const int32_t *rowsum,
                            const uint32_t *packed, const double *gamma, const float *bias, int64_t m,
                            int64_t n, int64_t k, int out_kind, void *out, hipStream_t st);

// gemm_int4.hip: grouped affine INT4 with fp16 activations or int8 codes;
// batch independent products laid out back to back (grid z).
hipError_t launch_gemm_int4_grouped(const uint16_t *x, const uint32_t *packed_w,
                                    const uint16_t *scales, const uint32_t *packed_zeros, const float *bias,
                                    int64_t group_size, int64_t m, int64_t n, int64_t k,
                                    int out_kind, void *out, hipStream_t st, int64_t batch = 1);
hipError_t launch_gemm_int4_grouped_i8(const int8_t *xq, const float *pts, const uint32_t *packed_w,
                                       const uint16_t *scales, const uint32_t *packed_zeros, const float *bias,
                                       int64_t group_size, int64_t m, int64_t n, int64_t k, int out_kind, void *out,
                                       hipStream_t st, int64_t batch = 1);

}  // namespace ql
