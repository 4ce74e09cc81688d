/*
 * qlinear.h - C ABI of the MI355X (gfx950) quantized linear layer library
 * (libqlinear.so).
 *
 * The layer: activations quantized per token to int8 (absmax, optionally
 * after a parameter-free RMSNorm), weights that are ternary (absmean),
 * int8, 4-bit grouped affine, or 4-bit per-tensor, and an integer-
 * accumulated product with a dequant epilogue
 *     out[m][n] = acc[m][n] * perTokenScale[m] * deqScale[n].
 *
 * Sources (web pages, cited by title and section):
 *   [Q4] bitorch-engine API docs, "Q4LinearFunction": forward.
 *   [BL] LLaMA-BitNet utils.py, "Class BitLinear": forward docstring steps
 *        1-5 and the forward body.
 *   [PT] Ascend CANN ATB docs, "Per-token Quantization for Matmul":
 *        Parameters, Input, Output, Example.
 *   [CA] frankenstein-transformer docs, "Common Attention Utilities":
 *        activation_quant, weight_quant, BitLinear.forward and
 *        bake_ternary_weights.
 *   [L4] docs.rs vyre-libs 0.7.2, "linear_4bit/mod.rs": module doc comment,
 *        QuantizedLinear4BitSpec, QuantizedLinear4BitPlannerEvidence.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, owned and allocated by the caller.
 *     The library never allocates, frees or synchronizes; it keeps no mutable
 *     global state and may be called from several threads.
 *   - Matrices are dense row-major.  Leading dimensions of a "(..., k)"
 *     activation are flattened into m by the caller ([CA] BitLinear.forward
 *     takes shape (..., in_features)).
 *   - Every tensor pointer must be 16-byte aligned ([PT] Input asks 32 bytes
 *     for deqScale; 32 is recommended, 16 is required).
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued asynchronously: a kernel fault surfaces at the
 *     caller's next synchronization, not as a return code.
 *   - Arguments are validated on the host before any launch.  An invalid
 *     call returns a negative ql_status and enqueues nothing.  A launch
 *     failure returns QL_ERR_HIP.  No C++ exception crosses the boundary.
 *   - NaN or Inf inputs give unspecified (but memory-safe) outputs.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QL_ABI_VERSION 8
/* Version of the 2-bit ternary weight layout written by qlinear_pack_ternary. */
#define QL_TERNARY_PACK_V1 1
/* Version of the 4-bit weight layout written by qlinear_pack_int4. */
#define QL_INT4_PACK_V1 1

typedef enum ql_status {
    QL_OK = 0,
    QL_ERR_NULL = -1,        /* a required pointer is NULL */
    QL_ERR_SHAPE = -2,       /* a size is out of range or breaks a divisibility rule */
    QL_ERR_DTYPE = -3,       /* a dtype this entry point does not accept */
    QL_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    QL_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than qlinear_workspace_bytes */
    QL_ERR_UNSUPPORTED = -6, /* a valid but not implemented combination */
    QL_ERR_HIP = -7,         /* the HIP runtime reported an error */
    /* Range markers, never returned: they make every enum of this header span
     * all 32-bit values, so any int a C caller passes is a valid value. */
    QL_STATUS_MIN_ENUM = -0x7fffffff - 1,
    QL_STATUS_MAX_ENUM = 0x7fffffff
} ql_status;

/* Element types.  QL_I32 as an output dtype exposes the raw int32
 * accumulator; QL_F32 exposes the fp32 value before the final rounding. */
typedef enum ql_dtype {
    QL_F32 = 0,
    QL_F16 = 1,
    QL_BF16 = 2,
    QL_I8 = 3,
    QL_U8 = 4,
    QL_I32 = 5,
    QL_DTYPE_MIN_ENUM = -0x7fffffff - 1,
    QL_DTYPE_MAX_ENUM = 0x7fffffff
} ql_dtype;

/* Weight layouts: [PT] Input gives weight [k, n]; [PT] Parameters
 * transposeB=true, and the nn.Linear weight of [BL], give [n, k]. */
typedef enum ql_wlayout {
    QL_W_KN = 0,
    QL_W_NK = 1,
    QL_WLAYOUT_MIN_ENUM = -0x7fffffff - 1,
    QL_WLAYOUT_MAX_ENUM = 0x7fffffff
} ql_wlayout;

/* Flags of qlinear_quant_act. */
#define QL_RMSNORM 1u

/* What qlinear_pack_int4 packs. */
typedef enum ql_int4_what {
    QL_INT4_WEIGHT = 0,
    QL_INT4_ZEROS = 1,
    QL_INT4_WHAT_MIN_ENUM = -0x7fffffff - 1,
    QL_INT4_WHAT_MAX_ENUM = 0x7fffffff
} ql_int4_what;

/* Operations that take a workspace (qlinear_workspace_bytes). */
typedef enum ql_op {
    QL_OP_PACK_TERNARY = 0,
    QL_OP_GEMM_A4W4 = 1,
    QL_OP_A4W4_OPERAND = 2,
    QL_OP_Q4_BACKWARD = 3,
    QL_OP_A4W4_PACKED = 4,
    QL_OP_MIN_ENUM = -0x7fffffff - 1,
    QL_OP_MAX_ENUM = 0x7fffffff
} ql_op;

/* Returns QL_ABI_VERSION of the built library. */
int qlinear_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *qlinear_status_string(ql_status s);

/* Bytes of workspace the operation needs for these sizes (0 if none).
 *   QL_OP_PACK_TERNARY: fp64 partial sums of the absmean; m is ignored.
 *   QL_OP_GEMM_A4W4:    the FP6 operand tiles of x [m,k] then of w [n,k]
 *                       (QL_OP_A4W4_OPERAND of each, rounded up to 256 bytes).
 *   QL_OP_A4W4_OPERAND: bytes of one FP6 operand of m rows and k columns:
 *                       roundup(m, 32) * roundup(k, 128) * 3 / 4; n is ignored.
 *   QL_OP_A4W4_PACKED:  bytes of one two-codes-per-byte operand of m rows and
 *                       k columns: roundup(m, 32) * roundup(k, 128) / 2.
 *   QL_OP_Q4_BACKWARD:  the transposed, zero-padded 16-bit operands of the
 *                       two backward products and the scale-gradient
 *                       partials of qlinear_q4_backward. */
size_t qlinear_workspace_bytes(ql_op op, int64_t m, int64_t n, int64_t k);

/*
 * Per-token int8 activation quantization.
 * [BL] forward steps 1-2 (parameter-free RMSNorm, then 8-bit per-token
 * quantization) and step 5; [CA] activation_quant (the last dimension is
 * scaled into [-128, 127] per token, rounded, and rescaled).
 *
 *   x       [m, k] QL_BF16, QL_F16 or QL_F32.
 *   flags   0 or QL_RMSNORM.
 *   r       = 1/sqrt(mean(x^2) + eps_norm) with QL_RMSNORM (fp32), else 1.
 *   q       [m, k] int8 out: clamp(rne(fl32(x * fl32(127 / a'))), -128, 127),
 *           a' = max(max_k |x|, eps_q / r): the guard applies to the absmax of
 *           the normalized row r x, which the quantizer sees.  Where
 *           r max|x| >= eps_q the codes do not depend on the RMSNorm (it
 *           multiplies the row by r > 0 and absmax codes are invariant).
 *   per_token_scale [m] fp32 out: a' * r / 127 (without RMSNorm correctly
 *           rounded; with it, from the fp32 r).
 *   rowsum  [m] int32 out, may be NULL: sum_k q[m, k].
 * 1 <= m < 2^31, 1 <= k <= 16909320 (the code sum must fit int32); eps_q a
 * positive finite number, eps_norm a finite number >= 0.
 * Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_UNSUPPORTED (flags or eps),
 * QL_ERR_DTYPE, QL_ERR_ALIGN.
 */
ql_status qlinear_quant_act(const void *x, ql_dtype x_dtype, int64_t m, int64_t k,
                            uint32_t flags, float eps_norm, float eps_q,
                            int8_t *q, float *per_token_scale, int32_t *rowsum,
                            void *stream);

/*
 * Per-tensor 4-bit quantization of [Q4] forward (activations and weights
 * both become 4-bit codes under their given scale; eps keeps the divisor
 * away from zero):  q = clamp(rne(fl32(x / max(*scale, eps))), -8, 7),
 * stored in int8.
 *   x      [count] QL_F16, QL_BF16 or QL_F32.
 *   scale  device fp32 scalar.
 * count >= 1.  Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_DTYPE, QL_ERR_ALIGN.
 */
ql_status qlinear_quant_int4_tensor(const void *x, ql_dtype x_dtype, int64_t count,
                                    const float *scale, float eps, int8_t *q,
                                    void *stream);

/*
 * Absmean ternary weight quantization and 2-bit pack (one-time, like
 * [CA] bake_ternary_weights).  [BL] forward step 3; [CA] weight_quant.
 *   w       fp32, [n, k] for QL_W_NK or [k, n] for QL_W_KN.
 *   gamma'  = max(sum|w| / (n*k), eps), summed in fp64 with a fixed order.
 *   code    = sign(w) if |w| > gamma'/2 else 0  (= clamp(rne(w/gamma'), -1, 1)).
 *   packed  [n*k/16] u32 out, layout QL_TERNARY_PACK_V1:
 *           blocks of 16 columns x 256 k, block (nb, kb) = 256 words from
 *           word (nb*(k/256) + kb)*256; word 4l+t (l < 64, t < 4) holds column
 *           16nb + l%16 and the 16 k from k0 = 256kb + 64(l/16) + 16t; element
 *           k0 + 4a + b is at bits [8b+2a, 8b+2a+1] as code+1 in {0, 1, 2}.
 *   gamma   device fp64 scalar out: gamma'.
 *   workspace >= qlinear_workspace_bytes(QL_OP_PACK_TERNARY, 0, n, k).
 * n % 16 == 0, k % 256 == 0.  Deterministic: the same input gives the same
 * gamma' and words on every call.
 */
ql_status qlinear_pack_ternary(const float *w, ql_wlayout layout, int64_t n, int64_t k,
                               double eps, uint32_t *packed, double *gamma,
                               void *workspace, size_t ws_bytes, void *stream);

/*
 * qlinear_pack_ternary with no workspace argument and no device allocation,
 * for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The absmean's fp64 chunk
 * partials go to a static device array inside the library (1 MiB per GPU,
 * held until the process ends), so n * k <= 2^31.  Same kernels, same
 * gamma' and words as qlinear_pack_ternary.  The caller still owns w,
 * packed and gamma.  All calls on one GPU share that array: calls that
 * overlap on one GPU (different streams, or threads without ordering) race,
 * and the caller must order them.  The device current at the call must be
 * the stream's device.
 * Errors: as qlinear_pack_ternary; QL_ERR_WORKSPACE when n * k > 2^31 (the
 * static array's capacity); QL_ERR_HIP when the array's address cannot be
 * obtained.
 */
ql_status qlinear_pack_ternary_noalloc(const float *w, ql_wlayout layout, int64_t n, int64_t k,
                                       double eps, uint32_t *packed, double *gamma,
                                       void *stream);

/*
 * 4-bit pack ([L4] module doc: eight nibbles per u32 word).  Only the low
 * nibble of each input byte is used.
 *   QL_INT4_WEIGHT: codes [rows=n, cols=k] -> packed [n*k/8] u32, layout
 *       QL_INT4_PACK_V1: blocks of 16 columns x 128 k, block (nb, kb) = 256
 *       words from word (nb*(k/128) + kb)*256; word 4l+t holds column
 *       16nb + l%16 and the 8 k from k0 = 128kb + 32(l/16) + 8t; nibble p
 *       holds k-offset 2p for p < 4 and 2(p-4)+1 for p >= 4.
 *       Requires n % 16 == 0, k % 128 == 0.
 *   QL_INT4_ZEROS: zero-points [rows=n, cols=groups] -> packed [groups][n/8]
 *       u32, column c in nibble c % 8.  Requires n % 8 == 0.
 */
ql_status qlinear_pack_int4(const uint8_t *codes, int64_t rows, int64_t cols,
                            ql_int4_what what, uint32_t *packed, void *stream);

/*
 * QL_BIAS - the optional bias of the three GEMM entry points below.
 * [PT] Parameters lists hasBias (accepted value: false only), [BL] forward
 * hands its (normally absent) bias to the linear call, and [L4]
 * QuantizedLinear4BitPlannerEvidence counts bias bytes.  These entry points
 * take the ordinary linear-layer meaning y = dequant(acc) + b: bias [n] fp32,
 * added once in fp32 to the dequantized fp32 value, before the rounding to
 * the output type.  NULL means no bias and gives exactly the bias-free
 * result.  (Read literally, [BL] forward would add the bias before the
 * rescale and so scale it by both quantization scales; that reading is not
 * taken.)
 */

/*
 * Per-token W8A8 linear ([PT] Input, Parameters, Output, Example):
 *   out[m][n] = (sum_k x[m][k] * w[k][n]) * per_token_scale[m] * deq_scale[n]
 * computed as an exact int32 accumulation, then fl32(fl32(acc * pts) * deq),
 * rounded to nearest even in the output type.
 *   x [m, k] int8; w [k, n] (QL_W_KN) or [n, k] (QL_W_NK) int8;
 *   deq_scale [n] fp32; per_token_scale [m] fp32;
 *   out [m, n] QL_F16 / QL_BF16, or QL_I32 for the raw accumulator (the
 *   scale pointers may then be NULL).
 *   bias [n] fp32 or NULL: when given, out = fl32(dequantized value + bias[n])
 *   before the output rounding (see QL_BIAS below); QL_I32 with a bias is
 *   QL_ERR_UNSUPPORTED.
 * m, n, k >= 1 (any sizes; edge tiles are masked); k <= 131071 so the int32
 * accumulator cannot overflow.
 */
ql_status qlinear_gemm_w8a8(const int8_t *x, const int8_t *w, ql_wlayout layout,
                            const float *deq_scale, const float *per_token_scale,
                            const float *bias, int64_t m, int64_t n, int64_t k,
                            ql_dtype out_dtype, void *out, void *stream);

/*
 * Batched per-token W8A8 linear ([PT] Input and Output: x [batch,m,k],
 * weight [batch,k,n], output [batch,m,n]): `batch` independent products,
 * each exactly qlinear_gemm_w8a8 on its own slice:
 *   out[b] = qlinear_gemm_w8a8(x[b], w[b], deq_scale + b*deq_batch_stride,
 *                              per_token_scale + b*m, bias)
 *   x [batch, m, k] int8; w [batch, k, n] (QL_W_KN) or [batch, n, k] (QL_W_NK);
 *   per_token_scale [batch, m] fp32 (one per token row);
 *   deq_scale fp32 [n] shared by every batch (deq_batch_stride 0, [PT] Input
 *   gives deqScale as [n]) or [batch, n] (deq_batch_stride n); other strides
 *   are QL_ERR_SHAPE;
 *   bias [n] fp32 or NULL, shared by every batch (QL_BIAS);
 *   out [batch, m, n] QL_F16 / QL_BF16 / QL_I32.
 * 1 <= batch <= 65535; m, n, k as for qlinear_gemm_w8a8.  One launch covers
 * every batch.
 */
ql_status qlinear_gemm_w8a8_batched(const int8_t *x, const int8_t *w, ql_wlayout layout,
                                    const float *deq_scale, int64_t deq_batch_stride,
                                    const float *per_token_scale, const float *bias,
                                    int64_t batch, int64_t m, int64_t n, int64_t k,
                                    ql_dtype out_dtype, void *out, void *stream);

/*
 * BitLinear product on packed ternary weights ([BL] forward steps 4-5):
 *   acc[m][n] = sum_k xq[m][k] * code[n][k]
 *   out[m][n] = fl32(fl32(acc * per_token_scale[m]) * fp32(*gamma))
 *   xq [m, k] int8 codes and rowsum [m] from qlinear_quant_act;
 *   packed / gamma from qlinear_pack_ternary;
 *   out [m, n] QL_BF16 / QL_F16, or QL_I32 for acc.
 *   bias [n] fp32 or NULL, added as in qlinear_gemm_w8a8 (QL_BIAS below);
 *   QL_I32 with a bias is QL_ERR_UNSUPPORTED.
 * The kernel multiplies by code+1 in {0, 1, 2} and subtracts rowsum.
 * m <= 64 takes the split-k decode kernel (as do 64 < m <= 128 at k >= 2048,
 * within column limits), larger m the tiled GEMM kernels.
 * n % 16 == 0, k % 256 == 0, k <= 131071.
 */
ql_status qlinear_gemm_w2a8(const int8_t *xq, const float *per_token_scale,
                            const int32_t *rowsum, const uint32_t *packed,
                            const double *gamma, const float *bias, int64_t m, int64_t n,
                            int64_t k, ql_dtype out_dtype, void *out, void *stream);

/*
 * Grouped affine INT4 linear ([L4] module doc: the packed u32 weight is
 * unpacked inside the k loop with its per-group scale and zero-point; no
 * dequantized weight buffer is written).  Two activation kinds:
 *   x_dtype QL_F16: x [m, k] fp16 activations,
 *     out[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g]);
 *     (q - z) is formed exactly in fp16, products accumulate in fp32 per
 *     128-k block (group_size a multiple of 128) or per 32-k step (other
 *     group sizes) and each partial sum is scaled once by its group's scale.
 *     per_token_scale is ignored.  out QL_F16, or QL_F32 for the value before
 *     rounding.
 *   x_dtype QL_I8: x [m, k] int8 activation codes with per_token_scale [m]
 *     fp32 (qlinear_quant_act; [BL] steps 2 and 5),
 *     out[m][n] = pts[m] * sum_g s[n][g] * sum_{k in g} xq[m][k] * (q[n][k] - z[n][g]);
 *     each 128-k block's (or, for group sizes that are not multiples of
 *     128, each 32-k step's) integer sum is exact (int32), scaled by s in
 *     fp32; pts multiplies the final sum.  out QL_F16, QL_BF16 or QL_F32.
 *   packed_w from qlinear_pack_int4(QL_INT4_WEIGHT);
 *   scales [n, k/group_size] fp16 (row-major, one per column and group);
 *   packed_zeros from qlinear_pack_int4(QL_INT4_ZEROS) of z [n, groups];
 *   bias [n] fp32 or NULL, added to the fp32 value before the output
 *   rounding (QL_BIAS below).
 * n % 16 == 0, k % 128 == 0, group_size >= 32, group_size % 32 == 0 (one
 * matrix-core step, so no step straddles two groups), k % group_size == 0,
 * n, k < 2^31.  Errors: QL_ERR_NULL, QL_ERR_SHAPE, QL_ERR_DTYPE, QL_ERR_ALIGN.
 */
ql_status qlinear_gemm_w4a8_grouped(const void *x, ql_dtype x_dtype,
                                    const float *per_token_scale,
                                    const uint32_t *packed_w, const uint16_t *scales,
                                    const uint32_t *packed_zeros, int64_t group_size,
                                    int64_t m, int64_t n, int64_t k, const float *bias,
                                    ql_dtype out_dtype, void *out, void *stream);

/*
 * Batched grouped affine INT4 linear ([L4] lists a batched form of the grouped
 * linear among the module's exports, by name only; read here as batch
 * independent products of qlinear_gemm_w4a8_grouped, one per slice):
 *   for b in [0, batch): the qlinear_gemm_w4a8_grouped product of
 *     x + b*m*k elements ([batch, m, k]), per_token_scale + b*m (QL_I8),
 *     packed_w + b*n*k/8 words, scales + b*n*(k/group_size),
 *     packed_zeros + b*(k/group_size)*n/8 words, bias + b*n (if not NULL),
 *     written to out + b*m*n elements ([batch, m, n]).
 * Every slice holds its own weights; the argument rules are those of
 * qlinear_gemm_w4a8_grouped, plus 1 <= batch <= 65535 (else QL_ERR_SHAPE).
 * Each slice's result equals a separate qlinear_gemm_w4a8_grouped call on
 * that slice, bit for bit.
 */
ql_status qlinear_gemm_w4a8_grouped_batched(int64_t batch, const void *x, ql_dtype x_dtype,
                                            const float *per_token_scale,
                                            const uint32_t *packed_w, const uint16_t *scales,
                                            const uint32_t *packed_zeros, int64_t group_size,
                                            int64_t m, int64_t n, int64_t k, const float *bias,
                                            ql_dtype out_dtype, void *out, void *stream);

/*
 * A4W4 product on 4-bit codes held in int8 ([Q4] forward, second half):
 *   out[m][n] = fl32(fl32(acc * s'_a) * s'_w),  acc = sum_k xq[m][k] * wq[n][k],
 *   s'_a = max(*scale_a, eps), s'_w = max(*scale_w, eps) (device fp32 scalars).
 *   xq [m, k], wq [n, k] int8 (codes in [-8, 7] from qlinear_quant_int4_tensor;
 *   any int8 values are multiplied exactly); out QL_F16 / QL_BF16 / QL_I32.
 * m, n, k >= 1; k <= 131071.
 */
ql_status qlinear_gemm_a4w4_codes(const int8_t *xq, const int8_t *wq,
                                  const float *scale_a, const float *scale_w, float eps,
                                  int64_t m, int64_t n, int64_t k, ql_dtype out_dtype,
                                  void *out, void *stream);

/*
 * QL_A4W4_OPERAND - the packed operand of the 4-bit product (this library's
 * own layout, not one of the pages').  Each 4-bit code c in [-8, 7] is stored
 * as the FP6 E3M2 number of value c (OCP Microscaling Formats v1.0: sign,
 * 3 exponent bits with bias 3, 2 mantissa bits; all 16 codes are exact), 6
 * bits per element, laid out as the register images the gfx950 32x32x64 FP6
 * matrix-core product reads.  A [rows, k] operand is padded with zero codes
 * to rows_p = roundup(rows, 32) and k_p = roundup(k, 128) and holds
 * (rows_p / 32) * (k_p / 64) tiles of 1536 bytes; tile (rb, ks) sits at byte
 * (rb * k_p/64 + ks) * 1536.  Slot l (0..63) of a tile is row 32rb + l%32,
 * k = 64ks + 32(l/32) + j for j = 0..31, as a 192-bit little-endian string
 * with element j in bits 6j..6j+5; its first 16 bytes are at tile byte 16l
 * and its last 8 at tile byte 1024 + 8l.  Size:
 * qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, rows, 0, k).
 */

/*
 * Per-tensor 4-bit quantization of x [rows, k] ([Q4] forward, first half)
 * straight into a QL_A4W4_OPERAND: the codes are those of
 * qlinear_quant_int4_tensor, clamp(rne(fl32(x / max(*scale, eps))), -8, 7).
 * x_dtype QL_F16 / QL_BF16 / QL_F32; k <= 131071.  A weight can be
 * quantized once and its operand reused by every later product.
 */
ql_status qlinear_quant_a4w4_operand(const void *x, ql_dtype x_dtype, int64_t rows, int64_t k,
                                     const float *scale, float eps, void *operand, void *stream);

/*
 * A4W4 product on two QL_A4W4_OPERANDs ([Q4] forward, second half):
 *   out[m][n] = fl32(fl32(acc * s'_a) * s'_w),  acc = sum_k xq[m][k] * wq[n][k],
 *   s'_a = max(*scale_a, eps), s'_w = max(*scale_w, eps) (device fp32 scalars)
 * with xa the operand of x [m, k] and wb that of w [n, k].  acc is exact (an
 * integer below 2^23 accumulated in fp32), so the result equals
 * qlinear_gemm_a4w4_codes on the same codes bit for bit.  out QL_F16 /
 * QL_BF16 / QL_I32 (acc; the scale pointers may then be NULL).
 * m, n, k >= 1; k <= 131071.
 */
ql_status qlinear_gemm_a4w4_operands(const void *xa, const void *wb, const float *scale_a,
                                     const float *scale_w, float eps, int64_t m, int64_t n,
                                     int64_t k, ql_dtype out_dtype, void *out, void *stream);

/*
 * QL_A4W4_PACKED - the 4-bit operand at two codes per byte (0.5 byte per
 * code; this library's own layout).  The tile grid of QL_A4W4_OPERAND, but a
 * tile is 1024 bytes at byte (rb * k_p/64 + ks) * 1024 and slot l is the 16
 * bytes at tile byte 16l (row 32rb + l%32, k 64ks + 32(l/32) + j, j = 0..31).
 * Element j is in the little-endian 32-bit word j/8 of the slot, in nibble
 * (j%8)/2 for even j%8 and 4 + (j%8)/2 for odd, stored as c + 8 in [0, 15].
 * Size: qlinear_workspace_bytes(QL_OP_A4W4_PACKED, rows, 0, k)
 * = roundup(rows, 32) * roundup(k, 128) / 2.
 */

/*
 * As qlinear_quant_a4w4_operand, writing a QL_A4W4_PACKED operand: the same
 * codes, two per byte.
 */
ql_status qlinear_quant_a4w4_packed(const void *x, ql_dtype x_dtype, int64_t rows, int64_t k,
                                    const float *scale, float eps, void *operand, void *stream);

/*
 * As qlinear_gemm_a4w4_operands on two QL_A4W4_PACKED operands: each slot is
 * expanded to its FP6 E3M2 register image on its way from HBM into LDS, then
 * multiplied on the FP6 matrix cores.  Same acc, same outputs bit for bit.
 */
ql_status qlinear_gemm_a4w4_packed(const void *xa, const void *wb, const float *scale_a,
                                   const float *scale_w, float eps, int64_t m, int64_t n,
                                   int64_t k, ql_dtype out_dtype, void *out, void *stream);

/*
 * Q4Linear forward ([Q4] forward): quantizes x [m, k] and w [n, k] (both
 * in_dtype: QL_F16, QL_BF16 or QL_F32) per tensor to 4 bits with
 * qlinear_quant_a4w4_operand into the workspace (x's operand at offset 0,
 * w's at offset roundup(QL_OP_A4W4_OPERAND bytes of x, 256)), then runs
 * qlinear_gemm_a4w4_operands.
 * workspace >= qlinear_workspace_bytes(QL_OP_GEMM_A4W4, m, n, k); on return
 * it holds the two operands.
 */
ql_status qlinear_gemm_a4w4(const void *x, const void *w, ql_dtype in_dtype,
                            const float *scale_a, const float *scale_w, float eps,
                            int64_t m, int64_t n, int64_t k, ql_dtype out_dtype, void *out,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * Q4Linear backward ([Q4] backward): gradients for the input, the weight
 * and the activation scale from the output gradient, adjusted to the
 * quantization range; scale_w and eps get none.  The page gives it only in
 * words; this is the straight-through reading, with v = fl32(t / s') the
 * quotient the forward code rounds and q its 4-bit code:
 *   dXh = G (s'_w q_w),  dWh = G^T (s'_a q_a)     (fp32 accumulation)
 *   grad_x = dXh where -8 <= v_a <= 7, else 0
 *   grad_w = dWh where -8 <= v_w <= 7, else 0
 *   *grad_scale_a = sum dXh * (q_a - v_a if inside the range, q_a outside),
 *                   0 when *scale_a <= eps  (learned step-size term)
 *   grad_out G [m, n], x [m, k], w [n, k]: all dtype QL_F16 or all QL_BF16
 *   (the products run on the fp16 or bf16 matrix cores; the codes are exact
 *   in both); scale_a, scale_w device fp32 scalars of the forward;
 *   grad_x [m, k] and grad_w [n, k] of grad_dtype QL_F32 / QL_F16 / QL_BF16;
 *   grad_scale_a a device fp32 scalar, summed in a fixed order
 *   (deterministic).
 * workspace >= qlinear_workspace_bytes(QL_OP_Q4_BACKWARD, m, n, k).
 * m, n, k >= 1.
 */
ql_status qlinear_q4_backward(const void *grad_out, const void *x, const void *w, ql_dtype dtype,
                              const float *scale_a, const float *scale_w, float eps,
                              int64_t m, int64_t n, int64_t k, ql_dtype grad_dtype,
                              void *grad_x, void *grad_w, float *grad_scale_a,
                              void *workspace, size_t ws_bytes, void *stream);

/* Words of the sink array of qlinear_hbm_read_stream. */
#define QL_HBM_STREAM_SINK_WORDS 16384

/*
 * Measurement aid (no page defines it): reads the `bytes` bytes at `buf`
 * once with 16-byte non-temporal loads spread over the whole device.  Each
 * wave XORs the 32-bit words it read into its own word of `sink`, a device
 * array of QL_HBM_STREAM_SINK_WORDS uint64 that the call does not clear;
 * the XOR of the whole array then changes by the XOR of every word of the
 * buffer.  Its time is the ceiling of any kernel that must stream as many
 * bytes from HBM once, such as the decode product's packed weight, measured
 * with the same load form.  buf and sink are device memory, 16-byte
 * aligned; bytes is a positive multiple of 16 (QL_ERR_SHAPE otherwise).
 * Asynchronous on `stream`; calls that overlap on one sink race on its
 * words.
 */
ql_status qlinear_hbm_read_stream(const void *buf, size_t bytes, uint64_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
