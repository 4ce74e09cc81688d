// C ABI of libqlinear (declared in include/qlinear.h): host-side argument
// validation, shape dispatch and launches on the caller's stream.  Nothing
// here allocates, frees or synchronizes; validation runs before any HIP call
// so an invalid call enqueues nothing.
#include "qlinear.h"

#include <hip/hip_runtime.h>

#include "ql_device.hpp"
#include "ql_launch.hpp"

namespace {

constexpr int64_t kMaxK = 131071;  // (-128)^2 * k must fit int32
// Longest row quant_act accepts: the int32 code sum of a row, at most 127 k
// in magnitude, must fit int32.
constexpr int64_t kMaxQuantK = 16909320;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ql_status hip_status(hipError_t e) { return e == hipSuccess ? QL_OK : QL_ERR_HIP; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

int in_kind(ql_dtype d) {
    switch (d) {
        case QL_F32: return ql::IN_F32;
        case QL_F16: return ql::IN_F16;
        case QL_BF16: return ql::IN_BF16;
        default: return -1;
    }
}

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int qlinear_abi_version(void) { return QL_ABI_VERSION; }

const char *qlinear_status_string(ql_status s) {
    switch (s) {
        case QL_OK: return "ok";
        case QL_ERR_NULL: return "a required pointer is NULL";
        case QL_ERR_SHAPE: return "invalid shape";
        case QL_ERR_DTYPE: return "unsupported dtype";
        case QL_ERR_ALIGN: return "pointer not 16-byte aligned";
        case QL_ERR_WORKSPACE: return "workspace missing or too small";
        case QL_ERR_UNSUPPORTED: return "unsupported combination";
        case QL_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

size_t qlinear_workspace_bytes(ql_op op, int64_t m, int64_t n, int64_t k) {
    if (n < 0 || k < 0 || m < 0) return 0;
    switch (op) {
        case QL_OP_PACK_TERNARY:
            return round256(ql::absmean_partial_count(n * k) * sizeof(double));
        case QL_OP_GEMM_A4W4:
            return round256(ql::a4w4_operand_bytes(m, k)) + round256(ql::a4w4_operand_bytes(n, k));
        case QL_OP_A4W4_OPERAND:
            return ql::a4w4_operand_bytes(m, k);
        case QL_OP_A4W4_PACKED:
            return ql::a4w4_packed_bytes(m, k);
        case QL_OP_Q4_BACKWARD:
            return ql::q4_backward_workspace(m, n, k);
        default: return 0;
    }
}

ql_status qlinear_quant_act(const void *x, ql_dtype x_dtype, int64_t m, int64_t k, uint32_t flags,
                            float eps_norm, float eps_q, int8_t *q, float *per_token_scale,
                            int32_t *rowsum, void *stream) {
    if (!x || !q || !per_token_scale) return QL_ERR_NULL;
    if (m < 1 || k < 1 || m > 0x7fffffff || k > kMaxQuantK) return QL_ERR_SHAPE;
    if ((flags & ~QL_RMSNORM) != 0) return QL_ERR_UNSUPPORTED;
    // eps_q guards a division and must be a positive number; eps_norm must
    // not be negative (NaN fails both comparisons).
    if (!(eps_q > 0.0f) || !(eps_q <= 3.4e38f) || !(eps_norm >= 0.0f) || !(eps_norm <= 3.4e38f))
        return QL_ERR_UNSUPPORTED;
    const int kind = in_kind(x_dtype);
    if (kind < 0) return QL_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(q) || !aligned16(per_token_scale) || (rowsum && !aligned16(rowsum)))
        return QL_ERR_ALIGN;
    return hip_status(ql::launch_quant_act(kind, x, m, k, (flags & QL_RMSNORM) != 0, eps_norm, eps_q, q,
                                           per_token_scale, rowsum, as_stream(stream)));
}

ql_status qlinear_quant_int4_tensor(const void *x, ql_dtype x_dtype, int64_t count, const float *scale,
                                    float eps, int8_t *q, void *stream) {
    if (!x || !scale || !q) return QL_ERR_NULL;
    if (count < 1) return QL_ERR_SHAPE;
    const int kind = in_kind(x_dtype);
    if (kind < 0) return QL_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(q)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_quant_int4_tensor(kind, x, count, scale, eps, q, as_stream(stream)));
}

ql_status qlinear_pack_ternary(const float *w, ql_wlayout layout, int64_t n, int64_t k, double eps,
                               uint32_t *packed, double *gamma, void *workspace, size_t ws_bytes,
                               void *stream) {
    if (!w || !packed || !gamma) return QL_ERR_NULL;
    if (layout != QL_W_KN && layout != QL_W_NK) return QL_ERR_UNSUPPORTED;
    if (n < 16 || k < 256 || n % 16 || k % 256) return QL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(gamma)) return QL_ERR_ALIGN;
    if (!workspace || ws_bytes < qlinear_workspace_bytes(QL_OP_PACK_TERNARY, 0, n, k)) return QL_ERR_WORKSPACE;
    if (!aligned16(workspace)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_pack_ternary(w, layout == QL_W_NK, n, k, eps, packed, gamma,
                                              static_cast<double *>(workspace), as_stream(stream)));
}

ql_status qlinear_pack_ternary_noalloc(const float *w, ql_wlayout layout, int64_t n, int64_t k, double eps,
                                       uint32_t *packed, double *gamma, void *stream) {
    if (!w || !packed || !gamma) return QL_ERR_NULL;
    if (layout != QL_W_KN && layout != QL_W_NK) return QL_ERR_UNSUPPORTED;
    if (n < 16 || k < 256 || n % 16 || k % 256) return QL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(packed) || !aligned16(gamma)) return QL_ERR_ALIGN;
    // The absmean partials must fit the library's static scratch.
    if (n > ((int64_t)1 << 31) / k || (int64_t)ql::absmean_partial_count(n * k) > ql::kPackScratchPartials)
        return QL_ERR_WORKSPACE;
    double *partials = nullptr;
    if (ql::pack_ternary_scratch(&partials) != hipSuccess) return QL_ERR_HIP;
    return hip_status(ql::launch_pack_ternary(w, layout == QL_W_NK, n, k, eps, packed, gamma, partials,
                                              as_stream(stream)));
}

ql_status qlinear_pack_int4(const uint8_t *codes, int64_t rows, int64_t cols, ql_int4_what what,
                            uint32_t *packed, void *stream) {
    if (!codes || !packed) return QL_ERR_NULL;
    if (!aligned16(codes) || !aligned16(packed)) return QL_ERR_ALIGN;
    if (what == QL_INT4_WEIGHT) {
        if (rows < 16 || cols < 128 || rows % 16 || cols % 128) return QL_ERR_SHAPE;
        return hip_status(ql::launch_pack_int4_weight(codes, rows, cols, packed, as_stream(stream)));
    }
    if (what == QL_INT4_ZEROS) {
        if (rows < 8 || cols < 1 || rows % 8) return QL_ERR_SHAPE;
        return hip_status(ql::launch_pack_int4_zeros(codes, rows, cols, packed, as_stream(stream)));
    }
    return QL_ERR_UNSUPPORTED;
}

ql_status qlinear_hbm_read_stream(const void *buf, size_t bytes, uint64_t *sink, void *stream) {
    if (!buf || !sink) return QL_ERR_NULL;
    if (bytes == 0 || bytes % 16 || bytes > (size_t)INT64_MAX) return QL_ERR_SHAPE;
    if (!aligned16(buf) || !aligned16(sink)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_hbm_read_stream(buf, (int64_t)bytes, sink, as_stream(stream)));
}

static ql_status gemm_out_kind(ql_dtype d, int *kind) {
    switch (d) {
        case QL_F16: *kind = ql::OUT_F16; return QL_OK;
        case QL_BF16: *kind = ql::OUT_BF16; return QL_OK;
        case QL_I32: *kind = ql::OUT_I32; return QL_OK;
        default: return QL_ERR_DTYPE;
    }
}

ql_status qlinear_gemm_w8a8(const int8_t *x, const int8_t *w, ql_wlayout layout, const float *deq_scale,
                            const float *per_token_scale, const float *bias, int64_t m, int64_t n, int64_t k,
                            ql_dtype out_dtype, void *out, void *stream) {
    int ok;
    if (!x || !w || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!deq_scale || !per_token_scale)) return QL_ERR_NULL;
    if (ok == ql::OUT_I32 && bias) return QL_ERR_UNSUPPORTED;
    if (layout != QL_W_KN && layout != QL_W_NK) return QL_ERR_UNSUPPORTED;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(bias)) return QL_ERR_ALIGN;
    if (ok != ql::OUT_I32 && (!aligned16(deq_scale) || !aligned16(per_token_scale))) return QL_ERR_ALIGN;
    ql::GemmI8Args a{x, w, layout == QL_W_NK, ql::EPI_ROWCOL, per_token_scale, deq_scale, nullptr,
                     nullptr, 0.0f, m, n, k, ok, out, bias};
    return hip_status(ql::launch_gemm_i8(a, as_stream(stream)));
}

ql_status qlinear_gemm_w8a8_batched(const int8_t *x, const int8_t *w, ql_wlayout layout, const float *deq_scale,
                                    int64_t deq_batch_stride, const float *per_token_scale, const float *bias,
                                    int64_t batch, int64_t m, int64_t n, int64_t k, ql_dtype out_dtype, void *out,
                                    void *stream) {
    if (batch < 1 || batch > 65535 || (deq_batch_stride != 0 && deq_batch_stride != n)) return QL_ERR_SHAPE;
    int ok;
    if (!x || !w || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!deq_scale || !per_token_scale)) return QL_ERR_NULL;
    if (ok == ql::OUT_I32 && bias) return QL_ERR_UNSUPPORTED;
    if (layout != QL_W_KN && layout != QL_W_NK) return QL_ERR_UNSUPPORTED;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(bias)) return QL_ERR_ALIGN;
    if (ok != ql::OUT_I32 && (!aligned16(deq_scale) || !aligned16(per_token_scale))) return QL_ERR_ALIGN;
    ql::GemmI8Args a{x, w, layout == QL_W_NK, ql::EPI_ROWCOL, per_token_scale, deq_scale, nullptr,
                     nullptr, 0.0f, m, n, k, ok, out, bias, batch, deq_batch_stride};
    return hip_status(ql::launch_gemm_i8(a, as_stream(stream)));
}

ql_status qlinear_gemm_w2a8(const int8_t *xq, const float *per_token_scale, const int32_t *rowsum,
                            const uint32_t *packed, const double *gamma, const float *bias, int64_t m, int64_t n,
                            int64_t k, ql_dtype out_dtype, void *out, void *stream) {
    int ok;
    if (!xq || !rowsum || !packed || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!per_token_scale || !gamma)) return QL_ERR_NULL;
    if (ok == ql::OUT_I32 && bias) return QL_ERR_UNSUPPORTED;
    if (m < 1 || n < 16 || k < 256 || n % 16 || k % 256 || k > kMaxK) return QL_ERR_SHAPE;
    if (!aligned16(xq) || !aligned16(rowsum) || !aligned16(packed) || !aligned16(out) || !aligned16(bias))
        return QL_ERR_ALIGN;
    if (ok != ql::OUT_I32 && (!aligned16(per_token_scale) || !aligned16(gamma))) return QL_ERR_ALIGN;
    return hip_status(ql::launch_gemm_w2a8(xq, per_token_scale, rowsum, packed, gamma, bias, m, n, k, ok, out,
                                           as_stream(stream)));
}

static ql_status grouped_int4(int64_t batch, const void *x, ql_dtype x_dtype, const float *per_token_scale,
                              const uint32_t *packed_w, const uint16_t *scales, const uint32_t *packed_zeros,
                              int64_t group_size, int64_t m, int64_t n, int64_t k, const float *bias,
                              ql_dtype out_dtype, void *out, void *stream) {
    if (!x || !packed_w || !scales || !packed_zeros || !out) return QL_ERR_NULL;
    if (x_dtype != QL_F16 && x_dtype != QL_I8) return QL_ERR_DTYPE;
    if (x_dtype == QL_I8 && !per_token_scale) return QL_ERR_NULL;
    if (out_dtype != QL_F16 && out_dtype != QL_F32 && !(x_dtype == QL_I8 && out_dtype == QL_BF16))
        return QL_ERR_DTYPE;
    if (m < 1 || n < 16 || k < 128 || n % 16 || k % 128 || group_size < 32 || group_size % 32 ||
        k % group_size || k > 0x7fffffff || n > 0x7fffffff || batch < 1 || batch > 65535)
        return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(packed_w) || !aligned16(scales) || !aligned16(packed_zeros) ||
        !aligned16(out) || !aligned16(bias) || (per_token_scale && !aligned16(per_token_scale)))
        return QL_ERR_ALIGN;
    const int ok = out_dtype == QL_F32 ? ql::OUT_F32 : out_dtype == QL_BF16 ? ql::OUT_BF16 : ql::OUT_F16;
    if (x_dtype == QL_I8)
        return hip_status(ql::launch_gemm_int4_grouped_i8(static_cast<const int8_t *>(x), per_token_scale,
                                                          packed_w, scales, packed_zeros, bias, group_size, m, n,
                                                          k, ok, out, as_stream(stream), batch));
    return hip_status(ql::launch_gemm_int4_grouped(static_cast<const uint16_t *>(x), packed_w, scales,
                                                   packed_zeros, bias, group_size, m, n, k, ok, out,
                                                   as_stream(stream), batch));
}

ql_status qlinear_gemm_w4a8_grouped(const void *x, ql_dtype x_dtype, const float *per_token_scale,
                                    const uint32_t *packed_w, const uint16_t *scales,
                                    const uint32_t *packed_zeros, int64_t group_size, int64_t m, int64_t n,
                                    int64_t k, const float *bias, ql_dtype out_dtype, void *out,
                                    void *stream) {
    return grouped_int4(1, x, x_dtype, per_token_scale, packed_w, scales, packed_zeros, group_size, m, n, k, bias,
                        out_dtype, out, stream);
}

ql_status qlinear_gemm_w4a8_grouped_batched(int64_t batch, const void *x, ql_dtype x_dtype,
                                            const float *per_token_scale, const uint32_t *packed_w,
                                            const uint16_t *scales, const uint32_t *packed_zeros,
                                            int64_t group_size, int64_t m, int64_t n, int64_t k,
                                            const float *bias, ql_dtype out_dtype, void *out, void *stream) {
    return grouped_int4(batch, x, x_dtype, per_token_scale, packed_w, scales, packed_zeros, group_size, m, n, k,
                        bias, out_dtype, out, stream);
}

ql_status qlinear_gemm_a4w4_codes(const int8_t *xq, const int8_t *wq, const float *scale_a,
                                  const float *scale_w, float eps, int64_t m, int64_t n, int64_t k,
                                  ql_dtype out_dtype, void *out, void *stream) {
    int ok;
    if (!xq || !wq || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!scale_a || !scale_w)) return QL_ERR_NULL;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(out)) return QL_ERR_ALIGN;
    ql::GemmI8Args a{xq, wq, true, ql::EPI_SCALARS, nullptr, nullptr, scale_a, scale_w, eps, m, n, k, ok, out};
    return hip_status(ql::launch_gemm_i8(a, as_stream(stream)));
}

ql_status qlinear_quant_a4w4_operand(const void *x, ql_dtype x_dtype, int64_t rows, int64_t k, const float *scale,
                                     float eps, void *operand, void *stream) {
    if (!x || !scale || !operand) return QL_ERR_NULL;
    const int kind = in_kind(x_dtype);
    if (kind < 0) return QL_ERR_DTYPE;
    if (rows < 1 || k < 1 || k > kMaxK) return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(operand)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_quant_a4w4_tiles(kind, x, rows, k, scale, eps, static_cast<uint8_t *>(operand),
                                                  as_stream(stream)));
}

ql_status qlinear_quant_a4w4_packed(const void *x, ql_dtype x_dtype, int64_t rows, int64_t k, const float *scale,
                                    float eps, void *operand, void *stream) {
    if (!x || !scale || !operand) return QL_ERR_NULL;
    const int kind = in_kind(x_dtype);
    if (kind < 0) return QL_ERR_DTYPE;
    if (rows < 1 || k < 1 || k > kMaxK || rows > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(operand)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_quant_a4w4_packed(kind, x, rows, k, scale, eps, static_cast<uint8_t *>(operand),
                                                   as_stream(stream)));
}

ql_status qlinear_gemm_a4w4_packed(const void *xa, const void *wb, const float *scale_a, const float *scale_w,
                                   float eps, int64_t m, int64_t n, int64_t k, ql_dtype out_dtype, void *out,
                                   void *stream) {
    int ok;
    if (!xa || !wb || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!scale_a || !scale_w)) return QL_ERR_NULL;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || m > 0x7fffffff || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(xa) || !aligned16(wb) || !aligned16(out)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_gemm_a4w4_packed(static_cast<const uint8_t *>(xa), static_cast<const uint8_t *>(wb),
                                                  scale_a, scale_w, eps, m, n, k, ok, out, as_stream(stream)));
}

ql_status qlinear_gemm_a4w4_operands(const void *xa, const void *wb, const float *scale_a, const float *scale_w,
                                     float eps, int64_t m, int64_t n, int64_t k, ql_dtype out_dtype, void *out,
                                     void *stream) {
    int ok;
    if (!xa || !wb || !out) return QL_ERR_NULL;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (ok != ql::OUT_I32 && (!scale_a || !scale_w)) return QL_ERR_NULL;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(xa) || !aligned16(wb) || !aligned16(out)) return QL_ERR_ALIGN;
    return hip_status(ql::launch_gemm_a4w4_tiles(static_cast<const uint8_t *>(xa), static_cast<const uint8_t *>(wb),
                                                 scale_a, scale_w, eps, m, n, k, ok, out, as_stream(stream)));
}

ql_status qlinear_gemm_a4w4(const void *x, const void *w, ql_dtype in_dtype, const float *scale_a,
                            const float *scale_w, float eps, int64_t m, int64_t n, int64_t k,
                            ql_dtype out_dtype, void *out, void *workspace, size_t ws_bytes, void *stream) {
    int ok;
    if (!x || !w || !scale_a || !scale_w || !out) return QL_ERR_NULL;
    const int kind = in_kind(in_dtype);
    if (kind < 0) return QL_ERR_DTYPE;
    const ql_status ds = gemm_out_kind(out_dtype, &ok);
    if (ds != QL_OK) return ds;
    if (m < 1 || n < 1 || k < 1 || k > kMaxK || n > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(w) || !aligned16(out)) return QL_ERR_ALIGN;
    if (!workspace || ws_bytes < qlinear_workspace_bytes(QL_OP_GEMM_A4W4, m, n, k)) return QL_ERR_WORKSPACE;
    if (!aligned16(workspace)) return QL_ERR_ALIGN;
    uint8_t *xa = static_cast<uint8_t *>(workspace);
    uint8_t *wb = xa + round256(ql::a4w4_operand_bytes(m, k));
    hipStream_t st = as_stream(stream);
    hipError_t e = ql::launch_quant_a4w4_tiles(kind, x, m, k, scale_a, eps, xa, st);
    if (e != hipSuccess) return QL_ERR_HIP;
    e = ql::launch_quant_a4w4_tiles(kind, w, n, k, scale_w, eps, wb, st);
    if (e != hipSuccess) return QL_ERR_HIP;
    return hip_status(ql::launch_gemm_a4w4_tiles(xa, wb, scale_a, scale_w, eps, m, n, k, ok, out, st));
}

ql_status qlinear_q4_backward(const void *grad_out, const void *x, const void *w, ql_dtype dtype,
                              const float *scale_a, const float *scale_w, float eps, int64_t m, int64_t n,
                              int64_t k, ql_dtype grad_dtype, void *grad_x, void *grad_w, float *grad_scale_a,
                              void *workspace, size_t ws_bytes, void *stream) {
    if (!grad_out || !x || !w || !scale_a || !scale_w || !grad_x || !grad_w || !grad_scale_a) return QL_ERR_NULL;
    if (dtype != QL_F16 && dtype != QL_BF16) return QL_ERR_DTYPE;
    int ok;
    switch (grad_dtype) {
        case QL_F32: ok = ql::OUT_F32; break;
        case QL_F16: ok = ql::OUT_F16; break;
        case QL_BF16: ok = ql::OUT_BF16; break;
        default: return QL_ERR_DTYPE;
    }
    if (m < 1 || n < 1 || k < 1 || m > 0x7fffffff || n > 0x7fffffff || k > 0x7fffffff) return QL_ERR_SHAPE;
    if (!aligned16(grad_out) || !aligned16(x) || !aligned16(w) || !aligned16(grad_x) || !aligned16(grad_w))
        return QL_ERR_ALIGN;
    if (!workspace || ws_bytes < qlinear_workspace_bytes(QL_OP_Q4_BACKWARD, m, n, k)) return QL_ERR_WORKSPACE;
    if (!aligned16(workspace)) return QL_ERR_ALIGN;
    ql::Q4BackwardArgs a{grad_out, x, w, dtype == QL_BF16, scale_a, scale_w, eps, m, n, k, ok,
                         grad_x, grad_w, grad_scale_a, workspace};
    return hip_status(ql::launch_q4_backward(a, as_stream(stream)));
}

}  // extern "C"
