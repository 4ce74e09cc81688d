"""Python binding of libqlinear, the gfx950 quantized linear layer library.

Argument marshalling only: every function takes torch tensors that live on
the GPU, checks dtype / shape / device, allocates missing outputs with torch
(PyTorch is used for device memory and streams only), and calls the C entry
point of the same name in ``libqlinear.so`` on the current HIP stream.
Every step of the layer runs in the library's HIP kernels; there is no CPU
fallback, and importing the library fails loudly when it is not built.

The C declarations, with the passages of the pages that define each
operation, are in ``include/qlinear.h``.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QLINEAR_LIB names another build of the same library (the sanitizer test
# loads a host-ASan/UBSan build this way); the default is the in-tree build.
LIB_PATH = os.environ.get("QLINEAR_LIB") or os.path.join(_HERE, "libqlinear.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qlinear.h")

# enums of qlinear.h
QL_OK = 0
QL_F32, QL_F16, QL_BF16, QL_I8, QL_U8, QL_I32 = range(6)
QL_W_KN, QL_W_NK = 0, 1
QL_RMSNORM = 1
QL_INT4_WEIGHT, QL_INT4_ZEROS = 0, 1
QL_OP_PACK_TERNARY, QL_OP_GEMM_A4W4, QL_OP_A4W4_OPERAND, QL_OP_Q4_BACKWARD, QL_OP_A4W4_PACKED = 0, 1, 2, 3, 4
STATUS = {0: "QL_OK", -1: "QL_ERR_NULL", -2: "QL_ERR_SHAPE", -3: "QL_ERR_DTYPE", -4: "QL_ERR_ALIGN",
          -5: "QL_ERR_WORKSPACE", -6: "QL_ERR_UNSUPPORTED", -7: "QL_ERR_HIP"}

_TORCH_TO_QL = {torch.float32: QL_F32, torch.float16: QL_F16, torch.bfloat16: QL_BF16,
                torch.int8: QL_I8, torch.uint8: QL_U8, torch.int32: QL_I32}
_QL_TO_TORCH = {v: k for k, v in _TORCH_TO_QL.items()}

_lib = None


# QL_ABI_VERSION of include/qlinear.h that the argument lists below follow.
ABI_VERSION = 8
# Words of the sink array of qlinear_hbm_read_stream (QL_HBM_STREAM_SINK_WORDS).
QL_HBM_STREAM_SINK_WORDS = 16384


class QLinearError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


def declared_functions() -> list[str]:
    """Names of the entry points declared in include/qlinear.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qlinear_\w+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Load libqlinear.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_quantized_linear_quant_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, u32, f32, f64, vp, sz = (ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_float,
                                           ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t)
        sigs = {
            "qlinear_abi_version": (i32, []),
            "qlinear_status_string": (ctypes.c_char_p, [i32]),
            "qlinear_workspace_bytes": (sz, [i32, i64, i64, i64]),
            "qlinear_quant_act": (i32, [vp, i32, i64, i64, u32, f32, f32, vp, vp, vp, vp]),
            "qlinear_quant_int4_tensor": (i32, [vp, i32, i64, vp, f32, vp, vp]),
            "qlinear_pack_ternary": (i32, [vp, i32, i64, i64, f64, vp, vp, vp, sz, vp]),
            "qlinear_pack_ternary_noalloc": (i32, [vp, i32, i64, i64, f64, vp, vp, vp]),
            "qlinear_pack_int4": (i32, [vp, i64, i64, i32, vp, vp]),
            "qlinear_hbm_read_stream": (i32, [vp, sz, vp, vp]),
            "qlinear_gemm_w8a8": (i32, [vp, vp, i32, vp, vp, vp, i64, i64, i64, i32, vp, vp]),
            "qlinear_gemm_w8a8_batched": (i32, [vp, vp, i32, vp, i64, vp, vp, i64, i64, i64, i64, i32, vp, vp]),
            "qlinear_gemm_w2a8": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]),
            "qlinear_gemm_w4a8_grouped": (i32, [vp, i32, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp,
                                                vp]),
            "qlinear_gemm_w4a8_grouped_batched": (i32, [i64, vp, i32, vp, vp, vp, vp, i64, i64, i64, i64, vp,
                                                        i32, vp, vp]),
            "qlinear_gemm_a4w4_codes": (i32, [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, vp]),
            "qlinear_gemm_a4w4": (i32, [vp, vp, i32, vp, vp, f32, i64, i64, i64, i32, vp, vp, sz, vp]),
            "qlinear_quant_a4w4_operand": (i32, [vp, i32, i64, i64, vp, f32, vp, vp]),
            "qlinear_gemm_a4w4_operands": (i32, [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, vp]),
            "qlinear_quant_a4w4_packed": (i32, [vp, i32, i64, i64, vp, f32, vp, vp]),
            "qlinear_gemm_a4w4_packed": (i32, [vp, vp, vp, vp, f32, i64, i64, i64, i32, vp, vp]),
            "qlinear_q4_backward": (i32, [vp, vp, vp, i32, vp, vp, f32, i64, i64, i64, i32, vp, vp, vp, vp, sz,
                                          vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        built = L.qlinear_abi_version()
        if built != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {built}, this binding needs {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _gpu(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _need(t, nbytes: int, name: str):
    """Reject a buffer smaller than the call reads or writes (the C ABI takes bare pointers)."""
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the call needs {nbytes}")
    return t


def _bias(bias, n: int, out_dtype):
    """Validate an optional fp32 bias ``[n]`` (added after the dequant, before the output rounding)."""
    if bias is None:
        return None
    if out_dtype == torch.int32:
        raise ValueError("a bias needs a floating-point output (int32 output is the raw accumulator)")
    return _need(_gpu(bias, "bias", torch.float32), 4 * n, "bias")


def _check(fn: str, rc: int) -> None:
    if rc != QL_OK:
        raise QLinearError(fn, rc)


def _empty(shape, dtype, like):
    return torch.empty(shape, dtype=dtype, device=like.device)


def qlinear_abi_version() -> int:
    return lib().qlinear_abi_version()


def qlinear_status_string(status: int) -> str:
    return lib().qlinear_status_string(status).decode()


def qlinear_workspace_bytes(op: int, m: int, n: int, k: int) -> int:
    return int(lib().qlinear_workspace_bytes(op, m, n, k))


def qlinear_quant_act(x, rmsnorm=False, eps_norm=1e-6, eps_q=1e-5, q=None, per_token_scale=None,
                      rowsum=None):
    """Per-token int8 codes of ``x[m, k]`` -> ``(q, per_token_scale, rowsum)``."""
    _gpu(x, "x")
    m, k = x.shape
    q = _empty((m, k), torch.int8, x) if q is None else _gpu(q, "q", torch.int8)
    pts = _empty((m,), torch.float32, x) if per_token_scale is None else _gpu(per_token_scale, "pts",
                                                                               torch.float32)
    rs = _empty((m,), torch.int32, x) if rowsum is None else _gpu(rowsum, "rowsum", torch.int32)
    _need(q, m * k, "q")
    _need(pts, 4 * m, "per_token_scale")
    _need(rs, 4 * m, "rowsum")
    _check("qlinear_quant_act", lib().qlinear_quant_act(
        _ptr(x), _TORCH_TO_QL[x.dtype], m, k, QL_RMSNORM if rmsnorm else 0, float(eps_norm), float(eps_q),
        _ptr(q), _ptr(pts), _ptr(rs), _stream(x)))
    return q, pts, rs


def qlinear_quant_int4_tensor(x, scale, eps=1e-5, q=None):
    """Per-tensor 4-bit codes (int8 storage) of ``x``; ``scale`` is a 1-element fp32 GPU tensor."""
    _gpu(x, "x")
    _gpu(scale, "scale", torch.float32)
    q = _empty(x.shape, torch.int8, x) if q is None else _gpu(q, "q", torch.int8)
    _need(q, x.numel(), "q")
    _check("qlinear_quant_int4_tensor", lib().qlinear_quant_int4_tensor(
        _ptr(x), _TORCH_TO_QL[x.dtype], x.numel(), _ptr(scale), float(eps), _ptr(q), _stream(x)))
    return q


def qlinear_pack_ternary(w, layout=QL_W_NK, eps=1e-5, packed=None, gamma=None, workspace=None):
    """Absmean ternary pack of fp32 ``w`` -> ``(packed u32 as int32, gamma fp64[1])``."""
    _gpu(w, "w", torch.float32)
    n, k = (w.shape if layout == QL_W_NK else (w.shape[1], w.shape[0]))
    packed = _empty((n * k // 16,), torch.int32, w) if packed is None else _gpu(packed, "packed")
    gamma = _empty((1,), torch.float64, w) if gamma is None else _gpu(gamma, "gamma", torch.float64)
    _need(packed, n * k // 4, "packed")
    ws_bytes = qlinear_workspace_bytes(QL_OP_PACK_TERNARY, 0, n, k)
    if workspace is None:
        workspace = _empty((max(ws_bytes, 1),), torch.uint8, w)
    _check("qlinear_pack_ternary", lib().qlinear_pack_ternary(
        _ptr(w), layout, n, k, float(eps), _ptr(packed), _ptr(gamma), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(w)))
    return packed, gamma


def qlinear_pack_ternary_noalloc(w, layout=QL_W_NK, eps=1e-5, packed=None, gamma=None):
    """As ``qlinear_pack_ternary`` through the entry point that allocates nothing on the device.

    The C function takes no workspace (its scratch is a static array of the library); output
    tensors are still allocated here when not given.
    """
    _gpu(w, "w", torch.float32)
    n, k = (w.shape if layout == QL_W_NK else (w.shape[1], w.shape[0]))
    packed = _empty((n * k // 16,), torch.int32, w) if packed is None else _gpu(packed, "packed")
    gamma = _empty((1,), torch.float64, w) if gamma is None else _gpu(gamma, "gamma", torch.float64)
    _need(packed, n * k // 4, "packed")
    _check("qlinear_pack_ternary_noalloc", lib().qlinear_pack_ternary_noalloc(
        _ptr(w), layout, n, k, float(eps), _ptr(packed), _ptr(gamma), _stream(w)))
    return packed, gamma


def qlinear_hbm_read_stream(buf, sink=None):
    """Read every byte of the device tensor ``buf`` once (HBM read-rate measurement aid).

    ``sink`` is a device int64 tensor of ``QL_HBM_STREAM_SINK_WORDS`` elements, XOR-accumulated
    word by word (not cleared); returns it.
    """
    _gpu(buf, "buf")
    if sink is None:
        sink = torch.zeros((QL_HBM_STREAM_SINK_WORDS,), dtype=torch.int64, device=buf.device)
    else:
        _gpu(sink, "sink", torch.int64)
        _need(sink, QL_HBM_STREAM_SINK_WORDS * 8, "sink")
    nbytes = buf.numel() * buf.element_size()
    _check("qlinear_hbm_read_stream", lib().qlinear_hbm_read_stream(_ptr(buf), nbytes, _ptr(sink), _stream(buf)))
    return sink


def qlinear_pack_int4(codes, what=QL_INT4_WEIGHT, packed=None):
    """Pack uint8 codes ``[rows, cols]`` (weights) or zero-points into u32 words (int32 tensor)."""
    _gpu(codes, "codes", torch.uint8)
    rows, cols = codes.shape
    packed = _empty((rows * cols // 8,), torch.int32, codes) if packed is None else _gpu(packed, "packed")
    _need(packed, rows * cols // 2, "packed")
    _check("qlinear_pack_int4", lib().qlinear_pack_int4(_ptr(codes), rows, cols, what, _ptr(packed),
                                                        _stream(codes)))
    return packed


def qlinear_gemm_w8a8(x, w, layout, deq_scale, per_token_scale, out_dtype=torch.float16, out=None, bias=None):
    """Per-token W8A8 linear: int8 ``x[m,k]`` times int8 ``w`` ([k,n] or [n,k]), optional fp32 ``bias[n]``."""
    _gpu(x, "x", torch.int8)
    _gpu(w, "w", torch.int8)
    m, k = x.shape
    n = w.shape[1] if layout == QL_W_KN else w.shape[0]
    if (w.shape[0] if layout == QL_W_KN else w.shape[1]) != k:
        raise ValueError(f"w {tuple(w.shape)} does not match x {tuple(x.shape)}")
    if out_dtype != torch.int32:
        _need(_gpu(deq_scale, "deq_scale", torch.float32), 4 * n, "deq_scale")
        _need(_gpu(per_token_scale, "per_token_scale", torch.float32), 4 * m, "per_token_scale")
    _bias(bias, n, out_dtype)
    out = _empty((m, n), out_dtype, x) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_w8a8", lib().qlinear_gemm_w8a8(
        _ptr(x), _ptr(w), layout, _ptr(deq_scale), _ptr(per_token_scale), _ptr(bias), m, n, k,
        _TORCH_TO_QL[out_dtype], _ptr(out), _stream(x)))
    return out


def qlinear_gemm_w8a8_batched(x, w, layout, deq_scale, per_token_scale, out_dtype=torch.float16, out=None,
                              bias=None):
    """``batch`` independent W8A8 products: ``x[batch,m,k]``, ``w[batch,k,n]`` or ``[batch,n,k]``,
    ``per_token_scale[batch,m]``, ``deq_scale[n]`` (shared) or ``[batch,n]``, optional ``bias[n]``."""
    _gpu(x, "x", torch.int8)
    _gpu(w, "w", torch.int8)
    if x.dim() != 3 or w.dim() != 3 or w.shape[0] != x.shape[0]:
        raise ValueError(f"x {tuple(x.shape)} and w {tuple(w.shape)} must be [batch, ., .] of one batch")
    batch, m, k = x.shape
    n = w.shape[2] if layout == QL_W_KN else w.shape[1]
    if (w.shape[1] if layout == QL_W_KN else w.shape[2]) != k:
        raise ValueError(f"w {tuple(w.shape)} does not match x {tuple(x.shape)}")
    deq_stride = 0
    if out_dtype != torch.int32:
        _gpu(deq_scale, "deq_scale", torch.float32)
        deq_stride = n if deq_scale.dim() == 2 else 0
        _need(deq_scale, 4 * n * (batch if deq_stride else 1), "deq_scale")
        _need(_gpu(per_token_scale, "per_token_scale", torch.float32), 4 * batch * m, "per_token_scale")
    _bias(bias, n, out_dtype)
    out = _empty((batch, m, n), out_dtype, x) if out is None else _gpu(out, "out", out_dtype)
    _need(out, batch * m * n * out.element_size(), "out")
    _check("qlinear_gemm_w8a8_batched", lib().qlinear_gemm_w8a8_batched(
        _ptr(x), _ptr(w), layout, _ptr(deq_scale), deq_stride, _ptr(per_token_scale), _ptr(bias), batch, m, n, k,
        _TORCH_TO_QL[out_dtype], _ptr(out), _stream(x)))
    return out


def qlinear_gemm_w2a8(xq, per_token_scale, rowsum, packed, gamma, n, out_dtype=torch.bfloat16, out=None,
                      bias=None):
    """BitLinear product of int8 codes ``xq[m,k]`` and packed ternary weights (``n`` columns), optional bias."""
    _gpu(xq, "xq", torch.int8)
    _gpu(rowsum, "rowsum", torch.int32)
    _gpu(packed, "packed")
    m, k = xq.shape
    _need(rowsum, 4 * m, "rowsum")
    _need(packed, n * k // 4, "packed")
    if out_dtype != torch.int32:
        _need(_gpu(per_token_scale, "per_token_scale", torch.float32), 4 * m, "per_token_scale")
        _gpu(gamma, "gamma", torch.float64)
    _bias(bias, n, out_dtype)
    out = _empty((m, n), out_dtype, xq) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_w2a8", lib().qlinear_gemm_w2a8(
        _ptr(xq), _ptr(per_token_scale), _ptr(rowsum), _ptr(packed), _ptr(gamma), _ptr(bias), m, n, k,
        _TORCH_TO_QL[out_dtype], _ptr(out), _stream(xq)))
    return out


def qlinear_gemm_w4a8_grouped(x, packed_w, scales, packed_zeros, group_size, n, out_dtype=torch.float16,
                              out=None, per_token_scale=None, bias=None):
    """Grouped affine INT4 linear; ``scales`` fp16 ``[n, k/group_size]``.

    ``x[m,k]`` is fp16 activations, or int8 activation codes with their fp32
    ``per_token_scale[m]`` (from ``qlinear_quant_act``).  ``bias`` is an
    optional fp32 ``[n]``.
    """
    _gpu(x, "x")
    if x.dtype == torch.int8:
        _need(_gpu(per_token_scale, "per_token_scale", torch.float32), 4 * x.shape[0], "per_token_scale")
    _gpu(packed_w, "packed_w")
    _gpu(scales, "scales", torch.float16)
    _gpu(packed_zeros, "packed_zeros")
    m, k = x.shape
    if group_size > 0 and k % group_size == 0:
        _need(packed_w, n * k // 2, "packed_w")
        _need(scales, 2 * n * (k // group_size), "scales")
        _need(packed_zeros, n * (k // group_size) // 2, "packed_zeros")
    _bias(bias, n, out_dtype)
    out = _empty((m, n), out_dtype, x) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_w4a8_grouped", lib().qlinear_gemm_w4a8_grouped(
        _ptr(x), _TORCH_TO_QL[x.dtype], _ptr(per_token_scale), _ptr(packed_w), _ptr(scales),
        _ptr(packed_zeros), group_size, m, n, k, _ptr(bias), _TORCH_TO_QL[out_dtype], _ptr(out),
        _stream(x)))
    return out


def qlinear_gemm_w4a8_grouped_batched(x, packed_w, scales, packed_zeros, group_size, n,
                                      out_dtype=torch.float16, out=None, per_token_scale=None, bias=None):
    """``batch`` independent grouped INT4 products: ``x[batch,m,k]`` (fp16, or
    int8 codes with ``per_token_scale[batch,m]``), each slice with its own
    packed weights ``[batch, n*k/8]`` words, fp16 scales ``[batch, n,
    k/group_size]``, packed zero-points and optional fp32 ``bias[batch,n]``;
    returns ``out[batch,m,n]``.
    """
    _gpu(x, "x")
    batch, m, k = x.shape
    if x.dtype == torch.int8:
        _need(_gpu(per_token_scale, "per_token_scale", torch.float32), 4 * batch * m, "per_token_scale")
    _gpu(packed_w, "packed_w")
    _gpu(scales, "scales", torch.float16)
    _gpu(packed_zeros, "packed_zeros")
    if group_size > 0 and k % group_size == 0:
        _need(packed_w, batch * n * k // 2, "packed_w")
        _need(scales, 2 * batch * n * (k // group_size), "scales")
        _need(packed_zeros, batch * n * (k // group_size) // 2, "packed_zeros")
    if bias is not None:
        _need(_gpu(bias, "bias", torch.float32), 4 * batch * n, "bias")
    out = _empty((batch, m, n), out_dtype, x) if out is None else _gpu(out, "out", out_dtype)
    _need(out, batch * m * n * out.element_size(), "out")
    _check("qlinear_gemm_w4a8_grouped_batched", lib().qlinear_gemm_w4a8_grouped_batched(
        batch, _ptr(x), _TORCH_TO_QL[x.dtype], _ptr(per_token_scale), _ptr(packed_w), _ptr(scales),
        _ptr(packed_zeros), group_size, m, n, k, _ptr(bias), _TORCH_TO_QL[out_dtype], _ptr(out), _stream(x)))
    return out


def qlinear_gemm_a4w4_codes(xq, wq, scale_a, scale_w, eps=1e-5, out_dtype=torch.float16, out=None):
    """A4W4 product of int8-held 4-bit codes ``xq[m,k]`` and ``wq[n,k]``."""
    _gpu(xq, "xq", torch.int8)
    _gpu(wq, "wq", torch.int8)
    m, k = xq.shape
    n = wq.shape[0]
    if wq.shape[1] != k:
        raise ValueError(f"wq {tuple(wq.shape)} does not match xq {tuple(xq.shape)}")
    if out_dtype != torch.int32:
        _gpu(scale_a, "scale_a", torch.float32)
        _gpu(scale_w, "scale_w", torch.float32)
    out = _empty((m, n), out_dtype, xq) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_a4w4_codes", lib().qlinear_gemm_a4w4_codes(
        _ptr(xq), _ptr(wq), _ptr(scale_a), _ptr(scale_w), float(eps), m, n, k, _TORCH_TO_QL[out_dtype],
        _ptr(out), _stream(xq)))
    return out


def qlinear_gemm_a4w4(x, w, scale_a, scale_w, eps=1e-5, out_dtype=torch.float16, out=None, workspace=None):
    """Q4Linear forward: per-tensor 4-bit quantization of ``x[m,k]`` and ``w[n,k]``, then the product."""
    _gpu(x, "x")
    _gpu(w, "w", x.dtype)
    _gpu(scale_a, "scale_a", torch.float32)
    _gpu(scale_w, "scale_w", torch.float32)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError(f"w {tuple(w.shape)} does not match x {tuple(x.shape)}")
    ws_bytes = qlinear_workspace_bytes(QL_OP_GEMM_A4W4, m, n, k)
    if workspace is None:
        workspace = _empty((ws_bytes,), torch.uint8, x)
    out = _empty((m, n), out_dtype, x) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_a4w4", lib().qlinear_gemm_a4w4(
        _ptr(x), _ptr(w), _TORCH_TO_QL[x.dtype], _ptr(scale_a), _ptr(scale_w), float(eps), m, n, k,
        _TORCH_TO_QL[out_dtype], _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(x)))
    return out, workspace


def a4w4_operands_from_workspace(workspace, m, n, k):
    """Byte views of the x and w FP6 operands that qlinear_gemm_a4w4 leaves in its workspace."""
    bx = qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, m, 0, k)
    bw = qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, n, 0, k)
    off = (bx + 255) // 256 * 256
    return workspace[:bx], workspace[off:off + bw]


def qlinear_quant_a4w4_operand(x, scale, eps=1e-5, operand=None):
    """Per-tensor 4-bit codes of ``x[rows,k]`` written as the packed FP6 operand (uint8 bytes)."""
    _gpu(x, "x")
    _gpu(scale, "scale", torch.float32)
    rows, k = x.shape
    nbytes = qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, rows, 0, k)
    operand = _empty((nbytes,), torch.uint8, x) if operand is None else _gpu(operand, "operand")
    _need(operand, nbytes, "operand")
    _check("qlinear_quant_a4w4_operand", lib().qlinear_quant_a4w4_operand(
        _ptr(x), _TORCH_TO_QL[x.dtype], rows, k, _ptr(scale), float(eps), _ptr(operand), _stream(x)))
    return operand


def qlinear_gemm_a4w4_operands(xa, wb, m, n, k, scale_a, scale_w, eps=1e-5, out_dtype=torch.float16, out=None):
    """A4W4 product of two packed FP6 operands (of ``x[m,k]`` and ``w[n,k]``)."""
    _gpu(xa, "xa")
    _gpu(wb, "wb")
    _need(xa, qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, m, 0, k), "xa")
    _need(wb, qlinear_workspace_bytes(QL_OP_A4W4_OPERAND, n, 0, k), "wb")
    if out_dtype != torch.int32:
        _gpu(scale_a, "scale_a", torch.float32)
        _gpu(scale_w, "scale_w", torch.float32)
    out = _empty((m, n), out_dtype, xa) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_a4w4_operands", lib().qlinear_gemm_a4w4_operands(
        _ptr(xa), _ptr(wb), _ptr(scale_a), _ptr(scale_w), float(eps), m, n, k, _TORCH_TO_QL[out_dtype],
        _ptr(out), _stream(xa)))
    return out


def qlinear_quant_a4w4_packed(x, scale, eps=1e-5, operand=None):
    """Per-tensor 4-bit codes of ``x[rows,k]`` written two per byte (the packed 4-bit operand, uint8 bytes)."""
    _gpu(x, "x")
    _gpu(scale, "scale", torch.float32)
    rows, k = x.shape
    nbytes = qlinear_workspace_bytes(QL_OP_A4W4_PACKED, rows, 0, k)
    operand = _empty((nbytes,), torch.uint8, x) if operand is None else _gpu(operand, "operand")
    _need(operand, nbytes, "operand")
    _check("qlinear_quant_a4w4_packed", lib().qlinear_quant_a4w4_packed(
        _ptr(x), _TORCH_TO_QL[x.dtype], rows, k, _ptr(scale), float(eps), _ptr(operand), _stream(x)))
    return operand


def qlinear_gemm_a4w4_packed(xa, wb, m, n, k, scale_a, scale_w, eps=1e-5, out_dtype=torch.float16, out=None):
    """A4W4 product of two packed 4-bit operands (of ``x[m,k]`` and ``w[n,k]``), two codes per byte."""
    _gpu(xa, "xa")
    _gpu(wb, "wb")
    _need(xa, qlinear_workspace_bytes(QL_OP_A4W4_PACKED, m, 0, k), "xa")
    _need(wb, qlinear_workspace_bytes(QL_OP_A4W4_PACKED, n, 0, k), "wb")
    if out_dtype != torch.int32:
        _gpu(scale_a, "scale_a", torch.float32)
        _gpu(scale_w, "scale_w", torch.float32)
    out = _empty((m, n), out_dtype, xa) if out is None else _gpu(out, "out", out_dtype)
    _need(out, m * n * out.element_size(), "out")
    _check("qlinear_gemm_a4w4_packed", lib().qlinear_gemm_a4w4_packed(
        _ptr(xa), _ptr(wb), _ptr(scale_a), _ptr(scale_w), float(eps), m, n, k, _TORCH_TO_QL[out_dtype],
        _ptr(out), _stream(xa)))
    return out


def qlinear_q4_backward(grad_out, x, w, scale_a, scale_w, eps=1e-5, grad_dtype=torch.float32, grad_x=None,
                        grad_w=None, grad_scale_a=None, workspace=None):
    """Q4Linear backward: ``(grad_x[m,k], grad_w[n,k], grad_scale_a[1])`` from ``grad_out[m,n]``.

    ``grad_out``, ``x`` and ``w`` share one dtype (fp16 or bf16); the scales
    are the forward's 1-element fp32 GPU tensors.
    """
    _gpu(grad_out, "grad_out")
    _gpu(x, "x", grad_out.dtype)
    _gpu(w, "w", grad_out.dtype)
    _gpu(scale_a, "scale_a", torch.float32)
    _gpu(scale_w, "scale_w", torch.float32)
    m, n = grad_out.shape
    k = x.shape[1]
    if x.shape[0] != m or w.shape != (n, k):
        raise ValueError(f"grad_out {tuple(grad_out.shape)}, x {tuple(x.shape)}, w {tuple(w.shape)} do not match")
    grad_x = _empty((m, k), grad_dtype, x) if grad_x is None else _gpu(grad_x, "grad_x", grad_dtype)
    grad_w = _empty((n, k), grad_dtype, x) if grad_w is None else _gpu(grad_w, "grad_w", grad_dtype)
    _need(grad_x, m * k * grad_x.element_size(), "grad_x")
    _need(grad_w, n * k * grad_w.element_size(), "grad_w")
    grad_scale_a = _empty((1,), torch.float32, x) if grad_scale_a is None else _gpu(grad_scale_a, "grad_scale_a",
                                                                                     torch.float32)
    ws_bytes = qlinear_workspace_bytes(QL_OP_Q4_BACKWARD, m, n, k)
    workspace = _empty((ws_bytes,), torch.uint8, x) if workspace is None else _gpu(workspace, "workspace")
    _check("qlinear_q4_backward", lib().qlinear_q4_backward(
        _ptr(grad_out), _ptr(x), _ptr(w), _TORCH_TO_QL[grad_out.dtype], _ptr(scale_a), _ptr(scale_w), float(eps),
        m, n, k, _TORCH_TO_QL[grad_dtype], _ptr(grad_x), _ptr(grad_w), _ptr(grad_scale_a), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(x)))
    return grad_x, grad_w, grad_scale_a
