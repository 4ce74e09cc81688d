"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The GPU library shares no code with it:
the arithmetic lives in ``qlinear_oracle.c`` (plain C loops, fp64 except
where a definition fixes a single fp32 operation) and this module only
converts numpy arrays to the C argument lists and back.

Sources (web pages, cited by title and section):

* bitorch-engine API docs, "Q4LinearFunction" -- forward (A4W4).
* LLaMA-BitNet utils.py, "Class BitLinear" -- forward docstring steps 1-5.
* Ascend CANN ATB docs, "Per-token Quantization for Matmul" -- Input,
  Parameters, Output, Example.
* frankenstein-transformer docs, "Common Attention Utilities" --
  activation_quant, weight_quant, BitLinear.bake_ternary_weights.
* docs.rs vyre-libs 0.7.2, "linear_4bit/mod.rs" -- module doc comment,
  QuantizedLinear4BitPlannerEvidence.

Every function here is pinned by ``tests/test_oracle_pins.py`` except the
three pack layouts (ternary words, 4-bit words, FP6 operand tiles), which are
this project's own definitions: "parity unpinned" beyond their round trip and
the end-to-end products that consume them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlinear_oracle.c")
# QLINEAR_ORACLE_LIB names a prebuilt copy of the oracle to load instead (the
# sanitizer test builds one with ASan/UBSan); it is never rebuilt from here.
_LIB_OVERRIDE = os.environ.get("QLINEAR_ORACLE_LIB")
_LIB_PATH = _LIB_OVERRIDE or os.path.join(_HERE, "liboracle.so")
_lib = None

# Plain C, no intrinsics, no BLAS.  -ffp-contract=off keeps every fl32 step
# of the definitions a single IEEE operation.
GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile ``qlinear_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, f32, f64, vp = (ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_double, ctypes.c_void_p)
        sig = {
            "oracle_quant_act": (i32, [vp, i64, i64, i32, f64, f32, vp, vp, vp]),
            "oracle_ternary_quant": (i32, [vp, i32, i64, i64, f64, vp, vp]),
            "oracle_ternary_tie_band": (i64, [vp, i64, f64, f64]),
            "oracle_pack_ternary_v1": (i32, [vp, i64, i64, vp]),
            "oracle_unpack_ternary_v1": (i32, [vp, i64, i64, vp]),
            "oracle_pack_int4_v1": (i32, [vp, i64, i64, vp]),
            "oracle_unpack_int4_v1": (i32, [vp, i64, i64, vp]),
            "oracle_pack_int4_zeros": (i32, [vp, i64, i64, vp]),
            "oracle_grouped_int4": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]),
            "oracle_grouped_int4_i8": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp]),
            "oracle_gemm_i8": (i32, [vp, vp, i32, i64, i64, i64, vp]),
            "oracle_dequant": (i32, [vp, vp, vp, i64, i64, vp]),
            "oracle_quant_int4_tensor": (i32, [vp, i64, f32, f32, vp]),
            "oracle_a4w4_operand_bytes": (i64, [i64, i64]),
            "oracle_q4_backward": (i32, [vp, vp, vp, f32, f32, f32, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
            "oracle_pack_a4w4_fp6": (i32, [vp, i64, i64, vp]),
            "oracle_a4w4_packed_bytes": (i64, [i64, i64]),
            "oracle_pack_a4w4_int4": (i32, [vp, i64, i64, vp]),
            "oracle_round_f16": (None, [vp, i64, vp]),
            "oracle_round_bf16": (None, [vp, i64, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(_lib, name)
            fn.restype = res
            fn.argtypes = args
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# --------------------------------------------------------------------------
# O1: per-token int8 activation quantization (absmax, optional RMSNorm).
# --------------------------------------------------------------------------
def quant_act(x, rmsnorm: bool = False, eps_norm: float = 1e-6, eps_q: float = 1e-5):
    """Per-token absmax int8 codes of ``x[m, k]`` (fp32 values).

    "Class BitLinear" forward steps 1-2 and 5; "Common Attention
    Utilities" activation_quant.  Returns ``(q int8[m,k], pts fp32[m],
    rowsum int32[m])``; ``pts`` is the per-token dequant scale
    ``a' * r / 127`` with ``r`` the RMSNorm factor (1 when off) and
    ``a' = max(absmax, fl32(eps_q / r))``: the guard applies to the absmax of
    the normalized row ``r * x``.
    """
    x = _c(x, np.float32)
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    pts = np.empty(m, np.float32)
    rs = np.empty(m, np.int32)
    _check(_load().oracle_quant_act(_p(x), m, k, int(rmsnorm), float(eps_norm),
                                    float(eps_q), _p(q), _p(pts), _p(rs)), "quant_act")
    return q, pts, rs


# --------------------------------------------------------------------------
# O2: absmean ternary weights and the 2-bit pack.
# --------------------------------------------------------------------------
def ternary_quant(w, layout_nk: bool = True, eps: float = 1e-5):
    """Ternary codes ``[n, k]`` and ``gamma' = max(mean|W|, eps)`` (fp64).

    "Class BitLinear" step 3; "Common Attention Utilities" weight_quant.
    ``layout_nk`` True means ``w`` is ``[n, k]``; False means ``[k, n]``.
    """
    w = _c(w, np.float32)
    if layout_nk:
        n, k = w.shape
    else:
        k, n = w.shape
    codes = np.empty((n, k), np.int8)
    g = ctypes.c_double(0.0)
    _check(_load().oracle_ternary_quant(_p(w), int(layout_nk), n, k, float(eps), _p(codes),
                                        ctypes.byref(g)), "ternary_quant")
    return codes, g.value


def ternary_tie_band(w, gamma: float, rel: float = 1e-12) -> int:
    """Number of weights within ``rel * gamma'`` of the threshold ``gamma'/2``."""
    w = _c(w, np.float32)
    return int(_load().oracle_ternary_tie_band(_p(w), w.size, float(gamma), float(rel)))


def pack_ternary(codes):
    """Pack ``[n, k]`` ternary codes into layout version 1 (u32 words)."""
    codes = _c(codes, np.int8)
    n, k = codes.shape
    out = np.empty(n * k // 16, np.uint32)
    _check(_load().oracle_pack_ternary_v1(_p(codes), n, k, _p(out)), "pack_ternary")
    return out


def unpack_ternary(packed, n: int, k: int):
    packed = _c(packed, np.uint32)
    out = np.empty((n, k), np.int8)
    _check(_load().oracle_unpack_ternary_v1(_p(packed), n, k, _p(out)), "unpack_ternary")
    return out


# --------------------------------------------------------------------------
# O3: 4-bit packs and the grouped affine INT4 product.
# --------------------------------------------------------------------------
def pack_int4(q):
    """Pack ``[n, k]`` uint4 codes (low nibble) into weight layout version 1."""
    q = _c(q, np.uint8)
    n, k = q.shape
    out = np.empty(n * k // 8, np.uint32)
    _check(_load().oracle_pack_int4_v1(_p(q), n, k, _p(out)), "pack_int4")
    return out


def unpack_int4(packed, n: int, k: int):
    packed = _c(packed, np.uint32)
    out = np.empty((n, k), np.uint8)
    _check(_load().oracle_unpack_int4_v1(_p(packed), n, k, _p(out)), "unpack_int4")
    return out


def pack_int4_zeros(z):
    """Pack zero-points ``z[n, g]`` group-major: ``[g, n/8]`` u32, column in nibble n%8."""
    z = _c(z, np.uint8)
    n, g = z.shape
    out = np.empty(g * n // 8, np.uint32)
    _check(_load().oracle_pack_int4_zeros(_p(z), n, g, _p(out)), "pack_int4_zeros")
    return out


def grouped_int4(x, q, s, z, group_size: int):
    """fp64 ``y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] * (q[n,k] - z[n,g])``.

    "linear_4bit/mod.rs" module doc (grouped affine INT4, scale plus
    zero-point sidecar).  Also returns ``bound[m,n] = sum_k |x * w|`` with the
    dequantized weight ``w = s * (q - z)``.
    """
    x = _c(x, np.float64)
    q = _c(q, np.uint8)
    s = _c(s, np.float64)
    z = _c(z, np.uint8)
    m, k = x.shape
    n = q.shape[0]
    assert q.shape == (n, k) and s.shape == z.shape == (n, k // group_size)
    y = np.empty((m, n), np.float64)
    b = np.empty((m, n), np.float64)
    _check(_load().oracle_grouped_int4(_p(x), _p(q), _p(s), _p(z), group_size, m, n, k,
                                       _p(y), _p(b)), "grouped_int4")
    return y, b


def grouped_int4_i8(xq, pts, q, s, z, group_size: int):
    """fp64 ``y[m,n] = pts[m] * sum_g s[n,g] * sum_{k in g} xq[m,k] * (q[n,k] - z[n,g])``.

    "linear_4bit/mod.rs" module doc for the weights; the per-token int8
    activation codes of "Class BitLinear" steps 2 and 5.  Group inner sums
    are exact integers.  Also returns ``bound[m,n] = |pts[m]| * sum_k
    |xq * s * (q - z)|``.
    """
    xq = _c(xq, np.int8)
    pts = _c(pts, np.float32)
    q = _c(q, np.uint8)
    s = _c(s, np.float64)
    z = _c(z, np.uint8)
    m, k = xq.shape
    n = q.shape[0]
    assert q.shape == (n, k) and s.shape == z.shape == (n, k // group_size) and pts.shape == (m,)
    y = np.empty((m, n), np.float64)
    b = np.empty((m, n), np.float64)
    _check(_load().oracle_grouped_int4_i8(_p(xq), _p(pts), _p(q), _p(s), _p(z), group_size, m, n, k,
                                          _p(y), _p(b)), "grouped_int4_i8")
    return y, b


# --------------------------------------------------------------------------
# O4: integer GEMM and the per-token dequant epilogue.
# --------------------------------------------------------------------------
def gemm_i8(x, w, layout_nk: bool):
    """int32 ``acc[m,n] = sum_k x[m,k] * w`` with ``w`` as ``[n,k]`` or ``[k,n]``.

    "Per-token Quantization for Matmul" Input / Example.
    """
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    m, k = x.shape
    n = w.shape[0] if layout_nk else w.shape[1]
    acc = np.empty((m, n), np.int32)
    _check(_load().oracle_gemm_i8(_p(x), _p(w), int(layout_nk), m, n, k, _p(acc)), "gemm_i8")
    return acc


def gemm_exact(x, w, layout_nk: bool):
    """``gemm_i8`` by a float64 matrix product (a library matmul as one step):
    every product of two int8 values and every partial sum of a k <= 2^37
    product is an integer below 2^53 in magnitude (127 * 128 * k), so the
    float64 result is exact whatever order the library sums in.  For
    products too large for the plain loops of ``gemm_i8``.

    "Per-token Quantization for Matmul" Input / Example.
    """
    x = np.asarray(x)
    w = np.asarray(w)
    assert x.dtype == np.int8 and w.dtype == np.int8
    k = x.shape[1]
    assert (w.shape[1] if layout_nk else w.shape[0]) == k and 127 * 128 * k < 2 ** 53
    wf = w.astype(np.float64)
    acc = x.astype(np.float64) @ (wf.T if layout_nk else wf)
    return acc.astype(np.int32)


def dequant(acc, pts, deq):
    """fp64 ``y[m,n] = acc[m,n] * pts[m] * deq[n]`` ("Per-token ... Example")."""
    acc = _c(acc, np.int32)
    pts = _c(pts, np.float32)
    deq = _c(deq, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), np.float64)
    _check(_load().oracle_dequant(_p(acc), _p(pts), _p(deq), m, n, _p(y)), "dequant")
    return y


def w8a8(x, w, layout_nk: bool, pts, deq):
    """Per-token W8A8 linear: ``(acc, y)``."""
    acc = gemm_i8(x, w, layout_nk)
    return acc, dequant(acc, pts, deq)


def w8a8_batched(x, w, layout_nk: bool, pts, deq):
    """``batch`` independent per-token W8A8 products ("Per-token Quantization
    for Matmul" Input / Output with a leading batch dimension): ``(acc, y)``
    of shapes ``[batch, m, n]``.  ``deq`` is ``[n]`` (every batch) or
    ``[batch, n]``; ``pts`` is ``[batch, m]``."""
    x, w = np.asarray(x), np.asarray(w)
    deq = np.asarray(deq)
    accs, ys = [], []
    for b in range(x.shape[0]):
        acc, y = w8a8(x[b], w[b], layout_nk, np.asarray(pts)[b], deq[b] if deq.ndim == 2 else deq)
        accs.append(acc)
        ys.append(y)
    return np.stack(accs), np.stack(ys)


def grouped_int4_batched(x, q, s, z, group_size: int, pts=None):
    """``batch`` independent grouped INT4 products ("linear_4bit/mod.rs" lists
    a batched grouped linear by name only; each slice has its own weights):
    ``grouped_int4`` of every slice, or ``grouped_int4_i8`` when the per-token
    scales ``pts[batch, m]`` of int8 codes are given.  Returns ``(y, bound)``
    of shape ``[batch, m, n]``."""
    ys, bs = [], []
    for b in range(len(x)):
        if pts is None:
            y, bd = grouped_int4(x[b], q[b], s[b], z[b], group_size)
        else:
            y, bd = grouped_int4_i8(x[b], pts[b], q[b], s[b], z[b], group_size)
        ys.append(y)
        bs.append(bd)
    return np.stack(ys), np.stack(bs)


def w2a8(xq, pts, codes, gamma: float):
    """BitLinear product on int8 activation codes and ternary codes ``[n,k]``.

    "Class BitLinear" steps 4-5: ``acc = xq @ codes^T`` and
    ``y = acc * pts[m] * fp32(gamma')``.
    """
    acc = gemm_i8(xq, codes, True)
    deq = np.full(codes.shape[0], np.float32(gamma), np.float32)
    return acc, dequant(acc, pts, deq)


def add_bias(y, bias):
    """fp64 ``y[m,n] + bias[n]``: the bias of a linear layer, added to the
    dequantized product ("Per-token Quantization for Matmul" Parameters
    hasBias; "linear_4bit/mod.rs" planner evidence bias bytes).  Not scaled
    by the quantization scales."""
    y = _c(y, np.float64)
    b = _c(bias, np.float32).astype(np.float64)
    assert b.shape == (y.shape[1],)
    return y + b[None, :]


# --------------------------------------------------------------------------
# O5: A4W4 per-tensor int4 quantization and product.
# --------------------------------------------------------------------------
def effective_scale(scale: float, eps: float) -> np.float32:
    """``max(scale, eps)`` in fp32 ("Q4LinearFunction" forward: eps guards the division)."""
    s, e = np.float32(scale), np.float32(eps)
    return s if s > e else e


def quant_int4_tensor(x, scale: float, eps: float):
    """``clamp(rne(fl32(x / max(scale, eps))), -8, 7)`` as int8 codes."""
    x = _c(x, np.float32)
    q = np.empty(x.shape, np.int8)
    _check(_load().oracle_quant_int4_tensor(_p(x), x.size, float(np.float32(scale)),
                                            float(np.float32(eps)), _p(q)), "quant_int4")
    return q


def a4w4(x, w, scale_a: float, scale_w: float, eps: float):
    """Q4Linear forward: ``(qa, qw, acc, y)`` with ``y = acc * s'_a * s'_w`` (fp64)."""
    qa = quant_int4_tensor(x, scale_a, eps)
    qw = quant_int4_tensor(w, scale_w, eps)
    acc = gemm_i8(qa, qw, True)
    sa, sw = effective_scale(scale_a, eps), effective_scale(scale_w, eps)
    y = acc.astype(np.float64) * float(sa) * float(sw)
    return qa, qw, acc, y


def q4_backward(g, x, w, scale_a: float, scale_w: float, eps: float):
    """Q4Linear backward ("Q4LinearFunction" backward, straight-through with
    the clip range and the learned step size term; see qlinear_oracle.c).

    ``g[m,n]`` output gradient, ``x[m,k]``, ``w[n,k]`` (fp32 copies of the
    16-bit tensors).  Returns ``(grad_x, grad_w, grad_scale_a, bx, bw, bs)``
    in fp64, the last three being the absolute-value sums the tolerances
    use: ``bx = s'_w sum_n |g q_w|``, ``bw = s'_a sum_m |g q_a|`` and
    ``bs = sum bx |q_a - v_a [in range]|``.
    """
    g = _c(g, np.float64)
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    m, n = g.shape
    k = x.shape[1]
    assert x.shape == (m, k) and w.shape == (n, k)
    gx = np.empty((m, k)); gw = np.empty((n, k)); bx = np.empty((m, k)); bw = np.empty((n, k))
    gs = np.zeros(1); bs = np.zeros(1)
    _check(_load().oracle_q4_backward(_p(g), _p(x), _p(w), float(np.float32(scale_a)), float(np.float32(scale_w)),
                                      float(np.float32(eps)), m, n, k, _p(gx), _p(gw), _p(gs), _p(bx), _p(bw),
                                      _p(bs)), "q4_backward")
    return gx, gw, float(gs[0]), bx, bw, float(bs[0])


def a4w4_operand_bytes(rows: int, k: int) -> int:
    return int(_load().oracle_a4w4_operand_bytes(rows, k))


def pack_a4w4_fp6(codes):
    """4-bit codes ``[rows, k]`` (int8, in [-8, 7]) as the packed FP6 E3M2
    operand tiles of the 4-bit product (this project's layout, defined in
    ``qlinear_oracle.c``).  Returns uint8 bytes."""
    codes = _c(codes, np.int8)
    rows, k = codes.shape
    out = np.zeros(a4w4_operand_bytes(rows, k), np.uint8)
    _check(_load().oracle_pack_a4w4_fp6(_p(codes), rows, k, _p(out)), "pack_a4w4_fp6")
    return out


def a4w4_packed_bytes(rows: int, k: int) -> int:
    return int(_load().oracle_a4w4_packed_bytes(rows, k))


def pack_a4w4_int4(codes):
    """4-bit codes ``[rows, k]`` (int8, in [-8, 7]) as the packed 4-bit operand of
    the 4-bit product: two codes per byte, stored as code + 8 (this project's
    layout, defined in ``qlinear_oracle.c``).  Returns uint8 bytes."""
    codes = _c(codes, np.int8)
    rows, k = codes.shape
    out = np.zeros(a4w4_packed_bytes(rows, k), np.uint8)
    _check(_load().oracle_pack_a4w4_int4(_p(codes), rows, k, _p(out)), "pack_a4w4_int4")
    return out


# --------------------------------------------------------------------------
# Output rounding and byte accounting.
# --------------------------------------------------------------------------
def round_f16(y) -> np.ndarray:
    """fp64 -> fp16 bit patterns, one round-to-nearest-even step."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_round_f16(_p(y), y.size, _p(out))
    return out


def round_bf16(y) -> np.ndarray:
    """fp64 -> bf16 bit patterns, one round-to-nearest-even step."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_round_bf16(_p(y), y.size, _p(out))
    return out


def int4_evidence_bytes(m: int, n: int, k: int, group_size: int, bias: bool = False) -> dict:
    """Byte fields of the grouped INT4 linear ("linear_4bit/mod.rs",
    QuantizedLinear4BitPlannerEvidence): packed 4-bit weight, the fp32
    dequantized matrix the fused path never writes, the scale (fp16) plus
    zero-point (4-bit) sidecar, bias, fp16 output, and the elided bytes."""
    g = k // group_size
    packed = n * k // 2
    deq = 4 * n * k
    return {
        "packed_weight_bytes": packed,
        "dequantized_weight_bytes": deq,
        "sidecar_bytes": g * n * 2 + g * n // 2,
        "bias_bytes": 2 * n if bias else 0,
        "output_bytes": 2 * m * n,
        "dequant_bytes_elided": deq,
    }
