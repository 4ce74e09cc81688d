"""Seeded synthetic inputs for the quantized linear layer.

The one module that both the CPU oracle's tests and the GPU path draw their
inputs from.  It holds random draws and dtype casts only -- none of the
layer's arithmetic.  numpy ``Generator(PCG64(seed))``; each workload's
default seed is 1000 + its number below.  Tensors are returned on the CPU
(torch is used only to hold bf16 / fp16 values, which numpy lacks).

Workloads (shapes and value distributions of the pages' problems; no public
benchmark or dataset exists for them, so these synthetic draws stand in):

1. per-token W8A8: int8 x[16,256], int8 w[256,128] ([k,n]), fp32 deqScale[128]
   and perTokenScale[16] uniform in [1e-3, 1e-2].
2. BitLinear forward: bf16 x[2048,4096] N(0,1) with 1% of entries x20,
   fp32 w[4096,4096] N(0, 0.02^2).
3. decode GEMV: bf16 x[M,8192] N(0,1) for M in {1,4,16}, fp32 w[28672,8192]
   N(0, 0.02^2).
4. grouped INT4: fp16 x[32,4096] N(0,1), uint4 codes[11008,4096], fp16
   scales[11008,32] uniform in [1e-3, 2e-2], uint4 zeros[11008,32], g=128.
5. A4W4: fp16 x[8192,8192] N(0,1), fp16 w[8192,8192] N(0, 0.02^2), scale_a
   and scale_w fp32 scalars set to max|t| / 7 of each tensor (the caller's
   per-tensor calibration), eps=1e-5.

An optional bias of any product is fp32 [n] drawn N(0, scale^2), scale
chosen by the caller near the output's magnitude (``bias``).
"""
from __future__ import annotations

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16)


def w8a8(m: int = 16, n: int = 128, k: int = 256, layout_nk: bool = False, seed: int = 1001):
    """Workload 1: int8 activations and weights, fp32 per-token and per-column scales."""
    g = rng(seed)
    x = g.integers(-128, 128, (m, k), dtype=np.int8)
    w_shape = (n, k) if layout_nk else (k, n)
    w = g.integers(-128, 128, w_shape, dtype=np.int8)
    deq = g.uniform(1e-3, 1e-2, n).astype(np.float32)
    pts = g.uniform(1e-3, 1e-2, m).astype(np.float32)
    return {"x": torch.from_numpy(x), "w": torch.from_numpy(w), "deq": torch.from_numpy(deq),
            "pts": torch.from_numpy(pts), "layout_nk": layout_nk}


def worked_example():
    """The 2x2x3 per-token example printed on "Per-token Quantization for Matmul"."""
    return {"x": torch.tensor([[1, 2], [3, 4]], dtype=torch.int8),
            "w": torch.tensor([[1, 2, 3], [4, 5, 6]], dtype=torch.int8),
            "deq": torch.tensor([1.0, 2.0, 3.0], dtype=torch.float32),
            "pts": torch.tensor([1.0, 2.0], dtype=torch.float32),
            "layout_nk": False}


def activations(m: int, k: int, seed: int, outliers: float = 0.0,
                dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """N(0,1) activations; a fraction ``outliers`` of entries scaled by 20."""
    g = rng(seed)
    x = g.standard_normal((m, k), dtype=np.float32)
    if outliers:
        mask = g.random((m, k)) < outliers
        x[mask] *= 20.0
    return _bf16(x) if dtype == torch.bfloat16 else (
        _f16(x) if dtype == torch.float16 else torch.from_numpy(x))


def master_weight(n: int, k: int, seed: int, std: float = 0.02) -> torch.Tensor:
    """fp32 N(0, std^2) weight in nn.Linear layout [n, k]."""
    g = rng(seed)
    w = g.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(std)
    return torch.from_numpy(w)


def bitlinear(m: int = 2048, n: int = 4096, k: int = 4096, seed: int = 1002):
    """Workload 2: BitLinear forward inputs (bf16 x with 1% outliers, fp32 weight)."""
    return {"x": activations(m, k, seed, outliers=0.01),
            "w": master_weight(n, k, seed + 100_000)}


def decode(ms=(1, 4, 16), n: int = 28672, k: int = 8192, seed: int = 1003):
    """Workload 3: decode-sized activations for each M and one shared fp32 weight."""
    return {"x": {m: activations(m, k, seed + m) for m in ms},
            "w": master_weight(n, k, seed + 100_000)}


def grouped_int4(m: int = 32, n: int = 11008, k: int = 4096, group_size: int = 128,
                 seed: int = 1004):
    """Workload 4: fp16 x, uint4 codes [n,k], fp16 scales and uint4 zeros [n, k/g]."""
    g = rng(seed)
    x = g.standard_normal((m, k), dtype=np.float32)
    q = g.integers(0, 16, (n, k), dtype=np.uint8)
    s = g.uniform(1e-3, 2e-2, (n, k // group_size)).astype(np.float32)
    z = g.integers(0, 16, (n, k // group_size), dtype=np.uint8)
    return {"x": _f16(x), "q": torch.from_numpy(q), "s": _f16(s), "z": torch.from_numpy(z),
            "group_size": group_size}


def a4w4(m: int = 8192, n: int = 8192, k: int = 8192, seed: int = 1005, eps: float = 1e-5,
         scale_div: float = 7.0):
    """Workload 5: fp16 x and w; per-tensor fp32 scales max|t| / scale_div."""
    g = rng(seed)
    x = _f16(g.standard_normal((m, k), dtype=np.float32))
    w32 = g.standard_normal((n, k), dtype=np.float32)
    w32 *= np.float32(0.02)
    w = _f16(w32)
    sa = np.float32(x.abs().max().float().item()) / np.float32(scale_div)
    sw = np.float32(w.abs().max().float().item()) / np.float32(scale_div)
    return {"x": x, "w": w, "scale_a": float(sa), "scale_w": float(sw), "eps": eps}


def bias(n: int, scale: float, seed: int) -> torch.Tensor:
    """fp32 bias [n], N(0, scale^2)."""
    return torch.from_numpy(rng(seed).normal(0.0, scale, n).astype(np.float32))
