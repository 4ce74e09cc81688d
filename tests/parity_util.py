"""Shared helpers of the GPU parity tests: tolerances and conversions.

Tolerances (relative to the oracle's fp64 value y):
  bf16 output: |gpu - y| <= 2^-7 |y| + 1e-6
  fp16 output: |gpu - y| <= 2^-10 |y| + 1e-6
  grouped INT4 (fp16 activations): |gpu - y| <= 1e-3 * sum_k |x_k * w_k|
  with a bias b, y is the oracle's y0 + b and the bound gains the fp32
  roundings of the dequant and the add: 2^-22 (|y0| + |b|)
Integer results (codes, packed words, int32 accumulators) must be identical.
"""
import numpy as np
import torch

TOL_REL = {torch.bfloat16: 2.0 ** -7, torch.float16: 2.0 ** -10}
TOL_ABS = 1e-6


def absmean_rel_tol(count: int) -> float:
    """Relative bound on |gamma_gpu - gamma_oracle| for the ternary absmean.

    The oracle's gamma is the exact sum of |W| rounded once, divided once
    (2 roundings).  The kernel sums |W| in fp64 along paths of at most
    64 sequential adds per thread (16384-element chunks over 256 threads),
    6 shuffle levels and 3 wave adds per workgroup, then in one 1024-thread
    workgroup ceil(chunks / 1024) sequential adds per thread, 6 shuffle levels
    and 15 wave adds, then divides once; a sum of non-negative terms along a
    path of d adds is off by at most d units of 2^-53 relative.
    """
    chunks = -(-count // 16384)
    depth = 64 + 6 + 3 + -(-chunks // 1024) + 6 + 15 + 1
    return (depth + 2) * 2.0 ** -53


def rms_pts_rel_tol(k: int) -> float:
    """Relative bound on |pts_gpu - pts_oracle| for quant_act with RMSNorm.

    The kernel sums x^2 in fp32 (squares of bf16 / fp16 values are exact,
    fp32 ones round once) along addition paths of depth d: rows of whole
    8-element chunks up to k = 8192 run one wave per row, each lane adding
    8 * NCH terms (NCH the smallest of 2, 4, 8, 16 with 64 * 8 * NCH >= k)
    then 6 shuffle levels; other rows run 256 threads per row, each adding
    8 * ceil(k / 2048) terms, then 6 shuffle levels and 3 adds across waves.
    A sum of non-negative terms along depth d is within (d + 1) u of exact
    (u = 2^-24).  Then ss / k and + eps_n round once each (the sum of two
    non-negative terms keeps the relative error), the square root halves the
    relative error and rounds once, 1 / sqrt and a' * r and / 127 round once
    each, and the oracle rounds its fp64 value once: (d + 3) / 2 + 5 units.
    Rows that reach the eps guard have pts = fl(fl(eps * D) / D) / 127 with
    the same D on both factors, within 7 units, which the bound covers.
    """
    if k % 8 == 0 and k <= 8192:
        nch = next(c for c in (2, 4, 8, 16) if 64 * 8 * c >= k)
        depth = 8 * nch + 6
    else:
        depth = 8 * (-(-k // 2048)) + 6 + 3
    return ((depth + 3) / 2 + 5) * 2.0 ** -24


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.numpy()


def words(t: torch.Tensor) -> np.ndarray:
    """Packed u32 words held in an int32 tensor."""
    return t.detach().cpu().numpy().view(np.uint32)


def assert_float_close(gpu: torch.Tensor, y: np.ndarray, what: str = "out", extra=None) -> None:
    """``extra`` (array or scalar) widens the bound by an absolute amount per element."""
    rel = TOL_REL[gpu.dtype]
    g = to_np(gpu).astype(np.float64)
    assert g.shape == y.shape, (g.shape, y.shape)
    err = np.abs(g - y)
    tol = rel * np.abs(y) + TOL_ABS + (0.0 if extra is None else extra)
    bad = ~(err <= tol)  # NaN counts as bad
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / tol, -1)), y.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {y.size} outside tolerance; worst at {idx}: "
                             f"gpu={g[idx]!r} oracle={y[idx]!r}")


def assert_equal(gpu, ref: np.ndarray, what: str) -> None:
    g = gpu if isinstance(gpu, np.ndarray) else gpu.detach().cpu().numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if not np.array_equal(g, ref):
        bad = np.argwhere(g != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ref.size} differ; first at {i}: gpu={g[i]} oracle={ref[i]}")


def poison(shape, dtype, device="cuda:0") -> torch.Tensor:
    """Output buffer filled with 0xFF bytes (NaN for floats, -1 for ints) to catch unwritten elements."""
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0xFF)
    return t
