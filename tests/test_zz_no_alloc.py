"""GPU tier: the allocation-free ternary pack (qlinear_pack_ternary_noalloc).

It must give exactly what qlinear_pack_ternary gives (same kernels, its
scratch in a static device array instead of a workspace), on consecutive
calls that share that array, the second with a smaller input, so a stale
partial of the first call would show.  Called through the C ABI (ctypes).
"""
import numpy as np
import pytest
import torch

import bit_quantized_linear_quant_amd as ql
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    ql.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _pack_both(w, layout):
    ref_p, ref_g = ql.qlinear_pack_ternary(w, layout)
    p = torch.full_like(ref_p, -1)
    g = torch.full_like(ref_g, float("nan"))
    ql.qlinear_pack_ternary_noalloc(w, layout, packed=p, gamma=g)
    torch.cuda.synchronize()
    return ref_p, ref_g, p, g


@pytest.mark.parametrize("layout", [1, 0])   # QL_W_NK, QL_W_KN
def test_noalloc_pack_matches_workspace_pack_on_consecutive_calls(layout):
    shapes = [(4096, 4096), (48, 512)]        # the second call smaller than the first
    for i, (n, k) in enumerate(shapes):
        w = synthetic.master_weight(n, k, 2000 + i).to(DEV)
        if layout == 0:
            w = w.t().contiguous()
        ref_p, ref_g, p, g = _pack_both(w, layout)
        assert torch.equal(p, ref_p), f"call {i} ({n}x{k}): packed words differ"
        assert torch.equal(g.view(torch.int64), ref_g.view(torch.int64)), f"call {i}: gamma differs"


def test_noalloc_pack_large_then_tiny():
    """A large call (8192 chunk partials), then a tiny one: partials beyond the tiny call's
    chunk count are left over from the large one and must not be read."""
    n, k = 16384, 8192                         # 2^27 weights: 8192 partials
    w = synthetic.master_weight(n, k, 2100).to(DEV)
    ref_p, ref_g, p, g = _pack_both(w, 1)
    assert torch.equal(p, ref_p) and torch.equal(g, ref_g)
    del w, ref_p, p
    w = synthetic.master_weight(16, 256, 2101).to(DEV)
    ref_p, ref_g, p, g = _pack_both(w, 1)
    assert torch.equal(p, ref_p) and torch.equal(g, ref_g)
    assert np.isfinite(g.item())
