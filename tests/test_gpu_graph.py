"""GPU tier: the kernels bench.py times through HIP-graph replays give, on every
replay, exactly what the same call gives eagerly.

Each call is captured alone into a graph; between replays the outputs are
cleared by ordinary (eager) device work and the host synchronizes, so a
replay that skipped or repeated work, or depended on state an eager call
left behind, shows up as a difference.  Inputs and outputs are allocated
before capture; nothing inside a captured call allocates.
"""
import numpy as np
import pytest
import torch

import bit_quantized_linear_quant_amd as ql
import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _library():
    ql.lib()  # raises if libqlinear.so is missing: no silent fallback
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _replays_match_eager(call, outs):
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(REPLAYS):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)
    del g


def test_graph_quant_act():
    x = synthetic.activations(64, 4096, seed=901, outliers=0.01, dtype=torch.bfloat16).to(DEV)
    q = torch.empty((64, 4096), dtype=torch.int8, device=DEV)
    pts = torch.empty((64,), dtype=torch.float32, device=DEV)
    rs = torch.empty((64,), dtype=torch.int32, device=DEV)
    _replays_match_eager(lambda: ql.qlinear_quant_act(x, rmsnorm=True, q=q, per_token_scale=pts, rowsum=rs),
                         [q, pts, rs])


@pytest.mark.parametrize("m,n,k", [(1, 4096, 2048), (16, 4096, 4096), (256, 512, 1024)])
def test_graph_w2a8(m, n, k):
    """Decode GEMV (one and sixteen rows) and the large-tile product."""
    d = synthetic.bitlinear(m, n, k, seed=902)
    packed, gamma = ql.qlinear_pack_ternary(d["w"].to(DEV), ql.QL_W_NK)
    xq, pts, rs = ql.qlinear_quant_act(d["x"].to(DEV), rmsnorm=True)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    _replays_match_eager(lambda: ql.qlinear_gemm_w2a8(xq, pts, rs, packed, gamma, n, out=out), [out])


@pytest.mark.parametrize("int8_codes", [False, True])
def test_graph_grouped_int4(int8_codes):
    m, n, k, g = 32, 2048, 1024, 128
    d = synthetic.grouped_int4(m, n, k, group_size=g, seed=903)
    pw = ql.qlinear_pack_int4(d["q"].to(DEV), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(d["z"].to(DEV), ql.QL_INT4_ZEROS)
    sc = d["s"].to(DEV)
    out = torch.empty((m, n), dtype=torch.float16, device=DEV)
    if int8_codes:
        xq, pts, _ = ql.qlinear_quant_act(d["x"].to(DEV))
        call = lambda: ql.qlinear_gemm_w4a8_grouped(xq, pw, sc, pz, g, n, out=out, per_token_scale=pts)
    else:
        x = d["x"].to(DEV)
        call = lambda: ql.qlinear_gemm_w4a8_grouped(x, pw, sc, pz, g, n, out=out)
    _replays_match_eager(call, [out])


def test_graph_w8a8_kn_decode():
    d = synthetic.w8a8()          # 16 x 256 x 128, weight [k, n]
    x, w = d["x"].to(DEV), d["w"].to(DEV)
    deq, pts = d["deq"].to(DEV), d["pts"].to(DEV)
    out = torch.empty((16, 128), dtype=torch.float16, device=DEV)
    _replays_match_eager(lambda: ql.qlinear_gemm_w8a8(x, w, ql.QL_W_KN, deq, pts, out=out), [out])


def test_graph_hbm_read_stream_reads_once_per_replay():
    """Each replay XORs every word into the sink once: the sink alternates
    between the eager result and its starting value."""
    buf = torch.randint(0, 256, (4 << 20,), dtype=torch.uint8, device=DEV)
    sink = torch.zeros((ql.QL_HBM_STREAM_SINK_WORDS,), dtype=torch.int64, device=DEV)
    ql.qlinear_hbm_read_stream(buf, sink)
    torch.cuda.synchronize()
    once = sink.clone()
    assert int(np.bitwise_xor.reduce(once.cpu().numpy() & 0xffffffff)) == \
        int(np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32)))
    sink.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ql.qlinear_hbm_read_stream(buf, sink)
    for rep in range(1, REPLAYS + 1):
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sink, once if rep % 2 == 1 else torch.zeros_like(sink))
    del g
