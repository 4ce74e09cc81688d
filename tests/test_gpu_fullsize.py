"""GPU tier at the workloads' full sizes, in the launch configuration the
benchmark times.

  W8A8         16 x 256 x 128, int8 [k, n] weight, fp16 / bf16 / int32 out
  BitLinear    x bf16 [2048, 4096] (1 % outliers x20), RMSNorm eps 1e-6,
               fp32 weight [4096, 4096] -> ternary, bf16 out
  Decode GEMV  M in {1, 4, 16}, K = 8192, N = 28672, bf16 out
  Grouped INT4 fp16 x [32, 4096], uint4 weight [11008, 4096], g = 128 (and 64, 32)
  A4W4         fp16 x, w [8192, 8192], per-tensor scales max|t| / 7

Codes, packed words and per-token scales are compared in full.  Products are
compared in full: the oracle's plain loops where they finish in seconds
(W8A8, decode GEMV, grouped INT4), its float64 library product of the codes
(``oracle.gemm_exact``, exact for these integers) for the BitLinear and
A4W4 products.  The Q4Linear backward is compared on sampled rows and
columns (rows at tile boundaries (127, 128, 255, 256, ...), the last row
and a seeded random set).
"""
import numpy as np
import pytest
import torch

import bit_quantized_linear_quant_amd as ql
import oracle
import synthetic
from parity_util import absmean_rel_tol, assert_equal, assert_float_close, poison, to_np, words

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    ql.lib()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _cuda(t):
    return t.to(DEV).contiguous()


def _rows(m: int, seed: int, extra: int = 40) -> np.ndarray:
    fixed = [r for r in (0, 1, 63, 64, 127, 128, 255, 256, 511, 512, 1023, 1024, m // 2, m - 2, m - 1) if r < m]
    rnd = synthetic.rng(seed).choice(m, size=min(extra, m), replace=False)
    return np.unique(np.concatenate([np.array(fixed, dtype=np.int64), rnd.astype(np.int64)]))


def test_w8a8_full_workload():
    d = synthetic.w8a8()                       # 16 x 256 x 128, weight [k, n]
    acc, y = oracle.w8a8(d["x"].numpy(), d["w"].numpy(), False, d["pts"].numpy(), d["deq"].numpy())
    args = (_cuda(d["x"]), _cuda(d["w"]), ql.QL_W_KN, _cuda(d["deq"]), _cuda(d["pts"]))
    oi = poison((16, 128), torch.int32)
    ql.qlinear_gemm_w8a8(*args, out_dtype=torch.int32, out=oi)
    for dt in (torch.float16, torch.bfloat16):
        o = poison((16, 128), dt)
        ql.qlinear_gemm_w8a8(*args, out_dtype=dt, out=o)
        torch.cuda.synchronize()
        assert_float_close(o, y, f"w8a8 {dt}")
    assert_equal(oi, acc, "w8a8 accumulator")


def test_bitlinear_full_workload():
    m, n, k = 2048, 4096, 4096
    d = synthetic.bitlinear(m, n, k)
    xf = d["x"].float().numpy()
    q_ref, pts_ref, rs_ref = oracle.quant_act(xf, rmsnorm=True, eps_norm=1e-6, eps_q=1e-5)
    codes, gamma = oracle.ternary_quant(d["w"].numpy())
    tol = absmean_rel_tol(n * k)
    assert oracle.ternary_tie_band(d["w"].numpy(), gamma, tol) == 0
    xq, pts, rs = ql.qlinear_quant_act(_cuda(d["x"]), rmsnorm=True, eps_norm=1e-6, eps_q=1e-5)
    packed, g = ql.qlinear_pack_ternary(_cuda(d["w"]), ql.QL_W_NK)
    ob = poison((m, n), torch.bfloat16)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.bfloat16, out=ob)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.int32, out=oi)
    torch.cuda.synchronize()
    assert_equal(xq, q_ref, "activation codes")
    assert_equal(rs, rs_ref, "rowsum")
    np.testing.assert_allclose(to_np(pts), pts_ref, rtol=1e-5)
    assert_equal(words(packed), oracle.pack_ternary(codes), "ternary words")
    assert abs(g.item() - gamma) <= tol * gamma
    acc = oracle.gemm_exact(q_ref, codes, True)
    y = oracle.dequant(acc, pts_ref, np.full(n, np.float32(gamma), np.float32))
    assert_equal(oi, acc, "w2a8 accumulator (every output)")
    assert_float_close(ob, y, "w2a8 bf16 (every output)")


@pytest.fixture(scope="module")
def decode_case():
    n, k = 28672, 8192
    d = synthetic.decode((1, 4, 16), n, k)
    codes, gamma = oracle.ternary_quant(d["w"].numpy())
    packed, g = ql.qlinear_pack_ternary(_cuda(d["w"]), ql.QL_W_NK)
    torch.cuda.synchronize()
    return d, codes, gamma, packed, g


def test_decode_pack_full_workload(decode_case):
    d, codes, gamma, packed, g = decode_case
    tol = absmean_rel_tol(codes.size)
    assert oracle.ternary_tie_band(d["w"].numpy(), gamma, tol) == 0
    assert abs(g.item() - gamma) <= tol * gamma
    assert_equal(words(packed), oracle.pack_ternary(codes), "decode ternary words")


@pytest.mark.parametrize("m", [1, 4, 16])
def test_decode_gemv_full_workload(decode_case, m):
    d, codes, gamma, packed, g = decode_case
    n = codes.shape[0]
    x = d["x"][m]
    q_ref, pts_ref, rs_ref = oracle.quant_act(x.float().numpy(), rmsnorm=True)
    acc, y = oracle.w2a8(q_ref, pts_ref, codes, gamma)
    xq, pts, rs = ql.qlinear_quant_act(_cuda(x), rmsnorm=True)
    ob = poison((m, n), torch.bfloat16)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.bfloat16, out=ob)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.int32, out=oi)
    torch.cuda.synchronize()
    assert_equal(xq, q_ref, "decode activation codes")
    assert_equal(oi, acc, "decode accumulator")
    assert_float_close(ob, y, "decode bf16")


@pytest.mark.parametrize("gs", [128, 64, 32])
def test_grouped_int4_full_workload(gs):
    """32 x 4096 x 11008 at the workload's group size 128 and at 64 and 32 (per-step scales)."""
    d = synthetic.grouped_int4(group_size=gs)
    m, n, k = 32, 11008, 4096
    y, bound = oracle.grouped_int4(d["x"].float().numpy(), d["q"].numpy(), d["s"].float().numpy(),
                                   d["z"].numpy(), gs)
    pw = ql.qlinear_pack_int4(_cuda(d["q"]), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(d["z"]), ql.QL_INT4_ZEROS)
    o16 = poison((m, n), torch.float16)
    ql.qlinear_gemm_w4a8_grouped(_cuda(d["x"]), pw, _cuda(d["s"]), pz, gs, n, out=o16)
    o32 = poison((m, n), torch.float32)
    ql.qlinear_gemm_w4a8_grouped(_cuda(d["x"]), pw, _cuda(d["s"]), pz, gs, n, out_dtype=torch.float32, out=o32)
    torch.cuda.synchronize()
    assert_equal(words(pw), oracle.pack_int4(d["q"].numpy()), "int4 weight words")
    assert_equal(words(pz), oracle.pack_int4_zeros(d["z"].numpy()), "int4 zero words")
    err = np.abs(to_np(o16).astype(np.float64) - y)
    assert np.all(err <= 1e-3 * bound), f"grouped fp16: max err/bound {np.max(err / bound)}"
    assert torch.equal(o16, o32.to(torch.float16))


@pytest.mark.parametrize("gs", [128, 32])
def test_grouped_int4_i8_full_shape(gs):
    """The grouped INT4 weights with int8 activation codes (quantized from the fp16
    activations of the same workload) at 32x4096x11008, g = 128 and 32."""
    d = synthetic.grouped_int4(group_size=gs)
    m, n, k = 32, 11008, 4096
    xq_ref, pts_ref, _ = oracle.quant_act(d["x"].float().numpy())
    y, bound = oracle.grouped_int4_i8(xq_ref, pts_ref, d["q"].numpy(), d["s"].float().numpy(), d["z"].numpy(), gs)
    xq, pts, _ = ql.qlinear_quant_act(_cuda(d["x"]))
    pw = ql.qlinear_pack_int4(_cuda(d["q"]), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(d["z"]), ql.QL_INT4_ZEROS)
    o16 = poison((m, n), torch.float16)
    ql.qlinear_gemm_w4a8_grouped(xq, pw, _cuda(d["s"]), pz, gs, n, out=o16, per_token_scale=pts)
    torch.cuda.synchronize()
    assert_equal(xq, xq_ref, "activation codes")
    err = np.abs(to_np(o16).astype(np.float64) - y)
    assert np.all(err <= 1e-3 * bound), f"grouped int8 fp16: max err/bound {np.max(err / bound)}"


def test_a4w4_full_workload():
    m = n = k = 8192
    d = synthetic.a4w4(m, n, k)
    eps = d["eps"]
    qa = oracle.quant_int4_tensor(d["x"].float().numpy(), d["scale_a"], eps)
    qw = oracle.quant_int4_tensor(d["w"].float().numpy(), d["scale_w"], eps)
    sag = torch.tensor([d["scale_a"]], dtype=torch.float32, device=DEV)
    swg = torch.tensor([d["scale_w"]], dtype=torch.float32, device=DEV)
    out = poison((m, n), torch.float16)
    out, ws = ql.qlinear_gemm_a4w4(_cuda(d["x"]), _cuda(d["w"]), sag, swg, eps, out=out)
    xa, wb = ql.a4w4_operands_from_workspace(ws, m, n, k)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, None, None, out_dtype=torch.int32, out=oi)
    torch.cuda.synchronize()
    assert_equal(xa, oracle.pack_a4w4_fp6(qa), "x operand")
    assert_equal(wb, oracle.pack_a4w4_fp6(qw), "w operand")
    acc = oracle.gemm_exact(qa, qw, True)
    sa = oracle.effective_scale(d["scale_a"], eps)
    sw = oracle.effective_scale(d["scale_w"], eps)
    y = oracle.dequant(acc, np.full(m, sa, np.float32), np.full(n, sw, np.float32))
    assert_equal(oi, acc, "a4w4 accumulator (every output)")
    assert_float_close(out, y, "a4w4 fp16 (every output)")


def test_a4w4_packed_full_workload():
    """The 8192^3 workload on two-codes-per-byte operands: both operands bit for bit, the
    whole fp16 output equal to the FP6-operand product's and, with the accumulator, to the oracle's."""
    m = n = k = 8192
    d = synthetic.a4w4(m, n, k)
    eps = d["eps"]
    qa = oracle.quant_int4_tensor(d["x"].float().numpy(), d["scale_a"], eps)
    qw = oracle.quant_int4_tensor(d["w"].float().numpy(), d["scale_w"], eps)
    sag = torch.tensor([d["scale_a"]], dtype=torch.float32, device=DEV)
    swg = torch.tensor([d["scale_w"]], dtype=torch.float32, device=DEV)
    xg, wg = _cuda(d["x"]), _cuda(d["w"])
    xp = ql.qlinear_quant_a4w4_packed(xg, sag, eps)
    wp = ql.qlinear_quant_a4w4_packed(wg, swg, eps)
    op = poison((m, n), torch.float16)
    ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, sag, swg, eps, out=op)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, None, None, out_dtype=torch.int32, out=oi)
    of, _ = ql.qlinear_gemm_a4w4(xg, wg, sag, swg, eps)
    torch.cuda.synchronize()
    assert_equal(xp, oracle.pack_a4w4_int4(qa), "x packed operand")
    assert_equal(wp, oracle.pack_a4w4_int4(qw), "w packed operand")
    assert torch.equal(op.view(torch.int16), of.view(torch.int16)), "packed vs FP6 operands, whole output"
    acc = oracle.gemm_exact(qa, qw, True)
    sa = oracle.effective_scale(d["scale_a"], eps)
    sw = oracle.effective_scale(d["scale_w"], eps)
    y = oracle.dequant(acc, np.full(m, sa, np.float32), np.full(n, sw, np.float32))
    assert_equal(oi, acc, "a4w4 packed accumulator (every output)")
    assert_float_close(op, y, "a4w4 packed fp16 (every output)")


def test_q4_backward_full_workload():
    """8192^3 backward of the A4W4 workload: sampled rows of grad_x and grad_w against the oracle."""
    m = n = k = 8192
    d = synthetic.a4w4(m, n, k)
    g = torch.from_numpy(synthetic.rng(1006).normal(0, 1, (m, n)).astype(np.float32)).to(torch.float16)
    sag = torch.tensor([d["scale_a"]], dtype=torch.float32, device=DEV)
    swg = torch.tensor([d["scale_w"]], dtype=torch.float32, device=DEV)
    gx, gw, gs = ql.qlinear_q4_backward(_cuda(g), _cuda(d["x"]), _cuda(d["w"]), sag, swg, d["eps"])
    torch.cuda.synchronize()
    x, w, gn = d["x"].float().numpy(), d["w"].float().numpy(), g.float().numpy()
    rows = _rows(m, 2007, extra=8)
    rx = oracle.q4_backward(gn[rows], x[rows], w, d["scale_a"], d["scale_w"], d["eps"])
    cols = _rows(n, 2008, extra=8)
    rw = oracle.q4_backward(gn[:, cols], x, w[cols], d["scale_a"], d["scale_w"], d["eps"])
    u = 2.0 ** -24
    got_x = to_np(gx[torch.from_numpy(rows).to(DEV)]).astype(np.float64)
    assert np.all(np.abs(got_x - rx[0]) <= n * u * rx[3] + 3 * u * np.abs(rx[0]) + 1e-30), "grad_x rows"
    got_w = to_np(gw[torch.from_numpy(cols).to(DEV)]).astype(np.float64)
    assert np.all(np.abs(got_w - rw[1]) <= m * u * rw[4] + 3 * u * np.abs(rw[1]) + 1e-30), "grad_w rows"
    assert np.isfinite(gs.item())

