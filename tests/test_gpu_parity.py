"""GPU tier: every C entry point against the CPU oracle, element by element.

Sizes are ones the oracle finishes in seconds while still spanning several
kernel tiles and a ragged tail; edge cases cover the smallest shapes, k not a
multiple of the vector width, the largest k the int32 accumulator allows, and
the degenerate inputs of each quantizer.  Every call goes through the C ABI
(ctypes) of libqlinear; outputs are poisoned first so an unwritten element
fails.
"""
import numpy as np
import pytest
import torch

import bit_quantized_linear_quant_amd as ql
import oracle
import synthetic
from parity_util import (TOL_REL, absmean_rel_tol, assert_equal, assert_float_close, poison, rms_pts_rel_tol,
                         to_np, words)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    ql.lib()  # raises if libqlinear.so is missing: no silent fallback
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _cuda(t):
    return t.to(DEV).contiguous()


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# W8A8 per-token product
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16, torch.int32])
def test_worked_example(out_dtype):
    ex = synthetic.worked_example()
    out = poison((2, 3), out_dtype)
    ql.qlinear_gemm_w8a8(_cuda(ex["x"]), _cuda(ex["w"]), ql.QL_W_KN, _cuda(ex["deq"]), _cuda(ex["pts"]),
                         out_dtype=out_dtype, out=out)
    _sync()
    want = [[9, 12, 15], [19, 26, 33]] if out_dtype == torch.int32 else [[9, 24, 45], [38, 104, 198]]
    assert to_np(out).tolist() == want


W8A8_SHAPES = [
    (16, 128, 256, False),     # the per-token W8A8 workload
    (1, 1, 1, False),
    (2, 3, 2, True),
    (300, 270, 200, True),
    (129, 257, 1000, False),
    (77, 45, 77, True),        # k not a multiple of 16: byte loads
    (33, 50, 77, False),
    (256, 256, 64, True),
    (130, 131, 4096, True),
    (512, 512, 64, True),      # m, n >= 512 but fewer than 128 tiles of 256 x 256: 128 x 128 kernel
    (520, 777, 192, True),     # ragged m and n
    (1024, 768, 1024, True),
    (2048, 4096, 64, True),    # at least 128 tiles of 256 x 256: the direct-to-LDS kernel
    (2100, 4000, 128, True),   # the same, ragged m and n
    (700, 600, 120, True),     # k % 64 != 0: general kernel at large m, n
    (1, 400, 512, True),       # decode kernel from here on (m <= 16, [n][k], k % 64 == 0)
    (5, 270, 320, True),       # k blocks cut short, n % 16 != 0
    (16, 1000, 768, True),
    (4, 6400, 256, True),      # 128-k register stages (more than 384 column blocks)
    (2, 13000, 128, True),     # n % 16 != 0 with 128-k stages
    (3, 28672, 64, True),      # a single k step
    (17, 400, 512, True),      # decode kernel with two to four 16-row blocks
    (33, 1000, 768, True),
    (64, 6400, 256, True),     # four column blocks per workgroup
    (48, 13000, 128, True),    # four column blocks per workgroup, the last one past n
    (20, 6400, 384, True),     # two row blocks, 128-k whole-line stages, more than 384 column blocks
    (27, 5000, 320, True),     # the same shape class with k % 128 != 0 (64-k stages), n % 16 != 0
    (96, 400, 512, True),      # six and eight row blocks (m <= 128, few columns)
    (128, 1000, 768, True),
    (100, 6400, 128, True),    # many columns: back to the 128x128 tiles
    (1, 4, 64, False),         # [k][n] decode kernel from here on (m <= 64, k % 64 == 0, n % 4 == 0)
    (5, 1004, 320, False),     # n % 16 != 0, k steps not a multiple of the waves, ragged XCD groups
    (33, 3000, 768, False),    # three row blocks
    (64, 2048, 4096, False),   # four row blocks, long k
    (48, 260, 128, False),
    (16, 16384, 256, False),   # 64-column groups with 16-byte row loads (n / 64 >= 256)
    (33, 16400, 128, False),   # the same, last column group partly past n
    (64, 16384, 320, False),   # the same with four row blocks, k steps not a multiple of the waves
    (16, 128, 200, False),     # k % 64 != 0 and n % 4 != 0: general kernel
    (9, 130, 256, False),
]


@pytest.mark.parametrize("m,n,k,nk", W8A8_SHAPES)
def test_w8a8_parity(m, n, k, nk):
    d = synthetic.w8a8(m, n, k, nk, seed=100 + m + n + k)
    x, w, deq, pts = (d[key] for key in ("x", "w", "deq", "pts"))
    acc, y = oracle.w8a8(x.numpy(), w.numpy(), nk, pts.numpy(), deq.numpy())
    layout = ql.QL_W_NK if nk else ql.QL_W_KN
    xg, wg, dg, pg = _cuda(x), _cuda(w), _cuda(deq), _cuda(pts)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_w8a8(xg, wg, layout, None, None, out_dtype=torch.int32, out=oi)
    for dt in (torch.float16, torch.bfloat16):
        o = poison((m, n), dt)
        ql.qlinear_gemm_w8a8(xg, wg, layout, dg, pg, out_dtype=dt, out=o)
        _sync()
        assert_float_close(o, y, f"w8a8 {dt}")
    assert_equal(oi, acc, "w8a8 int32 accumulator")


def test_w8a8_max_k_extremes():
    """k = 131071 with every operand -128: the largest accumulator the ABI allows."""
    m, n, k = 3, 5, 131071
    x = torch.full((m, k), -128, dtype=torch.int8)
    w = torch.full((n, k), -128, dtype=torch.int8)
    w[1, ::2] = 127
    acc = oracle.gemm_i8(x.numpy(), w.numpy(), True)
    assert int(acc[0, 0]) == 128 * 128 * k
    o = poison((m, n), torch.int32)
    ql.qlinear_gemm_w8a8(_cuda(x), _cuda(w), ql.QL_W_NK, None, None, out_dtype=torch.int32, out=o)
    _sync()
    assert_equal(o, acc, "w8a8 max-k accumulator")


def test_w8a8_decode_max_k():
    """The decode kernel at k = 131008 (the largest multiple of 64 the ABI allows), operands at -128."""
    m, n, k = 3, 5, 131008
    x = torch.full((m, k), -128, dtype=torch.int8)
    w = torch.full((n, k), -128, dtype=torch.int8)
    w[1, ::2] = 127
    x[2, 1::3] = 5
    acc = oracle.gemm_i8(x.numpy(), w.numpy(), True)
    assert int(acc[0, 0]) == 128 * 128 * k
    o = poison((m, n), torch.int32)
    ql.qlinear_gemm_w8a8(_cuda(x), _cuda(w), ql.QL_W_NK, None, None, out_dtype=torch.int32, out=o)
    _sync()
    assert_equal(o, acc, "w8a8 decode max-k accumulator")


def test_w8a8_decode_kn_max_k():
    """The [k][n] decode kernel at k = 131008, operands at -128 (and a few larger codes)."""
    m, n, k = 3, 8, 131008
    x = torch.full((m, k), -128, dtype=torch.int8)
    w = torch.full((k, n), -128, dtype=torch.int8)
    w[::2, 1] = 127
    x[2, 1::3] = 5
    acc = oracle.gemm_i8(x.numpy(), w.numpy(), False)
    assert int(acc[0, 0]) == 128 * 128 * k
    o = poison((m, n), torch.int32)
    ql.qlinear_gemm_w8a8(_cuda(x), _cuda(w), ql.QL_W_KN, None, None, out_dtype=torch.int32, out=o)
    _sync()
    assert_equal(o, acc, "w8a8 [k][n] decode max-k accumulator")


def test_w8a8_deterministic():
    d = synthetic.w8a8(200, 300, 512, True, seed=5)
    args = [_cuda(d[key]) for key in ("x", "w")]
    o1 = ql.qlinear_gemm_w8a8(*args, ql.QL_W_NK, _cuda(d["deq"]), _cuda(d["pts"]))
    o2 = ql.qlinear_gemm_w8a8(*args, ql.QL_W_NK, _cuda(d["deq"]), _cuda(d["pts"]))
    _sync()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("batch,m,n,k,nk,per_batch_deq", [
    (3, 16, 128, 256, False, False),    # the per-token W8A8 workload, batched
    (4, 300, 270, 200, True, True),
    (2, 520, 777, 192, True, False),
    (2, 2048, 2080, 64, True, True),    # 2 x 72 tiles of 256 x 256: the direct-to-LDS kernel
    (3, 512, 512, 128, True, True),
    (5, 77, 45, 77, True, True),        # byte loads
    (2, 33, 50, 77, False, False),
    (2, 1, 1, 1, False, True),
    (3, 16, 270, 320, True, True),      # decode kernel
    (2, 40, 900, 192, True, False),     # decode kernel, three row blocks
    (2, 40, 900, 192, False, True),     # [k][n] decode kernel, three row blocks
])
def test_w8a8_batched_parity(batch, m, n, k, nk, per_batch_deq):
    ds = [synthetic.w8a8(m, n, k, nk, seed=1900 + 10 * b + m + n + k) for b in range(batch)]
    x = torch.stack([d["x"] for d in ds])
    w = torch.stack([d["w"] for d in ds])
    pts = torch.stack([d["pts"] for d in ds])
    deq = torch.stack([d["deq"] for d in ds]) if per_batch_deq else ds[0]["deq"]
    b = synthetic.bias(n, 1.0, seed=2000 + n)
    acc, y = oracle.w8a8_batched(x.numpy(), w.numpy(), nk, pts.numpy(), deq.numpy())
    layout = ql.QL_W_NK if nk else ql.QL_W_KN
    args = (_cuda(x), _cuda(w), layout, _cuda(deq), _cuda(pts))
    oi = poison((batch, m, n), torch.int32)
    ql.qlinear_gemm_w8a8_batched(args[0], args[1], layout, None, None, out_dtype=torch.int32, out=oi)
    outs = {}
    for dt in (torch.float16, torch.bfloat16):
        outs[dt] = poison((batch, m, n), dt)
        ql.qlinear_gemm_w8a8_batched(*args, out_dtype=dt, out=outs[dt])
    ob = poison((batch, m, n), torch.float16)
    ql.qlinear_gemm_w8a8_batched(*args, out_dtype=torch.float16, out=ob, bias=_cuda(b))
    _sync()
    assert_equal(oi, acc, "batched int32 accumulator")
    for dt, o in outs.items():
        assert_float_close(o, y, f"batched {dt}")
    yb = np.stack([oracle.add_bias(y[i], b.numpy()) for i in range(batch)])
    assert_float_close(ob, yb, "batched + bias", extra=np.stack([_bias_tol(y[i], b.numpy()) for i in range(batch)]))


# ---------------------------------------------------------------------------
# Per-token activation quantization
# ---------------------------------------------------------------------------
# (rows of whole 8-element chunks up to 8192 run W = 4, 2 or 1 waves per row
# by the launch's size; the ragged ones leave a split row's last waves
# partly or wholly past the row)
QUANT_SHAPES = [(1, 8192), (16, 8192), (7, 4097), (33, 77), (5, 1), (3, 20000), (64, 4096), (2, 8),
                (40, 1000), (9, 2056), (3, 6144)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("m,k", QUANT_SHAPES)
def test_quant_act_parity(dtype, rms, m, k):
    x = synthetic.activations(m, k, seed=200 + m * 7 + k, outliers=0.01, dtype=dtype)
    q_ref, pts_ref, rs_ref = oracle.quant_act(x.float().numpy(), rmsnorm=rms, eps_norm=1e-6, eps_q=1e-5)
    q = poison((m, k), torch.int8)
    pts = poison((m,), torch.float32)
    rs = poison((m,), torch.int32)
    ql.qlinear_quant_act(_cuda(x), rmsnorm=rms, eps_norm=1e-6, eps_q=1e-5, q=q, per_token_scale=pts,
                         rowsum=rs)
    _sync()
    assert_equal(q, q_ref, "codes")
    assert_equal(rs, rs_ref, "rowsum")
    if rms:
        np.testing.assert_allclose(to_np(pts).astype(np.float64), pts_ref.astype(np.float64),
                                   rtol=rms_pts_rel_tol(k), atol=0)
    else:
        assert_equal(pts, pts_ref, "per-token scale")


@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("m,k", [(4096, 4096), (4097, 4096), (4096, 3592), (8192, 4096), (8193, 4096), (4096, 3584), (5000, 8192)])
def test_quant_act_split_routes(rms, m, k):
    """Launch sizes around the switch from four to two to one waves per row."""
    x = synthetic.activations(m, k, seed=250 + m + k, outliers=0.01, dtype=torch.bfloat16)
    q_ref, pts_ref, rs_ref = oracle.quant_act(x.float().numpy(), rmsnorm=rms, eps_norm=1e-6, eps_q=1e-5)
    q, pts, rs = ql.qlinear_quant_act(_cuda(x), rmsnorm=rms, eps_norm=1e-6, eps_q=1e-5)
    _sync()
    assert_equal(q, q_ref, "codes")
    assert_equal(rs, rs_ref, "rowsum")
    if rms:
        np.testing.assert_allclose(to_np(pts).astype(np.float64), pts_ref.astype(np.float64),
                                   rtol=rms_pts_rel_tol(k), atol=0)
    else:
        assert_equal(pts, pts_ref, "per-token scale")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [96, 4096, 4097])
def test_quant_act_rmsnorm_guard_on_tiny_rows(dtype, k):
    """Rows whose normalized absmax falls below eps_q: the guard acts on r * max|x|.

    Where r * a >= eps_q the codes are those of x (bit-exact).  Below it the
    codes are rne(x * 127 / (eps_q / r)) and depend on the RMSNorm factor r,
    which the kernel computes in fp32 and the oracle in fp64: they may differ
    by one only where x * 127 r / eps_q lies within 1e-4 of a rounding tie.
    """
    rng = np.random.default_rng(k)
    scales = [1.0, 1e-6, 3e-8, 1e-9, 1e-10, 1e-12, 0.0]
    rows = [rng.standard_normal(k) * s for s in scales]
    rows.append(np.full(k, 1e-6) * np.sign(rng.standard_normal(k)))
    x = torch.tensor(np.stack(rows), dtype=torch.float32).to(dtype)
    xf = x.float().numpy()
    q_ref, pts_ref, rs_ref = oracle.quant_act(xf, rmsnorm=True, eps_norm=1e-6, eps_q=1e-5)
    q, pts, rs = ql.qlinear_quant_act(_cuda(x), rmsnorm=True, eps_norm=1e-6, eps_q=1e-5)
    _sync()
    xd = xf.astype(np.float64)
    r = 1.0 / np.sqrt((xd * xd).mean(axis=1) + 1e-6)
    ar = np.abs(xd).max(axis=1) * r
    g = q.cpu().numpy()
    assert np.all(np.abs(g[-1]) == 127)  # the +-1e-6 row is far above the guard after the norm
    for i in range(x.shape[0]):
        if ar[i] >= 1e-5 * (1 + 1e-4):
            assert_equal(g[i], q_ref[i], f"codes of row {i}")
        else:
            v = np.abs(xd[i] * 127.0 * r[i] / 1e-5)
            tie = np.abs(v - np.floor(v) - 0.5) < 1e-4
            diff = g[i].astype(np.int32) - q_ref[i].astype(np.int32)
            assert np.all((diff == 0) | (tie & (np.abs(diff) == 1))), f"codes of row {i}"
    assert_equal(rs, g.astype(np.int64).sum(axis=1).astype(np.int32), "rowsum")
    np.testing.assert_allclose(to_np(pts).astype(np.float64), pts_ref.astype(np.float64),
                               rtol=rms_pts_rel_tol(k), atol=0)


def test_quant_act_degenerate_rows():
    x = torch.zeros(4, 300, dtype=torch.bfloat16)
    x[1, 17] = -3.5
    x[2, :] = 2.0
    x[3, 5] = 1e-30  # below eps_q: scale guarded
    q_ref, pts_ref, rs_ref = oracle.quant_act(x.float().numpy())
    q, pts, rs = ql.qlinear_quant_act(_cuda(x))
    _sync()
    assert_equal(q, q_ref, "codes")
    assert_equal(pts, pts_ref, "pts")
    assert_equal(rs, rs_ref, "rowsum")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("count", [1, 7, 8, 1000, 65537])
@pytest.mark.parametrize("scale_mul", [1.0, 0.25, 0.0])
def test_quant_int4_tensor_parity(dtype, count, scale_mul):
    x = synthetic.activations(1, count, seed=300 + count, dtype=dtype).reshape(count)
    scale = float(np.float32(x.abs().max().float().item()) / np.float32(7.0)) * scale_mul
    ref = oracle.quant_int4_tensor(x.float().numpy(), scale, 1e-5)
    q = poison((count,), torch.int8)
    ql.qlinear_quant_int4_tensor(_cuda(x), torch.tensor([scale], dtype=torch.float32, device=DEV), 1e-5, q=q)
    _sync()
    assert_equal(q, ref, "int4 codes")


# ---------------------------------------------------------------------------
# Packs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,k", [(16, 256), (48, 768), (400, 512)])
@pytest.mark.parametrize("nk", [True, False])
def test_pack_ternary_parity(n, k, nk):
    w = synthetic.master_weight(n, k, seed=400 + n + k)
    wl = w if nk else w.t().contiguous()
    codes, gamma = oracle.ternary_quant(wl.numpy(), layout_nk=nk)
    tol = absmean_rel_tol(n * k)
    assert oracle.ternary_tie_band(w.numpy(), gamma, tol) == 0
    ref = oracle.pack_ternary(codes)
    layout = ql.QL_W_NK if nk else ql.QL_W_KN
    packed = poison((n * k // 16,), torch.int32)
    wg = _cuda(wl)
    p1, g1 = ql.qlinear_pack_ternary(wg, layout, packed=packed)
    p2, g2 = ql.qlinear_pack_ternary(wg, layout)
    _sync()
    assert_equal(words(p1), ref, "ternary words")
    assert abs(g1.item() - gamma) <= tol * gamma
    assert torch.equal(p1, p2) and torch.equal(g1.view(torch.int64), g2.view(torch.int64))


def test_pack_ternary_eps_guard():
    w = torch.zeros(32, 256)
    packed, g = ql.qlinear_pack_ternary(_cuda(w), ql.QL_W_NK, eps=1e-5)
    _sync()
    assert g.item() == 1e-5
    assert_equal(words(packed), oracle.pack_ternary(np.zeros((32, 256), np.int8)), "zero weight words")


@pytest.mark.parametrize("n,k", [(16, 128), (48, 384), (400, 512)])
def test_pack_int4_parity(n, k):
    d = synthetic.grouped_int4(1, n, k, 128, seed=500 + n)
    hi = torch.from_numpy(synthetic.rng(501 + n).integers(0, 16, tuple(d["q"].shape), dtype=np.uint8))
    q = d["q"] | hi * 16  # high nibbles are ignored
    ref = oracle.pack_int4(q.numpy())
    out = poison((n * k // 8,), torch.int32)
    ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT, packed=out)
    zref = oracle.pack_int4_zeros(d["z"].numpy())
    zout = ql.qlinear_pack_int4(_cuda(d["z"]), ql.QL_INT4_ZEROS)
    _sync()
    assert_equal(words(out), ref, "int4 weight words")
    assert_equal(words(zout), zref, "int4 zero words")


# ---------------------------------------------------------------------------
# BitLinear: quant_act -> pack_ternary -> w2a8
# ---------------------------------------------------------------------------
# m >= 256 takes the large-tile kernel: one exact tile with fewer 128-k
# slices than ring stages, ragged m and n over several tiles, a longer k.
# m <= 64 takes the decode kernel with one to four 16-row blocks and one,
# three or four column blocks per workgroup (the last past n).
W2A8_SHAPES = [(1, 400, 512), (2, 256, 768), (4, 400, 512), (5, 64, 256), (16, 400, 768), (17, 400, 512),
               (33, 400, 768), (64, 6400, 512), (40, 20000, 256), (64, 16400, 256),
               (130, 256, 768), (300, 400, 512), (256, 128, 256), (513, 272, 1280), (600, 528, 2304),
               # 4 < m <= 64 with k >= 2048: x through LDS in whole lines, one to four row blocks
               (12, 400, 2048), (20, 400, 2048), (33, 1008, 4096), (48, 6400, 2304), (64, 16400, 2048),
               # 64 < m <= 96 with k >= 2048: six row blocks on four waves
               (65, 400, 2048), (96, 1008, 2304),
               # 96 < m <= 128, k >= 2048, at most 768 column blocks: two decode launches
               (100, 400, 2048), (128, 1008, 4096),
               # 64 < m <= 128 with more than 1024 column blocks or k < 2048: the 128x256 tiles
               # (one tile row, ragged), also 128 < m < 256 (two tile rows)
               (96, 16400, 2048), (120, 16400, 2048), (80, 400, 1024), (128, 272, 256), (65, 64, 512),
               (200, 528, 768), (112, 13312, 2048),
               # 4 < m <= 16, 2048 <= k <= 8192: every k block of a wave loaded at the start
               (9, 1008, 8192), (16, 48, 2304), (5, 400, 4096)]


@pytest.mark.parametrize("m,n,k", W2A8_SHAPES)
def test_w2a8_parity(m, n, k):
    d = synthetic.bitlinear(m, n, k, seed=600 + m + n)
    x, w = d["x"], d["w"]
    xq_ref, pts_ref, rs_ref = oracle.quant_act(x.float().numpy(), rmsnorm=True)
    codes, gamma = oracle.ternary_quant(w.numpy())
    acc_ref, y_ref = oracle.w2a8(xq_ref, pts_ref, codes, gamma)
    xq, pts, rs = ql.qlinear_quant_act(_cuda(x), rmsnorm=True)
    packed, g = ql.qlinear_pack_ternary(_cuda(w), ql.QL_W_NK)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.int32, out=oi)
    ob = poison((m, n), torch.bfloat16)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.bfloat16, out=ob)
    of = poison((m, n), torch.float16)
    ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=torch.float16, out=of)
    _sync()
    assert_equal(xq, xq_ref, "activation codes")
    assert_equal(words(packed), oracle.pack_ternary(codes), "ternary words")
    assert_equal(oi, acc_ref, "w2a8 accumulator")
    assert_float_close(ob, y_ref, "w2a8 bf16")
    assert_float_close(of, y_ref, "w2a8 fp16")


def test_w2a8_gemv_deterministic():
    d = synthetic.bitlinear(16, 512, 1024, seed=7)
    xq, pts, rs = ql.qlinear_quant_act(_cuda(d["x"]), rmsnorm=True)
    packed, g = ql.qlinear_pack_ternary(_cuda(d["w"]), ql.QL_W_NK)
    a = ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, 512)
    b = ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, 512)
    _sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# Grouped affine INT4
# ---------------------------------------------------------------------------
GROUPED_SHAPES = [(1, 48, 256, 128), (5, 400, 512, 128), (32, 400, 512, 256),
                  (40, 64, 384, 128), (32, 16, 128, 128), (3, 32, 1024, 1024),
                  (5, 64, 8192, 256),    # more than 4 k blocks per wave: pipelined stages
                  # groups smaller than a 128-k block: per-step scales after the cross-row transpose
                  (1, 48, 256, 32), (5, 400, 512, 32), (32, 400, 512, 64), (17, 64, 384, 96),
                  (3, 32, 1024, 64), (40, 64, 8192, 32), (16, 48, 128, 32), (33, 160, 640, 160),
                  # four k blocks per wave with one scale and zero-point pair per column block and
                  # lane: whole rounds, and a last round whose blocks past k are clamped and masked
                  (32, 400, 4096, 128), (48, 160, 2560, 256), (7, 96, 2816, 128), (16, 400, 4096, 512),
                  (32, 48, 2304, 2304)]


@pytest.mark.parametrize("m,n,k,g", GROUPED_SHAPES)
def test_grouped_int4_parity(m, n, k, g):
    d = synthetic.grouped_int4(m, n, k, g, seed=700 + m + n + k)
    x, q, s, z = d["x"], d["q"], d["s"], d["z"]
    y, bound = oracle.grouped_int4(x.float().numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    o32 = poison((m, n), torch.float32)
    ql.qlinear_gemm_w4a8_grouped(_cuda(x), pw, _cuda(s), pz, g, n, out_dtype=torch.float32, out=o32)
    o16 = poison((m, n), torch.float16)
    ql.qlinear_gemm_w4a8_grouped(_cuda(x), pw, _cuda(s), pz, g, n, out_dtype=torch.float16, out=o16)
    _sync()
    for o, name in ((o32, "fp32"), (o16, "fp16")):
        err = np.abs(to_np(o).astype(np.float64) - y)
        assert np.all(err <= 1e-3 * bound), f"grouped {name}: max err/bound {np.max(err / bound)}"
    # the fp16 output is the fp32 output rounded once to nearest even
    assert torch.equal(o16, o32.to(torch.float16))


@pytest.mark.parametrize("g", [128, 32, 64])
def test_grouped_int4_zero_point_equals_code_gives_zero(g):
    m, n, k = 4, 32, 256
    d = synthetic.grouped_int4(m, n, k, g, seed=9)
    z = d["z"]
    q = torch.repeat_interleave(z, g, dim=1).contiguous()
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    o = ql.qlinear_gemm_w4a8_grouped(_cuda(d["x"]), pw, _cuda(d["s"]), pz, g, n, out_dtype=torch.float32)
    _sync()
    assert torch.count_nonzero(o).item() == 0


def _grouped_i8_inputs(m, n, k, g, seed):
    d = synthetic.grouped_int4(m, n, k, g, seed=seed)
    r = synthetic.rng(seed + 17)
    xq = torch.from_numpy(r.integers(-127, 128, (m, k), dtype=np.int8))
    pts = torch.from_numpy(r.uniform(1e-3, 1e-2, m).astype(np.float32))
    return xq, pts, d["q"], d["s"], d["z"]


@pytest.mark.parametrize("m,n,k,g", [(1, 48, 256, 128), (5, 400, 512, 128), (16, 64, 256, 128),
                                     (17, 400, 512, 256), (32, 400, 512, 128), (40, 64, 384, 128),
                                     (3, 32, 1024, 1024), (17, 64, 8192, 128),
                                     (1, 48, 256, 32), (17, 400, 512, 64), (32, 400, 512, 32),
                                     (5, 64, 384, 96), (17, 64, 8192, 32), (16, 48, 1024, 64),
                                     # four k blocks per wave, shared scale and zero-point pairs
                                     (32, 400, 4096, 128), (48, 160, 2560, 256), (7, 96, 2816, 128),
                                     (16, 400, 4096, 512)])
def test_grouped_int4_i8_parity(m, n, k, g):
    """int8 activation codes: fp32 output within the arithmetic's bound, 16-bit outputs
    within the grouped bar and equal to the fp32 output rounded once."""
    xq, pts, q, s, z = _grouped_i8_inputs(m, n, k, g, seed=900 + m + n + k)
    y, bound = oracle.grouped_int4_i8(xq.numpy(), pts.numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    outs = {}
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        o = poison((m, n), dt)
        ql.qlinear_gemm_w4a8_grouped(_cuda(xq), pw, _cuda(s), pz, g, n, out_dtype=dt, out=o,
                                     per_token_scale=_cuda(pts))
        outs[dt] = o
    _sync()
    # exact int32 partials (per 128-k block, or per 32-k step for smaller groups); each is
    # scaled and added with one fp32 fma, the waves' partials are added (7 adds) and pts
    # multiplies once: at most k/step + 9 roundings of partial sums bounded by `bound`
    step = 128 if g % 128 == 0 else 32
    err32 = np.abs(to_np(outs[torch.float32]).astype(np.float64) - y)
    tol32 = (k // step + 9) * 2.0 ** -24 * bound
    assert np.all(err32 <= tol32 + 1e-30), f"fp32: max err/tol {np.max(err32 / tol32)}"
    for dt in (torch.float16, torch.bfloat16):
        err = np.abs(to_np(outs[dt]).astype(np.float64) - y)
        assert np.all(err <= 1e-3 * bound), f"{dt}: max err/bound {np.max(err / bound)}"
        assert torch.equal(outs[dt], outs[torch.float32].to(dt))


@pytest.mark.parametrize("batch,m,n,k,g,int8_codes,with_bias", [
    (3, 5, 400, 512, 128, False, False), (2, 33, 160, 768, 256, False, True),
    (3, 16, 128, 256, 128, True, False), (2, 40, 64, 384, 128, True, True),
    (2, 17, 160, 256, 32, True, True), (2, 9, 64, 512, 64, False, False)])
def test_grouped_int4_batched_parity(batch, m, n, k, g, int8_codes, with_bias):
    """Every slice within the grouped bar of the oracle, and bit-equal to a separate
    non-batched call on that slice."""
    ds = [synthetic.grouped_int4(m, n, k, g, seed=1100 + 7 * b + m) for b in range(batch)]
    q = torch.stack([d["q"] for d in ds])
    s = torch.stack([d["s"] for d in ds])
    z = torch.stack([d["z"] for d in ds])
    if int8_codes:
        r = synthetic.rng(1200 + m)
        x = torch.from_numpy(r.integers(-127, 128, (batch, m, k), dtype=np.int8))
        pts = torch.from_numpy(r.uniform(1e-3, 1e-2, (batch, m)).astype(np.float32))
        y, bound = oracle.grouped_int4_batched(x.numpy(), q.numpy(), s.float().numpy(), z.numpy(), g,
                                               pts=pts.numpy())
    else:
        x = torch.stack([d["x"] for d in ds])
        pts = None
        y, bound = oracle.grouped_int4_batched(x.float().numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    bias = torch.from_numpy(synthetic.rng(1300 + m).uniform(-1, 1, (batch, n)).astype(np.float32)) \
        if with_bias else None
    pw = torch.stack([ql.qlinear_pack_int4(_cuda(q[b]), ql.QL_INT4_WEIGHT) for b in range(batch)])
    pz = torch.stack([ql.qlinear_pack_int4(_cuda(z[b]), ql.QL_INT4_ZEROS) for b in range(batch)])
    cp = _cuda(pts) if int8_codes else None
    cb = _cuda(bias) if with_bias else None
    o = poison((batch, m, n), torch.float32)
    ql.qlinear_gemm_w4a8_grouped_batched(_cuda(x), pw, _cuda(s), pz, g, n, out_dtype=torch.float32, out=o,
                                         per_token_scale=cp, bias=cb)
    singles = [ql.qlinear_gemm_w4a8_grouped(_cuda(x[b]), pw[b], _cuda(s[b]), pz[b], g, n,
                                            out_dtype=torch.float32,
                                            per_token_scale=None if cp is None else cp[b].clone(),
                                            bias=None if cb is None else cb[b].clone()) for b in range(batch)]
    _sync()
    for b in range(batch):
        assert torch.equal(o[b], singles[b]), f"slice {b} differs from its separate call"
    ref = y + (bias.numpy().astype(np.float64)[:, None, :] if with_bias else 0.0)
    err = np.abs(to_np(o).astype(np.float64) - ref)
    tol = 1e-3 * bound + (2.0 ** -23 * np.abs(ref) if with_bias else 0.0)
    assert np.all(err <= tol), f"batched grouped: max err/bound {np.max(err / bound)}"


@pytest.mark.parametrize("g", [128, 32, 64])
def test_grouped_int4_i8_zero_point_equals_code_gives_zero(g):
    m, n, k = 4, 32, 256
    xq, pts, _, s, z = _grouped_i8_inputs(m, n, k, g, seed=19)
    q = torch.repeat_interleave(z, g, dim=1).contiguous()
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    o = ql.qlinear_gemm_w4a8_grouped(_cuda(xq), pw, _cuda(s), pz, g, n, out_dtype=torch.float32,
                                     per_token_scale=_cuda(pts))
    _sync()
    assert torch.count_nonzero(o).item() == 0


@pytest.mark.parametrize("g", [128, 32])
def test_grouped_int4_i8_extreme_codes(g):
    """All activation codes -127 or 127 and all weight codes 0 or 15 with zero-point 0 or 15."""
    m, n, k = 16, 32, 512
    r = synthetic.rng(23)
    xq = torch.from_numpy(np.where(r.random((m, k)) < 0.5, -127, 127).astype(np.int8))
    q = torch.from_numpy(np.where(r.random((n, k)) < 0.5, 0, 15).astype(np.uint8))
    z = torch.from_numpy(np.where(r.random((n, k // g)) < 0.5, 0, 15).astype(np.uint8))
    s = torch.ones((n, k // g), dtype=torch.float16)
    pts = torch.ones(m, dtype=torch.float32)
    y, _ = oracle.grouped_int4_i8(xq.numpy(), pts.numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    o = ql.qlinear_gemm_w4a8_grouped(_cuda(xq), pw, _cuda(s), pz, g, n, out_dtype=torch.float32,
                                     per_token_scale=_cuda(pts))
    _sync()
    # every term is an integer and the sums stay below 2^24: exact in fp32
    assert np.array_equal(to_np(o).astype(np.float64), y)


# ---------------------------------------------------------------------------
# Optional bias: fp32 [n] added to the dequantized fp32 value, then rounded
# ---------------------------------------------------------------------------
def _bias_tol(y, b):
    """Extra bound of a biased output: two fp32 roundings of the dequant and one of the add."""
    return 2.0 ** -22 * (np.abs(y) + np.abs(b.astype(np.float64))[None, :])


@pytest.mark.parametrize("m,n,k,nk", [(300, 270, 200, True), (77, 45, 77, True), (129, 257, 1000, False),
                                      (520, 777, 192, True), (1024, 768, 1024, True), (1, 1, 1, False),
                                      (5, 300, 256, True), (40, 300, 256, True), (16, 128, 256, False),
                                      (40, 300, 256, False)])
def test_w8a8_bias_parity(m, n, k, nk):
    d = synthetic.w8a8(m, n, k, nk, seed=1200 + m + n + k)
    x, w, deq, pts = (d[key] for key in ("x", "w", "deq", "pts"))
    b = synthetic.bias(n, 1.0, seed=1300 + n)
    _, y = oracle.w8a8(x.numpy(), w.numpy(), nk, pts.numpy(), deq.numpy())
    yb = oracle.add_bias(y, b.numpy())
    layout = ql.QL_W_NK if nk else ql.QL_W_KN
    args = (_cuda(x), _cuda(w), layout, _cuda(deq), _cuda(pts))
    for dt in (torch.float16, torch.bfloat16):
        o = poison((m, n), dt)
        ql.qlinear_gemm_w8a8(*args, out_dtype=dt, out=o, bias=_cuda(b))
        o0 = ql.qlinear_gemm_w8a8(*args, out_dtype=dt, bias=torch.zeros(n, dtype=torch.float32, device=DEV))
        onb = ql.qlinear_gemm_w8a8(*args, out_dtype=dt)
        _sync()
        assert_float_close(o, yb, f"w8a8+bias {dt}", extra=_bias_tol(y, b.numpy()))
        assert torch.equal(o0, onb), "a zero bias must leave the result unchanged"


@pytest.mark.parametrize("m,n,k", [(1, 400, 512), (16, 400, 768), (40, 400, 512), (130, 256, 768), (300, 400, 512),
                                   (100, 400, 2048),    # two decode launches (64 and 36 rows)
                                   (16, 400, 4096)])    # one-stage decode kernel
def test_w2a8_bias_parity(m, n, k):
    d = synthetic.bitlinear(m, n, k, seed=1400 + m + n)
    xq_ref, pts_ref, _ = oracle.quant_act(d["x"].float().numpy(), rmsnorm=True)
    codes, gamma = oracle.ternary_quant(d["w"].numpy())
    _, y = oracle.w2a8(xq_ref, pts_ref, codes, gamma)
    b = synthetic.bias(n, 1.0, seed=1500 + n)
    yb = oracle.add_bias(y, b.numpy())
    xq, pts, rs = ql.qlinear_quant_act(_cuda(d["x"]), rmsnorm=True)
    packed, g = ql.qlinear_pack_ternary(_cuda(d["w"]), ql.QL_W_NK)
    for dt in (torch.bfloat16, torch.float16):
        o = poison((m, n), dt)
        ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=dt, out=o, bias=_cuda(b))
        o0 = ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=dt,
                                  bias=torch.zeros(n, dtype=torch.float32, device=DEV))
        onb = ql.qlinear_gemm_w2a8(xq, pts, rs, packed, g, n, out_dtype=dt)
        _sync()
        assert_equal(xq, xq_ref, "activation codes")
        assert_float_close(o, yb, f"w2a8+bias {dt}", extra=_bias_tol(y, b.numpy()))
        assert torch.equal(o0, onb), "a zero bias must leave the result unchanged"


@pytest.mark.parametrize("m,n,k,g", [(1, 48, 256, 128), (17, 400, 512, 256), (40, 64, 384, 128)])
def test_grouped_int4_bias_parity(m, n, k, g):
    d = synthetic.grouped_int4(m, n, k, g, seed=1600 + m + n + k)
    x, q, s, z = d["x"], d["q"], d["s"], d["z"]
    b = synthetic.bias(n, 1.0, seed=1700 + n)
    pw = ql.qlinear_pack_int4(_cuda(q), ql.QL_INT4_WEIGHT)
    pz = ql.qlinear_pack_int4(_cuda(z), ql.QL_INT4_ZEROS)
    ab = np.abs(b.numpy().astype(np.float64))[None, :]
    # fp16 activations
    y, bound = oracle.grouped_int4(x.float().numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    yb = oracle.add_bias(y, b.numpy())
    o32 = ql.qlinear_gemm_w4a8_grouped(_cuda(x), pw, _cuda(s), pz, g, n, out_dtype=torch.float32, bias=_cuda(b))
    o16 = ql.qlinear_gemm_w4a8_grouped(_cuda(x), pw, _cuda(s), pz, g, n, out_dtype=torch.float16, bias=_cuda(b))
    _sync()
    # the grouped bar on the product, plus the fp32 add, plus (fp16) one rounding of y + b
    for o, rel in ((o32, 2.0 ** -23), (o16, 2.0 ** -10)):
        err = np.abs(to_np(o).astype(np.float64) - yb)
        tol = 1e-3 * bound + rel * np.abs(yb) + 2.0 ** -23 * ab
        assert np.all(err <= tol), f"grouped+bias {o.dtype}: max err/tol {np.max(err / tol)}"
    assert torch.equal(o16, o32.to(torch.float16))
    # int8 activation codes
    xq, pts, _, _, _ = _grouped_i8_inputs(m, n, k, g, seed=1800 + m)
    y, bound = oracle.grouped_int4_i8(xq.numpy(), pts.numpy(), q.numpy(), s.float().numpy(), z.numpy(), g)
    yb = oracle.add_bias(y, b.numpy())
    outs = {dt: ql.qlinear_gemm_w4a8_grouped(_cuda(xq), pw, _cuda(s), pz, g, n, out_dtype=dt,
                                             per_token_scale=_cuda(pts), bias=_cuda(b))
            for dt in (torch.float32, torch.float16, torch.bfloat16)}
    _sync()
    err32 = np.abs(to_np(outs[torch.float32]).astype(np.float64) - yb)
    assert np.all(err32 <= 2.0 ** -18 * bound + 2.0 ** -23 * (np.abs(y) + ab) + 1e-30), "grouped i8+bias fp32"
    # 16-bit outputs: the fp32 value rounded once to nearest even
    for dt in (torch.float16, torch.bfloat16):
        err = np.abs(to_np(outs[dt]).astype(np.float64) - yb)
        tol = 1e-3 * bound + TOL_REL[dt] * np.abs(yb) + 2.0 ** -23 * ab
        assert np.all(err <= tol), f"grouped i8+bias {dt}: max err/tol {np.max(err / tol)}"
        assert torch.equal(outs[dt], outs[torch.float32].to(dt))


def test_bias_with_int32_output_is_rejected():
    d = synthetic.w8a8(4, 8, 16, True, seed=3)
    with pytest.raises(ValueError):
        ql.qlinear_gemm_w8a8(_cuda(d["x"]), _cuda(d["w"]), ql.QL_W_NK, None, None, out_dtype=torch.int32,
                             bias=torch.zeros(8, dtype=torch.float32, device=DEV))


# ---------------------------------------------------------------------------
# A4W4
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,k", [(33, 20, 130), (256, 256, 512), (129, 65, 1000), (1, 1, 1), (600, 520, 640),
                                   (1024, 1024, 256), (16, 300, 512), (48, 200, 256)])
@pytest.mark.parametrize("scale_mul", [1.0, 0.25])
def test_a4w4_parity(m, n, k, scale_mul):
    d = synthetic.a4w4(m, n, k, seed=800 + m + n + k)
    sa, sw = d["scale_a"] * scale_mul, d["scale_w"] * scale_mul
    qa, qw, acc, y = oracle.a4w4(d["x"].float().numpy(), d["w"].float().numpy(), sa, sw, d["eps"])
    sag = torch.tensor([sa], dtype=torch.float32, device=DEV)
    swg = torch.tensor([sw], dtype=torch.float32, device=DEV)
    out = poison((m, n), torch.float16)
    out, ws = ql.qlinear_gemm_a4w4(_cuda(d["x"]), _cuda(d["w"]), sag, swg, d["eps"], out=out)
    xa, wb = ql.a4w4_operands_from_workspace(ws, m, n, k)
    oi = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, None, None, out_dtype=torch.int32, out=oi)
    ob = ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, sag, swg, d["eps"], out_dtype=torch.bfloat16)
    # the int8-code product on the oracle's codes
    oi8 = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_codes(_cuda(torch.from_numpy(qa)), _cuda(torch.from_numpy(qw)), sag, swg, d["eps"],
                               out_dtype=torch.int32, out=oi8)
    o16 = ql.qlinear_gemm_a4w4_codes(_cuda(torch.from_numpy(qa)), _cuda(torch.from_numpy(qw)), sag, swg, d["eps"])
    _sync()
    assert_equal(xa, oracle.pack_a4w4_fp6(qa), "x operand")
    assert_equal(wb, oracle.pack_a4w4_fp6(qw), "w operand")
    assert_equal(oi, acc, "a4w4 accumulator (fp6 operands)")
    assert_equal(oi8, acc, "a4w4 accumulator (int8 codes)")
    assert_float_close(out, y, "a4w4 fp16")
    assert_float_close(ob, y, "a4w4 bf16")
    assert_float_close(o16, y, "a4w4 codes fp16")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("rows,k", [(45, 200), (32, 128), (70, 77), (300, 1000)])
def test_a4w4_operand_quant_parity(dt, rows, k):
    """Codes of every input type and ragged shape (k % 8 != 0 takes element loads) packed bit for bit."""
    r = synthetic.rng(3000 + rows + k)
    x = torch.from_numpy(r.normal(0, 1, (rows, k)).astype(np.float32)).to(dt)
    scale = 0.3
    q = oracle.quant_int4_tensor(x.float().numpy(), scale, 1e-5)
    op = ql.qlinear_quant_a4w4_operand(_cuda(x), torch.tensor([scale], dtype=torch.float32, device=DEV))
    _sync()
    assert_equal(op, oracle.pack_a4w4_fp6(q), f"operand {dt}")


def test_a4w4_operands_max_k_extremes():
    """k = 131071 with every code -8: acc = 64 k = 8388544, exact in the fp32 accumulator."""
    m, n, k = 3, 5, 131071
    x = torch.full((m, k), -8.0, dtype=torch.float16)
    w = torch.full((n, k), -8.0, dtype=torch.float16)
    w[1, ::2] = 7.0
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    qa = oracle.quant_int4_tensor(x.float().numpy(), 1.0, 1e-5)
    qw = oracle.quant_int4_tensor(w.float().numpy(), 1.0, 1e-5)
    acc = oracle.gemm_i8(qa, qw, True)
    assert int(acc[0, 0]) == 64 * k
    xa = ql.qlinear_quant_a4w4_operand(_cuda(x), one)
    wb = ql.qlinear_quant_a4w4_operand(_cuda(w), one)
    o = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, None, None, out_dtype=torch.int32, out=o)
    _sync()
    assert_equal(o, acc, "a4w4 max-k accumulator")


@pytest.mark.parametrize("m,n,k", [(512, 512, 512), (520, 777, 300), (256, 1024, 8192)])
def test_a4w4_operands_equal_int8_codes_bit_for_bit(m, n, k):
    """The FP6 product and the int8 product of the same codes agree exactly in every output type."""
    d = synthetic.a4w4(m, n, k, seed=3100 + m + k)
    sag = torch.tensor([d["scale_a"]], dtype=torch.float32, device=DEV)
    swg = torch.tensor([d["scale_w"]], dtype=torch.float32, device=DEV)
    xg, wg = _cuda(d["x"]), _cuda(d["w"])
    xa = ql.qlinear_quant_a4w4_operand(xg, sag, d["eps"])
    wb = ql.qlinear_quant_a4w4_operand(wg, swg, d["eps"])
    xq = ql.qlinear_quant_int4_tensor(xg.view(-1), sag, d["eps"]).view(m, k)
    wq = ql.qlinear_quant_int4_tensor(wg.view(-1), swg, d["eps"]).view(n, k)
    for dt in (torch.int32, torch.float16, torch.bfloat16):
        a = ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, sag, swg, d["eps"], out_dtype=dt)
        b = ql.qlinear_gemm_a4w4_codes(xq, wq, sag, swg, d["eps"], out_dtype=dt)
        _sync()
        assert torch.equal(a.view(torch.int16) if dt != torch.int32 else a,
                           b.view(torch.int16) if dt != torch.int32 else b), f"{dt}"
    qa = oracle.quant_int4_tensor(d["x"].float().numpy(), d["scale_a"], d["eps"])
    assert_equal(xq, qa, "x codes")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("rows,k", [(45, 200), (32, 128), (70, 77), (300, 1000), (1, 1)])
def test_a4w4_packed_operand_quant_parity(dt, rows, k):
    """The two-codes-per-byte operand, bit for bit, for every input type and ragged shape."""
    r = synthetic.rng(3200 + rows + k)
    x = torch.from_numpy(r.normal(0, 1, (rows, k)).astype(np.float32)).to(dt)
    scale = 0.3
    q = oracle.quant_int4_tensor(x.float().numpy(), scale, 1e-5)
    op = poison((oracle.a4w4_packed_bytes(rows, k),), torch.uint8)
    ql.qlinear_quant_a4w4_packed(_cuda(x), torch.tensor([scale], dtype=torch.float32, device=DEV), operand=op)
    _sync()
    assert_equal(op, oracle.pack_a4w4_int4(q), f"packed operand {dt}")


@pytest.mark.parametrize("m,n,k", [(33, 20, 130), (256, 256, 512), (129, 65, 1000), (1, 1, 1), (600, 520, 640),
                                   (1024, 1024, 256), (16, 300, 512), (520, 777, 300), (256, 1024, 8192)])
def test_a4w4_packed_parity(m, n, k):
    """Packed 4-bit operands: exact accumulators against the oracle, and every output type
    bit-identical to the FP6-operand product of the same codes."""
    d = synthetic.a4w4(m, n, k, seed=3300 + m + n + k)
    sa, sw = d["scale_a"] * 0.5, d["scale_w"] * 0.5     # some codes clamp at -8 / 7
    qa, qw, acc, y = oracle.a4w4(d["x"].float().numpy(), d["w"].float().numpy(), sa, sw, d["eps"])
    sag = torch.tensor([sa], dtype=torch.float32, device=DEV)
    swg = torch.tensor([sw], dtype=torch.float32, device=DEV)
    xg, wg = _cuda(d["x"]), _cuda(d["w"])
    xp = ql.qlinear_quant_a4w4_packed(xg, sag, d["eps"])
    wp = ql.qlinear_quant_a4w4_packed(wg, swg, d["eps"])
    xa = ql.qlinear_quant_a4w4_operand(xg, sag, d["eps"])
    wb = ql.qlinear_quant_a4w4_operand(wg, swg, d["eps"])
    outs = {}
    for dt in (torch.int32, torch.float16, torch.bfloat16):
        o = poison((m, n), dt)
        ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, sag, swg, d["eps"], out_dtype=dt, out=o)
        f = ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, sag, swg, d["eps"], out_dtype=dt)
        outs[dt] = (o, f)
    _sync()
    assert_equal(xp, oracle.pack_a4w4_int4(qa), "x packed operand")
    assert_equal(wp, oracle.pack_a4w4_int4(qw), "w packed operand")
    assert_equal(outs[torch.int32][0], acc, "a4w4 accumulator (packed operands)")
    for dt in (torch.float16, torch.bfloat16):
        o, f = outs[dt]
        assert torch.equal(o.view(torch.int16), f.view(torch.int16)), f"packed vs FP6 operands {dt}"
        assert_float_close(o, y, f"a4w4 packed {dt}")


def test_a4w4_packed_max_k_extremes():
    """k = 131071 with every code -8 (and 7 on alternate k of one row): acc = 64 k exactly."""
    m, n, k = 3, 5, 131071
    x = torch.full((m, k), -8.0, dtype=torch.float16)
    w = torch.full((n, k), -8.0, dtype=torch.float16)
    w[1, ::2] = 7.0
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    qa = oracle.quant_int4_tensor(x.float().numpy(), 1.0, 1e-5)
    qw = oracle.quant_int4_tensor(w.float().numpy(), 1.0, 1e-5)
    acc = oracle.gemm_i8(qa, qw, True)
    xp = ql.qlinear_quant_a4w4_packed(_cuda(x), one)
    wp = ql.qlinear_quant_a4w4_packed(_cuda(w), one)
    o = poison((m, n), torch.int32)
    ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, None, None, out_dtype=torch.int32, out=o)
    _sync()
    assert_equal(o, acc, "a4w4 packed max-k accumulator")


# ---------------------------------------------------------------------------
# Q4Linear backward
# ---------------------------------------------------------------------------
U24 = 2.0 ** -24


def _q4_bwd_inputs(m, n, k, dt, seed, clip=0.6):
    r = synthetic.rng(seed)
    x = torch.from_numpy(r.normal(0, 1, (m, k)).astype(np.float32)).to(dt)
    w = torch.from_numpy((0.02 * r.normal(0, 1, (n, k))).astype(np.float32)).to(dt)
    g = torch.from_numpy(r.normal(0, 1, (m, n)).astype(np.float32)).to(dt)
    sa = float(np.float32(x.float().abs().max().item() / 7 * clip))
    sw = float(np.float32(w.float().abs().max().item() / 7 * clip))
    return g, x, w, sa, sw


def _q4_bwd_check(gx, gw, gs, ref, n, m, what):
    """fp32 accumulation over a sum of n (grad_x) or m (grad_w) exact products,
    then one fp32 multiply and the output rounding; the scale gradient adds
    each term's error, at most (n + 1) u bx |t|, and is rounded to fp32 once."""
    rx, rw, rs, bx, bw, bs = ref
    for got, want, b, depth, name in ((gx, rx, bx, n, "grad_x"), (gw, rw, bw, m, "grad_w")):
        rel = {torch.float32: U24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}[got.dtype]
        g = to_np(got).astype(np.float64)
        tol = depth * U24 * b + 2 * U24 * np.abs(want) + rel * np.abs(want) + 1e-30
        err = np.abs(g - want)
        assert np.all(err <= tol), f"{what} {name}: max err/tol {np.max(err / tol)}"
        assert np.array_equal(g == 0, want == 0) or np.all(g[want == 0] == 0), f"{what} {name}: range mask"
    # + one fp32 multiply per term and the fp32 rounding of the fp64 sum
    assert abs(float(gs) - rs) <= (n + 1) * U24 * bs + U24 * abs(rs) + 1e-30, f"{what} grad_scale_a {float(gs)} vs {rs}"


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("m,n,k", [(64, 48, 40), (300, 270, 200), (512, 512, 512), (520, 777, 300), (1, 1, 1),
                                   (33, 64, 1000)])
def test_q4_backward_parity(dt, m, n, k):
    g, x, w, sa, sw = _q4_bwd_inputs(m, n, k, dt, seed=4000 + m + n + k)
    ref = oracle.q4_backward(g.float().numpy(), x.float().numpy(), w.float().numpy(), sa, sw, 1e-5)
    sag = torch.tensor([sa], dtype=torch.float32, device=DEV)
    swg = torch.tensor([sw], dtype=torch.float32, device=DEV)
    gx = poison((m, k), torch.float32)
    gw = poison((n, k), torch.float32)
    gx, gw, gs = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), sag, swg, 1e-5, grad_x=gx, grad_w=gw)
    _sync()
    _q4_bwd_check(gx, gw, gs.item(), ref, n, m, f"{dt} {m}x{n}x{k}")


@pytest.mark.parametrize("gdt", [torch.float16, torch.bfloat16])
def test_q4_backward_16bit_grads(gdt):
    m, n, k = 300, 256, 320
    g, x, w, sa, sw = _q4_bwd_inputs(m, n, k, torch.float16, seed=4100)
    ref = oracle.q4_backward(g.float().numpy(), x.float().numpy(), w.float().numpy(), sa, sw, 1e-5)
    sag = torch.tensor([sa], dtype=torch.float32, device=DEV)
    swg = torch.tensor([sw], dtype=torch.float32, device=DEV)
    gx, gw, gs = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), sag, swg, 1e-5, grad_dtype=gdt)
    gx32, gw32, gs32 = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), sag, swg, 1e-5)
    _sync()
    _q4_bwd_check(gx, gw, gs.item(), ref, n, m, f"grads {gdt}")
    # the 16-bit gradients are the fp32 ones rounded once
    assert torch.equal(gx, gx32.to(gdt)) and torch.equal(gw, gw32.to(gdt))
    assert gs.item() == gs32.item()


def test_q4_backward_deterministic_and_eps():
    m, n, k = 520, 300, 260
    g, x, w, sa, sw = _q4_bwd_inputs(m, n, k, torch.float16, seed=4200)
    sag = torch.tensor([sa], dtype=torch.float32, device=DEV)
    swg = torch.tensor([sw], dtype=torch.float32, device=DEV)
    a = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), sag, swg, 1e-5)
    b = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), sag, swg, 1e-5)
    # a scale below eps: no scale gradient
    tiny = torch.tensor([1e-9], dtype=torch.float32, device=DEV)
    c = ql.qlinear_q4_backward(_cuda(g), _cuda(x), _cuda(w), tiny, swg, 1e-5)
    _sync()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert a[2].item() == b[2].item()
    assert c[2].item() == 0.0



# ---------------------------------------------------------------------------
# HBM read-stream measurement aid: every 32-bit word is read exactly once
# (a word read twice cancels in the XOR, a word skipped is missing)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nbytes", [16, 48, 4096 * 16 + 16, 2048 * 128 + 32, 8 << 20, (64 << 20) + 16 * 3])
def test_hbm_read_stream_reads_every_word_once(nbytes):
    g = torch.Generator().manual_seed(nbytes % 1000003)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    want = int(np.bitwise_xor.reduce(words.numpy().view(np.uint32)))
    sink = ql.qlinear_hbm_read_stream(_cuda(words))
    _sync()
    assert int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint64))) == want
    ql.qlinear_hbm_read_stream(_cuda(words), sink=sink)   # a second pass cancels the first
    _sync()
    assert not sink.cpu().numpy().any()
