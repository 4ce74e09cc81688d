"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values
printed on the pages (``tests/golden``), textbook results computed by a
library routine the oracle does not use (numpy integer / fp64 matmul), exact
rational arithmetic (``fractions.Fraction``) on tiny inputs, closed forms and
invariants.  A dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_values(x: torch.Tensor) -> np.ndarray:
    return x.float().numpy()


# ---------------------------------------------------------------------------
# O4: integer GEMM + per-token epilogue
# ---------------------------------------------------------------------------
def test_worked_example_exact():
    """"Per-token Quantization for Matmul", Example: printed output and sums."""
    with open(os.path.join(GOLDEN, "per_token_example.json")) as f:
        ex = json.load(f)
    x = np.array(ex["x"], np.int8)
    w = np.array(ex["weight_kn"], np.int8)
    acc, y = oracle.w8a8(x, w, False, np.array(ex["perTokenScale"], np.float32),
                         np.array(ex["deqScale"], np.float32))
    assert acc.tolist() == ex["acc"]
    assert y.tolist() == ex["output"]
    # every printed output is exactly representable in fp16 and bf16
    out = np.array(ex["output"], np.float64)
    assert np.array_equal(oracle.round_f16(y).view(np.float16).astype(np.float64), out)
    bf = (oracle.round_bf16(y).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(bf, out)


@pytest.mark.parametrize("m,n,k,layout_nk", [(1, 1, 1, True), (5, 7, 3, False), (17, 33, 65, True),
                                             (33, 18, 300, False), (64, 48, 512, True)])
def test_gemm_unit_scales_is_textbook_matmul(m, n, k, layout_nk):
    """pts = deq = 1 reduces to integer matmul (numpy int64 ``@``)."""
    d = synthetic.w8a8(m, n, k, layout_nk, seed=7 + m)
    x, w = d["x"].numpy(), d["w"].numpy()
    ones_m, ones_n = np.ones(m, np.float32), np.ones(n, np.float32)
    acc, y = oracle.w8a8(x, w, layout_nk, ones_m, ones_n)
    wk = w.T if layout_nk else w  # [k, n]
    ref = x.astype(np.int64) @ wk.astype(np.int64)
    assert np.array_equal(acc.astype(np.int64), ref)
    assert np.array_equal(y, ref.astype(np.float64))


@pytest.mark.parametrize("layout_nk", [False, True])
def test_dequant_brute_force_fp64(layout_nk):
    """y equals the fp64 matmul of the dequantized operands (x*pts) @ (w*deq)."""
    d = synthetic.w8a8(19, 23, 77, layout_nk, seed=11)
    x, w, pts, deq = (d[k].numpy() for k in ("x", "w", "pts", "deq"))
    _, y = oracle.w8a8(x, w, layout_nk, pts, deq)
    wk = (w.T if layout_nk else w).astype(np.float64)
    ref = (x.astype(np.float64) * pts.astype(np.float64)[:, None]) @ (wk * deq.astype(np.float64)[None, :])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)


def test_bias_is_added_per_output_column_unscaled():
    """x = identity, pts = 2, deq = 1/4: y + b = w / 2 + b[n] exactly, and the
    whole product equals torch's fp64 ``F.linear(x * pts, w * deq, b)``."""
    k = n = 24
    x = np.eye(k, dtype=np.int8)
    w = synthetic.w8a8(k, n, k, True, seed=31)["w"].numpy()  # [n, k]
    b = synthetic.bias(n, 3.0, seed=32).numpy()
    pts, deq = np.full(k, 2.0, np.float32), np.full(n, 0.25, np.float32)
    _, y = oracle.w8a8(x, w, True, pts, deq)
    yb = oracle.add_bias(y, b)
    assert np.array_equal(yb, w.T.astype(np.float64) / 2 + b.astype(np.float64)[None, :])
    d = synthetic.w8a8(9, 13, 40, True, seed=33)
    x, w, pts, deq = (d[key].numpy() for key in ("x", "w", "pts", "deq"))
    b = synthetic.bias(13, 0.1, seed=34).numpy()
    _, y = oracle.w8a8(x, w, True, pts, deq)
    ref = torch.nn.functional.linear(torch.from_numpy(x.astype(np.float64) * pts.astype(np.float64)[:, None]),
                                     torch.from_numpy(w.astype(np.float64) * deq.astype(np.float64)[:, None]),
                                     torch.from_numpy(b.astype(np.float64))).numpy()
    np.testing.assert_allclose(oracle.add_bias(y, b), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout_nk,per_batch_deq", [(False, False), (True, True)])
def test_batched_is_independent_products(layout_nk, per_batch_deq):
    """Each batch is its own product: numpy int64 ``einsum`` for the
    accumulators, fp64 dequant of each batch's slices for y."""
    batch, m, n, k = 3, 5, 7, 40
    ds = [synthetic.w8a8(m, n, k, layout_nk, seed=40 + b) for b in range(batch)]
    x = np.stack([d["x"].numpy() for d in ds])
    w = np.stack([d["w"].numpy() for d in ds])
    pts = np.stack([d["pts"].numpy() for d in ds])
    deq = np.stack([d["deq"].numpy() for d in ds]) if per_batch_deq else ds[0]["deq"].numpy()
    acc, y = oracle.w8a8_batched(x, w, layout_nk, pts, deq)
    wk = np.swapaxes(w, 1, 2) if layout_nk else w  # [batch, k, n]
    ref = np.einsum("bmk,bkn->bmn", x.astype(np.int64), wk.astype(np.int64))
    assert np.array_equal(acc.astype(np.int64), ref)
    d2 = deq if per_batch_deq else np.broadcast_to(deq, (batch, n))
    yref = ref.astype(np.float64) * pts.astype(np.float64)[:, :, None] * d2.astype(np.float64)[:, None, :]
    np.testing.assert_allclose(y, yref, rtol=1e-15, atol=0)


@pytest.mark.parametrize("int8_codes", [False, True])
def test_grouped_batched_is_independent_products(int8_codes):
    """Each slice is its own product: fp64 dequantize-then-matmul per slice
    with numpy einsum, the per-token scale applied to the int8 codes' rows."""
    batch, m, n, k, g = 3, 4, 16, 256, 128
    ds = [synthetic.grouped_int4(m, n, k, g, seed=60 + b) for b in range(batch)]
    q = np.stack([d["q"].numpy() for d in ds])
    s = np.stack([d["s"].float().numpy() for d in ds]).astype(np.float64)
    z = np.stack([d["z"].numpy() for d in ds])
    if int8_codes:
        r = synthetic.rng(66)
        x = r.integers(-127, 128, (batch, m, k), dtype=np.int8)
        pts = r.uniform(1e-3, 1e-2, (batch, m)).astype(np.float32)
        y, _ = oracle.grouped_int4_batched(x, q, s, z, g, pts=pts)
        xd = x.astype(np.float64) * pts.astype(np.float64)[:, :, None]
    else:
        x = np.stack([d["x"].float().numpy() for d in ds])
        y, _ = oracle.grouped_int4_batched(x, q, s, z, g)
        xd = x.astype(np.float64)
    w = (q.astype(np.float64) - np.repeat(z, g, axis=2)) * np.repeat(s, g, axis=2)  # [batch, n, k]
    ref = np.einsum("bmk,bnk->bmn", xd, w)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("m,n,k,layout_nk", [(1, 1, 1, True), (7, 5, 300, True), (33, 17, 1000, False),
                                              (64, 48, 4096, True)])
def test_gemm_exact_equals_the_loop_product(m, n, k, layout_nk):
    """The float64 library product of integer codes is the int32 loop product exactly,
    including the extreme codes (-128 * -128 summed over the whole k)."""
    r = synthetic.rng(m * 1000 + n + k)
    x = r.integers(-128, 128, (m, k), dtype=np.int8)
    w = r.integers(-128, 128, (n, k) if layout_nk else (k, n), dtype=np.int8)
    x[0, :] = -128
    if layout_nk:
        w[0, :] = -128
    else:
        w[:, 0] = -128
    got = oracle.gemm_exact(x, w, layout_nk)
    assert got.dtype == np.int32
    assert np.array_equal(got, oracle.gemm_i8(x, w, layout_nk))
    assert int(got[0, 0]) == 128 * 128 * k


def test_gemm_int32_overflow_is_reported():
    """The definition asserts the accumulator fits int32: (-128)^2 * 2^17 = 2^31 does not."""
    k = 1 << 17
    x = np.full((1, k), -128, np.int8)
    with pytest.raises(ValueError):
        oracle.gemm_i8(x, x, True)
    # one fewer term fits
    acc = oracle.gemm_i8(x[:, :k - 1], x[:, :k - 1], True)
    assert int(acc[0, 0]) == 128 * 128 * (k - 1)


# ---------------------------------------------------------------------------
# O1: per-token absmax int8 quantization
# ---------------------------------------------------------------------------
def _act_rows(seed=3, m=24, k=257):
    return _bf16_values(synthetic.activations(m, k, seed, outliers=0.01))


def test_quant_act_invariants():
    """"Common Attention Utilities" activation_quant: range [-128,127], per-token scale."""
    x = _act_rows()
    q, pts, rs = oracle.quant_act(x)
    assert q.min() >= -127 and q.max() <= 127          # 127/absmax scaling never reaches -128
    a = np.abs(x).max(axis=1)
    ap = np.maximum(a, np.float32(1e-5))
    for i in range(x.shape[0]):
        j = int(np.argmax(np.abs(x[i])))
        assert abs(int(q[i, j])) == 127 and np.sign(q[i, j]) == np.sign(x[i, j])
    # reconstruction within half a step (plus fp32 slack)
    step = ap.astype(np.float64) / 127.0
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * step[:, None])
    assert np.all(err <= step[:, None] * (0.5 + 1e-6))
    assert np.array_equal(rs, q.astype(np.int64).sum(axis=1).astype(np.int32))
    # pts without RMSNorm is the correctly rounded fp32 of a'/127
    assert np.array_equal(pts, (ap.astype(np.float64) / 127.0).astype(np.float32))


def test_quant_act_idempotent():
    """Re-quantizing the dequantized codes returns the same codes."""
    x = _act_rows(seed=5)
    q, pts, _ = oracle.quant_act(x)
    xr = q.astype(np.float32) * pts[:, None]
    q2, _, _ = oracle.quant_act(xr)
    assert np.array_equal(q, q2)


def test_quant_act_exact_rational_brute_force():
    """Codes from exact arithmetic: s = RN32(127/a'), v = RN32(x*s), q = round-half-even(v).

    fp64 carries each fp32 step exactly (products of two fp32 values are exact
    in fp64; fp64 division rounded to fp32 is the correctly rounded fp32
    quotient), and Python's ``round`` on Fraction is round-half-to-even.
    """
    x = _act_rows(seed=9, m=6, k=64)
    q, _, _ = oracle.quant_act(x)
    for i in range(x.shape[0]):
        a = max(abs(float(v)) for v in x[i])
        ap = max(a, float(np.float32(1e-5)))
        s = float(np.float32(127.0 / ap))
        for j in range(x.shape[1]):
            v = float(np.float32(float(x[i, j]) * s))
            c = round(Fraction(v))
            c = max(-128, min(127, c))
            assert int(q[i, j]) == c


def test_quant_act_rmsnorm_folding():
    """"Class BitLinear" steps 1-2: RMSNorm leaves codes unchanged and scales pts by r."""
    x = _act_rows(seed=13)
    q0, p0, r0 = oracle.quant_act(x, rmsnorm=False)
    q1, p1, r1 = oracle.quant_act(x, rmsnorm=True, eps_norm=1e-6)
    assert np.array_equal(q0, q1) and np.array_equal(r0, r1)
    xd = x.astype(np.float64)
    r = 1.0 / np.sqrt((xd * xd).mean(axis=1) + 1e-6)
    np.testing.assert_allclose(p1.astype(np.float64) / p0.astype(np.float64), r, rtol=2e-7)
    # literal pipeline: normalize in fp64, then absmax-quantize the normalized row
    lit = np.rint(np.clip((xd * r[:, None]) * (127.0 / np.abs(xd * r[:, None]).max(axis=1))[:, None],
                          -128, 127))
    assert np.mean(lit != q1) < 1e-3


def test_quant_act_degenerate_rows():
    x = np.zeros((3, 40), np.float32)
    x[1, 7] = -3.5          # one-hot
    x[2, :] = 2.0           # constant
    q, pts, rs = oracle.quant_act(x)
    assert np.all(q[0] == 0) and pts[0] == np.float32(np.float64(np.float32(1e-5)) / 127.0)
    assert q[1, 7] == -127 and np.count_nonzero(q[1]) == 1
    assert np.all(q[2] == 127) and rs[2] == 127 * 40


def test_quant_act_guard_applies_to_the_normalized_row():
    """"Class BitLinear" steps 1-2: the quantizer sees the normalized row r*x.

    The eps guard of the absmax protects the division of the quantizer, so it
    applies to max|r x|, not to max|x|.  Checked against a literal fp64
    normalize-then-quantize pipeline on rows from 1e-12 to 1: where r*a is at
    least eps the codes are those of x itself (127 at the absmax); below, the
    codes are rne(r x 127 / eps) and pts = eps / 127.
    """
    rng = np.random.default_rng(77)
    eps_q, eps_n = 1e-5, 1e-6
    rows = []
    for scale in (1.0, 1e-3, 1e-6, 3e-8, 1e-9, 1e-10, 1e-12):
        rows.append((rng.standard_normal(96) * scale).astype(np.float32))
    rows.append(np.full(96, 1e-6, np.float32) * np.sign(rng.standard_normal(96)).astype(np.float32))
    rows.append(np.zeros(96, np.float32))
    x = np.stack(rows)
    q, pts, rs = oracle.quant_act(x, rmsnorm=True, eps_norm=eps_n, eps_q=eps_q)
    xd = x.astype(np.float64)
    r = 1.0 / np.sqrt((xd * xd).mean(axis=1) + eps_n)
    y = xd * r[:, None]
    ay = np.maximum(np.abs(y).max(axis=1), eps_q)
    v = y * (127.0 / ay)[:, None]
    lit = np.clip(np.rint(v), -128, 127)
    near_tie = np.abs(np.abs(v - np.trunc(v)) - 0.5) < 1e-4
    assert np.all((lit == q) | near_tie)
    assert np.count_nonzero(near_tie) < 3
    # the +-1e-6 row: normalized absmax is about 1e-3, far above eps, so every code is +-127
    assert np.all(np.abs(q[7]) == 127)
    # rows whose normalized absmax is below eps use eps: pts = eps / 127, codes below 127
    small = np.abs(y).max(axis=1) < eps_q
    assert small[4:7].all() and small[8] and not small[:4].any() and not small[7]
    np.testing.assert_allclose(pts[small].astype(np.float64), eps_q / 127.0, rtol=2 ** -22)
    assert np.all(np.abs(q[5]) < 127) and np.all(q[8] == 0)
    np.testing.assert_allclose(pts.astype(np.float64), ay / 127.0, rtol=2 ** -22)
    assert np.array_equal(rs, q.astype(np.int64).sum(axis=1).astype(np.int32))


# ---------------------------------------------------------------------------
# O2: absmean ternary
# ---------------------------------------------------------------------------
def test_ternary_exact_rational_brute_force():
    """Codes equal clamp(round-half-even(W / gamma), -1, 1) with exact rational gamma."""
    w = synthetic.master_weight(16, 48, seed=21).numpy()
    codes, g = oracle.ternary_quant(w)
    sx = sum(Fraction(abs(float(v))) for v in w.ravel())
    gx = sx / w.size
    # gamma = fl64(fl64(exact sum) / count): Python's int / int division rounds correctly
    assert g == float(sx) / w.size
    assert abs(Fraction(g) - gx) <= gx * Fraction(1, 2 ** 51)
    assert oracle.ternary_tie_band(w, g) == 0
    for (i, j), v in np.ndenumerate(w):
        c = max(-1, min(1, round(Fraction(float(v)) / gx)))
        assert int(codes[i, j]) == c


def test_ternary_absmean_sum_is_exact():
    """The mean comes from the exact sum of |W|, rounded once: inputs on which
    a running fp64 sum rounds differently, spanning denormals to 2^127."""
    cases = [
        [1.0] + [2.0 ** -53] * 15,          # a running sum stays at 1.0; exactly 1 + 15 * 2^-53
        [2.0 ** 127, 2.0 ** -149, 1.0, 3.0 ** 20] + [-(2.0 ** 70)] * 12,
        [2.0 ** -149] * 8 + [1.5 * 2.0 ** -126] * 8,
        [float(np.float32(v)) for v in synthetic.rng(25).standard_normal(16) * 1e30],
    ]
    for vals in cases:
        w = np.repeat(np.array([vals], np.float32), 16, axis=0)
        assert np.all(np.isfinite(w))
        _, g = oracle.ternary_quant(w, eps=0.0)
        exact = sum(Fraction(abs(float(v))) for v in w.ravel())
        assert g == float(exact) / w.size, vals
    # the first case is one a running fp64 sum gets wrong
    w = np.repeat(np.array([cases[0]], np.float32), 16, axis=0)
    running = 0.0
    for v in w.ravel():
        running += abs(float(v))
    assert running / w.size != oracle.ternary_quant(w, eps=0.0)[1]


def test_ternary_half_tie_rounds_to_zero():
    """A weight exactly at gamma'/2 rounds half-to-even to 0; just above gives +-1."""
    w = np.array([[1.0, -1.0, 0.5, -0.5, 3.0, 0.0, -3.0, 2.0]], np.float32)  # mean|w| = 1.375
    w = np.repeat(w, 16, axis=0)
    codes, g = oracle.ternary_quant(w)
    assert g == 1.375
    assert codes[0].tolist() == [1, -1, 0, 0, 1, 0, -1, 1]
    # mean|w| = 2, so +-1 sit exactly on gamma'/2: W/gamma' = +-0.5 rounds to 0,
    # 2/2 = 1 stays 1 and 5/2 = 2.5 clamps to 1
    w2 = np.repeat(np.array([[5.0, -5.0, 1.0, -1.0, 2.0, 0.0, -1.0, 1.0]], np.float32), 16, axis=0)
    codes2, g2 = oracle.ternary_quant(w2)
    assert g2 == 2.0
    exp = [max(-1, min(1, round(Fraction(float(v)) / Fraction(g2)))) for v in w2[0]]
    assert codes2[0].tolist() == exp == [1, -1, 0, 0, 1, 0, 0, 0]
    assert oracle.ternary_tie_band(w2, g2) == 4 * 16


def test_ternary_eps_guard_and_layouts():
    w = synthetic.master_weight(32, 64, seed=22).numpy()
    c_nk, g1 = oracle.ternary_quant(w, layout_nk=True)
    c_kn, g2 = oracle.ternary_quant(np.ascontiguousarray(w.T), layout_nk=False)
    assert np.array_equal(c_nk, c_kn) and abs(g1 - g2) <= 1e-15 * g1
    z = np.zeros((16, 16), np.float32)
    cz, gz = oracle.ternary_quant(z, eps=1e-5)
    assert gz == 1e-5 and not cz.any()


def test_ternary_sign_and_bake_idempotence():
    """"Common Attention Utilities" bake_ternary_weights: re-baking changes no code."""
    w = synthetic.master_weight(64, 256, seed=23).numpy()
    codes, g = oracle.ternary_quant(w)
    nz = codes != 0
    assert np.all(np.sign(w[nz]) == codes[nz])
    assert np.all(np.abs(w[~nz]) <= g / 2) and np.all(np.abs(w[nz]) > g / 2)
    baked = codes.astype(np.float32) * np.float32(g)
    codes2, g2 = oracle.ternary_quant(baked)
    assert np.array_equal(codes, codes2)
    # the scale drifts to p * fp32(gamma'), p = nonzero fraction: why baking is guarded
    p = nz.mean()
    assert abs(g2 - p * float(np.float32(g))) <= 1e-12 * g2


def test_ternary_gaussian_zero_fraction():
    """For Gaussian weights the zero fraction is erf(0.5*sqrt(2/pi)/sqrt(2)) ~ 0.310."""
    w = synthetic.master_weight(256, 4096, seed=24).numpy()
    codes, _ = oracle.ternary_quant(w)
    expect = math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))
    assert abs((codes == 0).mean() - expect) < 3e-3


def test_ternary_pack_round_trip_and_fragments():
    w = synthetic.master_weight(48, 768, seed=25).numpy()
    codes, _ = oracle.ternary_quant(w)
    packed = oracle.pack_ternary(codes)
    assert packed.size == 48 * 768 // 16
    assert np.array_equal(oracle.unpack_ternary(packed, 48, 768), codes)
    # no 2-bit field ever holds 3
    fields = np.stack([(packed >> s) & 3 for s in range(0, 32, 2)])
    assert not np.any(fields == 3)
    # each word unpacks to 16 consecutive k of one column: bytes of (word >> 2a) & 0x03030303
    kblocks = 768 // 256
    for nb, kb, l, t in [(0, 0, 0, 0), (2, 1, 37, 3), (1, 2, 63, 2)]:
        word = int(packed[(nb * kblocks + kb) * 256 + 4 * l + t])
        col = 16 * nb + l % 16
        k0 = 256 * kb + 64 * (l // 16) + 16 * t
        got = [((word >> (2 * a)) >> (8 * b)) & 3 for a in range(4) for b in range(4)]
        assert got == [int(c) + 1 for c in codes[col, k0:k0 + 16]]


# ---------------------------------------------------------------------------
# O3: grouped affine INT4
# ---------------------------------------------------------------------------
def _grouped(m=5, n=32, k=256, g=64, seed=31):
    d = synthetic.grouped_int4(m, n, k, g, seed=seed)
    return (d["x"].float().numpy().astype(np.float64), d["q"].numpy(),
            d["s"].float().numpy().astype(np.float64), d["z"].numpy(), g)


def test_grouped_zero_when_zero_point_equals_code():
    x, q, s, z, g = _grouped()
    zq = np.ascontiguousarray(np.repeat(q[:, ::g][:, :, None], 1, axis=2)[:, :, 0])
    qq = np.repeat(zq, g, axis=1)  # every code equals its group's zero
    y, _ = oracle.grouped_int4(x, qq, s, zq, g)
    assert np.all(y == 0.0)


def test_grouped_unit_scale_zero_offset_is_matmul():
    x, q, s, z, g = _grouped()
    y, _ = oracle.grouped_int4(x, q, np.ones_like(s), np.zeros_like(z), g)
    np.testing.assert_allclose(y, x @ q.astype(np.float64).T, rtol=1e-13)


@pytest.mark.parametrize("g", [32, 128, 256])
def test_grouped_brute_force_dequant_then_matmul(g):
    x, q, s, z, _ = _grouped(g=g, seed=33)
    w = np.repeat(s, g, axis=1) * (q.astype(np.float64) - np.repeat(z.astype(np.float64), g, axis=1))
    y, bound = oracle.grouped_int4(x, q, s, z, g)
    ref = x @ w.T
    assert np.all(np.abs(y - ref) <= 1e-12 * bound + 1e-300)
    np.testing.assert_allclose(bound, np.abs(x) @ np.abs(w).T, rtol=1e-12)
    # linearity in x (scaling by 2 is exact)
    y2, _ = oracle.grouped_int4(2 * x, q, s, z, g)
    assert np.array_equal(y2, 2 * y)


def _grouped_i8_case(m, n, k, g, seed):
    r = synthetic.rng(seed)
    xq = r.integers(-127, 128, (m, k), dtype=np.int8)
    pts = r.uniform(1e-3, 1e-2, m).astype(np.float32)
    d = synthetic.grouped_int4(m, n, k, g, seed=seed)
    return xq, pts, d["q"].numpy(), d["s"].float().numpy().astype(np.float64), d["z"].numpy()


def test_grouped_i8_equals_fp_grouped_on_dequantized_activations():
    """int8 codes times their per-token scale, fed to the fp64 grouped oracle, give the same y."""
    xq, pts, q, s, z = _grouped_i8_case(5, 48, 256, 128, seed=41)
    y, bound = oracle.grouped_int4_i8(xq, pts, q, s, z, 128)
    x = xq.astype(np.float64) * pts.astype(np.float64)[:, None]
    y2, bound2 = oracle.grouped_int4(x, q, s, z, 128)
    assert np.all(np.abs(y - y2) <= 1e-12 * bound + 1e-300)
    np.testing.assert_allclose(bound, bound2, rtol=1e-12)


def test_grouped_i8_unit_scale_zero_offset_is_integer_matmul():
    xq, _, q, s, z = _grouped_i8_case(4, 32, 256, 128, seed=42)
    y, _ = oracle.grouped_int4_i8(xq, np.ones(4, np.float32), q, np.ones_like(s), np.zeros_like(z), 128)
    assert np.array_equal(y, (xq.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))


def test_grouped_i8_zero_point_equal_to_code_gives_zero():
    xq, pts, _, s, z = _grouped_i8_case(3, 16, 256, 128, seed=43)
    q = np.repeat(z, 128, axis=1)
    y, _ = oracle.grouped_int4_i8(xq, pts, q, s, z, 128)
    assert not y.any()


@pytest.mark.parametrize("g", [128, 256])
def test_grouped_i8_brute_force(g):
    xq, pts, q, s, z = _grouped_i8_case(3, 16, 512, g, seed=44 + g)
    y, _ = oracle.grouped_int4_i8(xq, pts, q, s, z, g)
    w = np.repeat(s, g, axis=1) * (q.astype(np.float64) - np.repeat(z, g, axis=1))
    ref = (xq.astype(np.float64) * pts.astype(np.float64)[:, None]) @ w.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15)


def test_int4_pack_round_trip_and_pairs():
    _, q, _, z, g = _grouped(n=48, k=384, g=128)
    packed = oracle.pack_int4(q)
    assert np.array_equal(oracle.unpack_int4(packed, 48, 384), q)
    # high nibbles of the codes are ignored
    assert np.array_equal(oracle.pack_int4(q | 0xF0), packed)
    # (word >> 4i) & 0x000F000F holds the pair (k0 + 2i, k0 + 2i + 1)
    kb_per = 384 // 128
    for nb, kb, l, t in [(0, 0, 0, 0), (2, 2, 45, 3), (1, 1, 18, 1)]:
        word = int(packed[(nb * kb_per + kb) * 256 + 4 * l + t])
        col = 16 * nb + l % 16
        k0 = 128 * kb + 32 * (l // 16) + 8 * t
        for i in range(4):
            pair = (word >> (4 * i)) & 0x000F000F
            assert (pair & 0xF, pair >> 16) == (int(q[col, k0 + 2 * i]), int(q[col, k0 + 2 * i + 1]))
    zp = oracle.pack_int4_zeros(z)
    ng = z.shape[1]
    for c in (0, 7, 8, 47):
        for gi in range(ng):
            assert (int(zp[gi * 6 + c // 8]) >> (4 * (c % 8))) & 15 == int(z[c, gi])


def test_int4_evidence_bytes():
    """"linear_4bit/mod.rs" module doc: the fused path avoids an 8x expansion (f32 vs 4-bit)."""
    b = oracle.int4_evidence_bytes(32, 11008, 4096, 128)
    assert b["packed_weight_bytes"] == 22_544_384
    assert b["dequantized_weight_bytes"] == 180_355_072
    assert b["dequantized_weight_bytes"] == 8 * b["packed_weight_bytes"]
    assert b["sidecar_bytes"] == 704_512 + 176_128
    assert b["output_bytes"] == 704_512


# ---------------------------------------------------------------------------
# O5: A4W4
# ---------------------------------------------------------------------------
def test_a4w4_integer_inputs_are_their_own_codes():
    g = synthetic.rng(41)
    x = g.integers(-8, 8, (9, 70)).astype(np.float32)
    q = oracle.quant_int4_tensor(x, 1.0, 1e-5)
    assert np.array_equal(q, x.astype(np.int8))


def test_a4w4_quant_brute_force_and_saturation():
    d = synthetic.a4w4(40, 24, 96, seed=42)
    x = d["x"].float().numpy()
    for scale in (d["scale_a"], d["scale_a"] / 4, 0.0):
        q = oracle.quant_int4_tensor(x, scale, 1e-5)
        sp = float(max(np.float32(scale), np.float32(1e-5)))
        quo = (x.astype(np.float64) / sp).astype(np.float32)  # correctly rounded fp32 quotient
        ref = np.clip([round(Fraction(float(v))) for v in quo.ravel()], -8, 7).reshape(x.shape)
        assert np.array_equal(q, ref)
    q_small = oracle.quant_int4_tensor(x, d["scale_a"] / 4, 1e-5)
    assert (q_small == -8).any() and (q_small == 7).any()


def test_a4w4_dequant_brute_force():
    d = synthetic.a4w4(33, 20, 130, seed=43)
    x, w = d["x"].float().numpy(), d["w"].float().numpy()
    qa, qw, acc, y = oracle.a4w4(x, w, d["scale_a"], d["scale_w"], d["eps"])
    sa = float(oracle.effective_scale(d["scale_a"], d["eps"]))
    sw = float(oracle.effective_scale(d["scale_w"], d["eps"]))
    ref = (qa.astype(np.float64) * sa) @ (qw.astype(np.float64) * sw).T
    np.testing.assert_allclose(y, ref, rtol=1e-12)
    assert np.array_equal(acc.astype(np.int64), qa.astype(np.int64) @ qw.astype(np.int64).T)


# ---------------------------------------------------------------------------
# Output rounding
# ---------------------------------------------------------------------------
def _e3m2_value(c: int) -> float:
    """OCP MX FP6 E3M2: (-1)^s 2^(e-3) (1 + m/4), or 2^-2 (m/4) when e = 0."""
    s, e, m = (c >> 5) & 1, (c >> 2) & 7, c & 3
    v = (m / 4) * 2.0 ** -2 if e == 0 else (1 + m / 4) * 2.0 ** (e - 3)
    return -v if s else v


def _unpack_a4w4_fp6(buf: np.ndarray, rows: int, k: int) -> np.ndarray:
    """Decode the operand tiles by their written definition (slot l of tile
    (rb, ks): row 32rb + l%32, k 64ks + 32(l//32) + j, 6 bits per element,
    bytes 0..15 at 16l and 16..23 at 1024 + 8l)."""
    rp, kp = -(-rows // 32) * 32, -(-k // 128) * 128
    out = np.full((rp, kp), np.nan)
    for rb in range(rp // 32):
        for ks in range(kp // 64):
            t = (rb * (kp // 64) + ks) * 1536
            for l in range(64):
                img = bytes(buf[t + 16 * l:t + 16 * l + 16]) + bytes(buf[t + 1024 + 8 * l:t + 1024 + 8 * l + 8])
                bits = int.from_bytes(img, "little")
                for j in range(32):
                    out[32 * rb + l % 32, 64 * ks + 32 * (l // 32) + j] = _e3m2_value((bits >> (6 * j)) & 63)
    return out


def test_a4w4_fp6_operand_encodes_every_code_exactly():
    """Every 4-bit code is its own FP6 E3M2 value; padding rows and k hold 0."""
    codes = np.arange(-8, 8, dtype=np.int8).reshape(1, 16)
    buf = oracle.pack_a4w4_fp6(codes)
    assert buf.size == oracle.a4w4_operand_bytes(1, 16) == 32 * 128 * 3 // 4
    dec = _unpack_a4w4_fp6(buf, 1, 16)
    assert dec[0, :16].tolist() == list(range(-8, 8))
    assert np.all(dec[1:, :] == 0) and np.all(dec[0, 16:] == 0)


@pytest.mark.parametrize("rows,k", [(45, 200), (32, 128), (64, 256)])
def test_a4w4_fp6_operand_round_trip(rows, k):
    codes = synthetic.rng(50 + rows).integers(-8, 8, (rows, k), dtype=np.int8)
    dec = _unpack_a4w4_fp6(oracle.pack_a4w4_fp6(codes), rows, k)
    assert np.array_equal(dec[:rows, :k], codes.astype(np.float64))
    assert np.all(dec[rows:, :] == 0) and np.all(dec[:, k:] == 0)


def _unpack_a4w4_int4(buf, rows, k):
    """Decode the packed 4-bit operand by its written definition (tile (rb, ks)
    of 1024 bytes, slot l at byte 16l: row 32rb + l%32, k 64ks + 32(l//32) + j;
    element j in little-endian word j//8, nibble j%8//2 for even j%8 and
    4 + j%8//2 for odd, holding code + 8)."""
    rp, kp = -(-rows // 32) * 32, -(-k // 128) * 128
    out = np.full((rp, kp), np.nan)
    for rb in range(rp // 32):
        for ks in range(kp // 64):
            t = (rb * (kp // 64) + ks) * 1024
            for l in range(64):
                words = [int.from_bytes(bytes(buf[t + 16 * l + 4 * w:t + 16 * l + 4 * w + 4]), "little")
                         for w in range(4)]
                for j in range(32):
                    e = j % 8
                    nib = e // 2 if e % 2 == 0 else 4 + e // 2
                    out[32 * rb + l % 32, 64 * ks + 32 * (l // 32) + j] = ((words[j // 8] >> (4 * nib)) & 15) - 8
    return out


def test_a4w4_int4_operand_encodes_every_code_exactly():
    """Two codes per byte: every code in [-8, 7] is stored as code + 8; padding holds code 0."""
    codes = np.arange(-8, 8, dtype=np.int8).reshape(1, 16)
    buf = oracle.pack_a4w4_int4(codes)
    assert buf.size == oracle.a4w4_packed_bytes(1, 16) == 32 * 128 // 2
    assert oracle.a4w4_packed_bytes(8192, 8192) * 3 == oracle.a4w4_operand_bytes(8192, 8192) * 2
    dec = _unpack_a4w4_int4(buf, 1, 16)
    assert dec[0, :16].tolist() == list(range(-8, 8))
    assert np.all(dec[1:, :] == 0) and np.all(dec[0, 16:] == 0)
    # slot 0's first word holds elements 0..7 as nibbles (0, 2, 4, 6, 1, 3, 5, 7)
    w0 = int.from_bytes(bytes(buf[0:4]), "little")
    assert [(w0 >> (4 * p)) & 15 for p in range(8)] == [0, 2, 4, 6, 1, 3, 5, 7]


@pytest.mark.parametrize("rows,k", [(45, 200), (32, 128), (64, 256), (1, 1)])
def test_a4w4_int4_operand_round_trip_and_matches_fp6(rows, k):
    codes = synthetic.rng(60 + rows).integers(-8, 8, (rows, k), dtype=np.int8)
    dec = _unpack_a4w4_int4(oracle.pack_a4w4_int4(codes), rows, k)
    assert np.array_equal(dec[:rows, :k], codes.astype(np.float64))
    assert np.all(dec[rows:, :] == 0) and np.all(dec[:, k:] == 0)
    # the same tile grid as the FP6 operand: both decode to the same padded code matrix
    assert np.array_equal(dec, _unpack_a4w4_fp6(oracle.pack_a4w4_fp6(codes), rows, k))


def _q4_autograd(g, x, w, sa, sw, eps):
    """Straight-through fake quantization in torch fp64 autograd: clamp passes
    the gradient inside [-8, 7] only, round passes it unchanged."""
    f64 = torch.float64
    sa_t = torch.tensor(float(np.float32(sa)), dtype=f64, requires_grad=True)
    x_t = torch.tensor(x, dtype=f64, requires_grad=True)
    w_t = torch.tensor(w, dtype=f64, requires_grad=True)
    e = torch.tensor(float(np.float32(eps)), dtype=f64)

    def fake(t, s):
        v = torch.clamp(t / s, -8.0, 7.0)
        return (v + (torch.round(v) - v).detach()) * s

    y = fake(x_t, torch.maximum(sa_t, e)) @ fake(w_t, torch.maximum(torch.tensor(float(np.float32(sw)), dtype=f64), e)).T
    y.backward(torch.tensor(g, dtype=f64))
    return x_t.grad.numpy(), w_t.grad.numpy(), float(sa_t.grad)


@pytest.mark.parametrize("m,n,k,clip", [(5, 7, 9, 0.5), (16, 12, 40, 1.0), (33, 17, 64, 0.3)])
def test_q4_backward_matches_autograd(m, n, k, clip):
    """torch autograd of the straight-through fake-quantized linear layer."""
    r = synthetic.rng(60 + m)
    x = r.normal(0, 1, (m, k)).astype(np.float16).astype(np.float32)
    w = (0.02 * r.normal(0, 1, (n, k))).astype(np.float16).astype(np.float32)
    g = r.normal(0, 1, (m, n)).astype(np.float16).astype(np.float64)
    sa = float(np.abs(x).max() / 7 * clip)
    sw = float(np.abs(w).max() / 7 * clip)
    gx, gw, gs, bx, bw, bs = oracle.q4_backward(g, x, w, sa, sw, 1e-5)
    ax, aw, asa = _q4_autograd(g, x, w, sa, sw, 1e-5)
    np.testing.assert_allclose(gx, ax, rtol=1e-12, atol=1e-12 * bx.max())
    np.testing.assert_allclose(gw, aw, rtol=1e-12, atol=1e-12 * bw.max())
    # the oracle's quotient v is fl32(x / s'), autograd's the fp64 one: they differ by at most
    # 2^-24 |v| <= 2^-24 * 8.5 inside the range, and each term carries |dXh| <= bx
    assert abs(gs - asa) <= 2.0 ** -24 * 8.5 * bx.sum() + 1e-12
    if clip < 1.0:
        assert np.count_nonzero(gx == 0) > 0 and np.count_nonzero(gw == 0) > 0


def test_q4_backward_special_cases():
    """Scale below eps: no scale gradient.  Inputs on the code grid inside the
    range: the step size term vanishes and grad_x is the plain G Wh."""
    r = synthetic.rng(70)
    m, n, k = 6, 5, 8
    g = r.normal(0, 1, (m, n))
    x = r.integers(-8, 8, (m, k)).astype(np.float32) * 0.25
    w = r.integers(-8, 8, (n, k)).astype(np.float32) * 0.5
    gx, gw, gs, _, _, _ = oracle.q4_backward(g, x, w, 0.25, 0.5, 1e-5)
    assert gs == 0.0
    np.testing.assert_allclose(gx, g @ w, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gw, g.T @ x, rtol=1e-13, atol=1e-13)
    _, _, gs0, _, _, _ = oracle.q4_backward(g, x * 1e-9, w, 1e-7, 0.5, 1e-5)
    assert gs0 == 0.0


def test_round_f16_matches_numpy():
    g = synthetic.rng(51)
    v = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-9, 6, 20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -70000.0, 2.0 ** -24, 2.0 ** -25,
                         3 * 2.0 ** -26, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]])
    got = oracle.round_f16(v)
    assert np.array_equal(got, v.astype(np.float16).view(np.uint16))


def test_round_bf16_matches_torch_on_fp32_values():
    g = synthetic.rng(52)
    v32 = (g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000)).astype(np.float32)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0e38, 1e-40], np.float32)
    v32 = np.concatenate([v32, ties])
    got = oracle.round_bf16(v32.astype(np.float64))
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert got[-5] == 0x3F80 and got[-4] == 0x3F82   # ties go to the even mantissa
