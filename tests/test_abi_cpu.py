"""CPU tier: libqlinear loads, exports every entry point of include/qlinear.h,
and rejects invalid arguments on the host before any HIP call.

No test here reaches a kernel launch: every call below fails validation (fake
but aligned addresses are never dereferenced by the host checks).
"""
import ctypes
import os
import re
import subprocess

import pytest

import bit_quantized_linear_quant_amd as ql
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000      # aligned fake device address (never dereferenced)
U = 0x10008      # misaligned fake address
NULL = None


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ql.LIB_PATH):
        pytest.fail(f"{ql.LIB_PATH} is not built (run __graft_entry__.build())")
    return ql.lib()


def test_exports_every_declared_symbol(L):
    declared = ql.declared_functions()
    assert len(declared) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", ql.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (qlinear_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for f in declared:
        assert hasattr(L, f)


def test_abi_version_and_status_strings(L):
    assert ql.qlinear_abi_version() == ql.ABI_VERSION == 8
    for code, name in ql.STATUS.items():
        s = ql.qlinear_status_string(code)
        assert isinstance(s, str) and s
    assert ql.qlinear_status_string(-99) == "unknown status"


def test_workspace_bytes():
    # a4w4: codes of x then w, each rounded to 256 bytes
    assert ql.qlinear_workspace_bytes(ql.QL_OP_GEMM_A4W4, 8192, 8192, 8192) == 2 * 8192 * 8192 * 3 // 4
    # 3 and 5 rows pad to 32, k = 7 to 128: 32 * 128 * 3/4 = 3072 bytes each
    assert ql.qlinear_workspace_bytes(ql.QL_OP_GEMM_A4W4, 3, 5, 7) == 3072 + 3072
    for rows, k in [(1, 1), (45, 200), (8192, 8192), (33, 129)]:
        assert ql.qlinear_workspace_bytes(ql.QL_OP_A4W4_OPERAND, rows, 0, k) == oracle.a4w4_operand_bytes(rows, k)
    # ternary: one fp64 partial per 16384-element chunk, rounded to 256 bytes
    assert ql.qlinear_workspace_bytes(ql.QL_OP_PACK_TERNARY, 0, 16, 256) == 256
    chunks = (28672 * 8192 + 16383) // 16384
    assert ql.qlinear_workspace_bytes(ql.QL_OP_PACK_TERNARY, 0, 28672, 8192) == (chunks * 8 + 255) // 256 * 256
    assert ql.qlinear_workspace_bytes(99, 1, 1, 1) == 0
    # the packed 4-bit operand: half a byte per padded element
    for rows, k in [(1, 1), (45, 200), (8192, 8192), (33, 129)]:
        assert ql.qlinear_workspace_bytes(ql.QL_OP_A4W4_PACKED, rows, 0, k) == oracle.a4w4_packed_bytes(rows, k)
    assert ql.qlinear_workspace_bytes(ql.QL_OP_A4W4_PACKED, 8192, 0, 8192) == 8192 * 8192 // 2


def test_quant_act_validation(L):
    f = L.qlinear_quant_act
    assert f(NULL, ql.QL_BF16, 4, 8, 0, 1e-6, 1e-5, A, A, A, NULL) == -1
    assert f(A, ql.QL_BF16, 0, 8, 0, 1e-6, 1e-5, A, A, A, NULL) == -2      # empty
    assert f(A, ql.QL_BF16, 4, 0, 0, 1e-6, 1e-5, A, A, A, NULL) == -2
    assert f(A, ql.QL_I8, 4, 8, 0, 1e-6, 1e-5, A, A, A, NULL) == -3
    assert f(U, ql.QL_BF16, 4, 8, 0, 1e-6, 1e-5, A, A, A, NULL) == -4
    assert f(A, ql.QL_BF16, 4, 8, 0x10, 1e-6, 1e-5, A, A, A, NULL) == -6   # unknown flag
    # the int32 code sum of a row (at most 127 k in magnitude) must fit int32
    assert f(A, ql.QL_BF16, 4, 16909321, 0, 1e-6, 1e-5, A, A, A, NULL) == -2
    assert 127 * 16909320 < 2 ** 31 <= 127 * 16909321
    # eps_q guards a division: positive and finite; eps_norm finite and >= 0
    for eq in (0.0, -1e-5, float("nan"), float("inf")):
        assert f(A, ql.QL_BF16, 4, 8, 0, 1e-6, eq, A, A, A, NULL) == -6
    for en in (-1e-6, float("nan"), float("inf")):
        assert f(A, ql.QL_BF16, 4, 8, 1, en, 1e-5, A, A, A, NULL) == -6


def test_quant_int4_validation(L):
    f = L.qlinear_quant_int4_tensor
    assert f(A, ql.QL_F16, 16, NULL, 1e-5, A, NULL) == -1
    assert f(A, ql.QL_F16, 0, A, 1e-5, A, NULL) == -2
    assert f(A, ql.QL_I32, 16, A, 1e-5, A, NULL) == -3
    assert f(A, ql.QL_F16, 16, A, 1e-5, U, NULL) == -4


def test_pack_validation(L):
    f = L.qlinear_pack_ternary
    assert f(NULL, ql.QL_W_NK, 16, 256, 1e-5, A, A, A, 1 << 20, NULL) == -1
    assert f(A, ql.QL_W_NK, 17, 256, 1e-5, A, A, A, 1 << 20, NULL) == -2   # n % 16
    assert f(A, ql.QL_W_NK, 16, 300, 1e-5, A, A, A, 1 << 20, NULL) == -2   # k % 256
    assert f(A, ql.QL_W_NK, 16, 256, 1e-5, A, A, NULL, 1 << 20, NULL) == -5
    assert f(A, ql.QL_W_NK, 16, 256, 1e-5, A, A, A, 8, NULL) == -5         # too small
    assert f(A, 7, 16, 256, 1e-5, A, A, A, 1 << 20, NULL) == -6
    nf = L.qlinear_pack_ternary_noalloc
    assert nf(NULL, ql.QL_W_NK, 16, 256, 1e-5, A, A, NULL) == -1
    assert nf(A, ql.QL_W_NK, 17, 256, 1e-5, A, A, NULL) == -2
    assert nf(A, ql.QL_W_NK, 16, 300, 1e-5, A, A, NULL) == -2
    assert nf(A, 7, 16, 256, 1e-5, A, A, NULL) == -6
    assert nf(A, ql.QL_W_NK, 16, 256, 1e-5, U, A, NULL) == -4
    # more than 2^31 weights: beyond the static scratch, rejected before any HIP call
    assert nf(A, ql.QL_W_NK, 2 ** 23 + 16, 256, 1e-5, A, A, NULL) == -5
    assert nf(A, ql.QL_W_NK, 1 << 40, 256, 1e-5, A, A, NULL) == -5
    g = L.qlinear_pack_int4
    assert g(A, 16, 100, ql.QL_INT4_WEIGHT, A, NULL) == -2
    assert g(A, 12, 4, ql.QL_INT4_ZEROS, A, NULL) == -2
    assert g(A, 16, 128, 5, A, NULL) == -6
    assert g(U, 16, 128, ql.QL_INT4_WEIGHT, A, NULL) == -4


def test_gemm_validation(L):
    w8 = L.qlinear_gemm_w8a8
    assert w8(A, A, ql.QL_W_KN, A, A, NULL, 2, 3, 2, ql.QL_BF16, NULL, NULL) == -1
    assert w8(A, A, ql.QL_W_KN, NULL, A, NULL, 2, 3, 2, ql.QL_F16, A, NULL) == -1   # scales needed
    assert w8(A, A, ql.QL_W_KN, A, A, NULL, 2, 3, 131072, ql.QL_F16, A, NULL) == -2  # int32 could overflow
    assert w8(A, A, ql.QL_W_KN, A, A, NULL, 0, 3, 2, ql.QL_F16, A, NULL) == -2
    assert w8(A, A, ql.QL_W_KN, A, A, NULL, 2, 3, 2, ql.QL_U8, A, NULL) == -3
    assert w8(A, A, 3, A, A, NULL, 2, 3, 2, ql.QL_F16, A, NULL) == -6
    assert w8(A, A, ql.QL_W_KN, A, A, A, 2, 3, 2, ql.QL_I32, A, NULL) == -6  # bias on the raw accumulator
    assert w8(A, A, ql.QL_W_KN, A, A, U, 2, 3, 2, ql.QL_F16, A, NULL) == -4
    wb = L.qlinear_gemm_w8a8_batched
    assert wb(A, A, ql.QL_W_NK, A, 0, A, NULL, 0, 2, 3, 2, ql.QL_F16, A, NULL) == -2      # batch 0
    assert wb(A, A, ql.QL_W_NK, A, 0, A, NULL, 65536, 2, 3, 2, ql.QL_F16, A, NULL) == -2  # grid z limit
    assert wb(A, A, ql.QL_W_NK, A, 5, A, NULL, 2, 2, 3, 2, ql.QL_F16, A, NULL) == -2      # deq stride not 0 or n
    assert wb(A, A, ql.QL_W_NK, NULL, 0, A, NULL, 2, 2, 3, 2, ql.QL_F16, A, NULL) == -1
    assert wb(A, A, ql.QL_W_NK, A, 3, A, A, 2, 2, 3, 2, ql.QL_I32, A, NULL) == -6
    assert wb(U, A, ql.QL_W_NK, A, 3, A, NULL, 2, 2, 3, 2, ql.QL_F16, A, NULL) == -4
    w2 = L.qlinear_gemm_w2a8
    assert w2(A, A, NULL, A, A, NULL, 1, 16, 256, ql.QL_BF16, A, NULL) == -1
    assert w2(A, A, A, A, A, NULL, 1, 24, 256, ql.QL_BF16, A, NULL) == -2
    assert w2(A, A, A, A, A, NULL, 1, 16, 128, ql.QL_BF16, A, NULL) == -2
    assert w2(A, A, A, U, A, NULL, 1, 16, 256, ql.QL_BF16, A, NULL) == -4
    assert w2(A, A, A, A, A, A, 1, 16, 256, ql.QL_I32, A, NULL) == -6
    assert w2(A, A, A, A, A, U, 1, 16, 256, ql.QL_BF16, A, NULL) == -4
    g4 = L.qlinear_gemm_w4a8_grouped
    assert g4(A, ql.QL_I8, NULL, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -1  # needs pts
    assert g4(A, ql.QL_I8, U, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -4
    assert g4(A, ql.QL_I8, A, A, A, A, 128, 1, 16, 128, NULL, ql.QL_I32, A, NULL) == -3
    assert g4(A, ql.QL_U8, A, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -3
    gb = L.qlinear_gemm_w4a8_grouped_batched
    assert gb(0, A, ql.QL_F16, NULL, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -2      # batch 0
    assert gb(65536, A, ql.QL_F16, NULL, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -2  # grid z limit
    assert gb(2, A, ql.QL_I8, NULL, A, A, A, 128, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -1       # needs pts
    assert gb(2, A, ql.QL_F16, NULL, A, A, A, 128, 1, 24, 128, NULL, ql.QL_F16, A, NULL) == -2      # n % 16
    assert gb(2, A, ql.QL_F16, NULL, A, A, A, 128, 1, 16, 128, U, ql.QL_F16, A, NULL) == -4         # bias alignment
    assert g4(A, ql.QL_F16, NULL, A, A, A, 48, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -2   # group % 32
    assert g4(A, ql.QL_F16, NULL, A, A, A, 16, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -2
    assert g4(A, ql.QL_F16, NULL, A, A, A, 0, 1, 16, 128, NULL, ql.QL_F16, A, NULL) == -2
    assert g4(A, ql.QL_F16, NULL, A, A, A, 256, 1, 16, 384, NULL, ql.QL_F16, A, NULL) == -2  # k % group
    assert g4(A, ql.QL_F16, NULL, A, A, A, 96, 1, 16, 320, NULL, ql.QL_F16, A, NULL) == -2   # k % 128
    assert g4(A, ql.QL_F16, NULL, A, A, A, 64, 1, 16, 128, NULL, ql.QL_U8, A, NULL) == -3    # 32 | 64 accepted
    assert g4(A, ql.QL_F16, NULL, A, A, A, 128, 1, 16, 128, U, ql.QL_F16, A, NULL) == -4  # bias alignment
    assert g4(A, ql.QL_F16, NULL, A, A, A, 128, 1, 16, 128, NULL, ql.QL_BF16, A, NULL) == -3
    qo = L.qlinear_quant_a4w4_operand
    assert qo(A, ql.QL_F16, 4, 8, NULL, 1e-5, A, NULL) == -1
    assert qo(A, ql.QL_I8, 4, 8, A, 1e-5, A, NULL) == -3
    assert qo(A, ql.QL_F16, 0, 8, A, 1e-5, A, NULL) == -2
    assert qo(A, ql.QL_F16, 4, 131072, A, 1e-5, A, NULL) == -2
    assert qo(A, ql.QL_F16, 4, 8, A, 1e-5, U, NULL) == -4
    qp = L.qlinear_quant_a4w4_packed
    assert qp(A, ql.QL_F16, 4, 8, NULL, 1e-5, A, NULL) == -1
    assert qp(A, ql.QL_I8, 4, 8, A, 1e-5, A, NULL) == -3
    assert qp(A, ql.QL_F16, 0, 8, A, 1e-5, A, NULL) == -2
    assert qp(A, ql.QL_F16, 4, 131072, A, 1e-5, A, NULL) == -2
    assert qp(A, ql.QL_F16, 4, 8, A, 1e-5, U, NULL) == -4
    gp = L.qlinear_gemm_a4w4_packed
    assert gp(A, A, NULL, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL) == -1
    assert gp(A, A, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, NULL) == -3
    assert gp(A, A, A, A, 1e-5, 4, 0, 4, ql.QL_F16, A, NULL) == -2
    assert gp(A, A, A, A, 1e-5, 4, 4, 131072, ql.QL_F16, A, NULL) == -2
    assert gp(U, A, A, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL) == -4
    go = L.qlinear_gemm_a4w4_operands
    assert go(A, A, NULL, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL) == -1
    assert go(A, A, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, NULL) == -3
    assert go(A, A, A, A, 1e-5, 4, 0, 4, ql.QL_F16, A, NULL) == -2
    assert go(U, A, A, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL) == -4
    qb = L.qlinear_q4_backward
    assert qb(A, A, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, A, NULL, A, 1 << 20, NULL) == -1
    assert qb(A, A, A, ql.QL_F32, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, A, A, A, 1 << 20, NULL) == -3
    assert qb(A, A, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_I32, A, A, A, A, 1 << 20, NULL) == -3
    assert qb(A, A, A, ql.QL_F16, A, A, 1e-5, 0, 4, 4, ql.QL_F32, A, A, A, A, 1 << 20, NULL) == -2
    assert qb(A, A, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, A, A, A, 10, NULL) == -5
    assert qb(A, U, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, A, A, A, 1 << 20, NULL) == -4
    a4 = L.qlinear_gemm_a4w4
    assert a4(A, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL, 0, NULL) == -5
    assert a4(A, A, ql.QL_F16, A, A, 1e-5, 4, 4, 4, ql.QL_F16, A, A, 100, NULL) == -5
    assert a4(A, A, ql.QL_I8, A, A, 1e-5, 4, 4, 4, ql.QL_F16, A, A, 1 << 20, NULL) == -3
    ac = L.qlinear_gemm_a4w4_codes
    assert ac(A, A, NULL, A, 1e-5, 4, 4, 4, ql.QL_F16, A, NULL) == -1
    assert ac(A, A, A, A, 1e-5, 4, 4, 4, ql.QL_F32, A, NULL) == -3


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        ql.qlinear_quant_act(torch.zeros(2, 8, dtype=torch.bfloat16))


def test_product_path_does_not_touch_the_oracle():
    """The library and its binding neither import nor link the CPU oracle."""
    pkg = os.path.join(ROOT, "bit_quantized_linear_quant_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "qlinear_oracle" not in text and "liboracle" not in text, fn
    out = subprocess.run(["nm", "-D", ql.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle_" not in out


def test_hbm_read_stream_validation(L):
    f = L.qlinear_hbm_read_stream
    assert f(NULL, 16, A, NULL) == -1
    assert f(A, 16, NULL, NULL) == -1
    assert f(A, 0, A, NULL) == -2          # empty
    assert f(A, 24, A, NULL) == -2         # not whole 16-byte chunks
    assert f(U, 16, A, NULL) == -4
    assert f(A, 16, U, NULL) == -4


def test_hbm_stream_sink_words_match_header():
    with open(os.path.join(ROOT, "include", "qlinear.h")) as f:
        words = int(re.search(r"#define QL_HBM_STREAM_SINK_WORDS (\d+)", f.read()).group(1))
    assert words == ql.QL_HBM_STREAM_SINK_WORDS
