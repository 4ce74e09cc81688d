"""CPU tier: the oracle and the host side of the C ABI under AddressSanitizer
and UndefinedBehaviorSanitizer.

Builds (in a temporary directory) the oracle with clang
-fsanitize=address,undefined, and libqlinear with its host code (argument
validation, dispatch) sanitized the same way -- the device code is built as
usual -- then runs the oracle pins and the ABI validation tests in a child
process with the sanitizer runtime preloaded.  Any out-of-bounds access, use
after free or undefined behaviour (signed overflow, bad shift, invalid
float-to-int conversion) aborts the child and fails this test.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
PKG = os.path.join(ROOT, "bit_quantized_linear_quant_amd")


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_oracle_and_abi_host_code_under_asan_ubsan(tmp_path):
    clang = os.path.join(LLVM, "bin", "clang")
    hipcc = "/opt/rocm/bin/hipcc"
    rt = _asan_runtime()
    if not (os.path.exists(clang) and os.path.exists(hipcc) and rt):
        pytest.skip("clang, hipcc or the ASan runtime is not installed")
    sys.path.insert(0, PKG)
    from bit_quantized_linear_quant_amd import build as qb   # noqa: E402

    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    # the oracle, plain C (OpenMP pragmas ignored: the loops are then sequential)
    ora = str(tmp_path / "liboracle_asan.so")
    subprocess.run([clang, "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    *san, os.path.join(ROOT, "oracle", "qlinear_oracle.c"), "-o", ora, "-lm"], check=True)
    # libqlinear: every source with its host pass sanitized (-Xarch_host before each flag)
    host_san = [f for flag in san for f in ("-Xarch_host", flag)]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        subprocess.run([hipcc, *qb.compile_flags(), *host_san, "-c", os.path.join(qb.CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(min(len(qb.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, qb.SOURCES))
    lib = str(tmp_path / "libqlinear_asan.so")
    subprocess.run([hipcc, f"--offload-arch={qb.ARCH}", "-shared", "-fPIC", "-shared-libsan",
                    "-fsanitize=address,undefined", *objs, "-o", lib], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, QLINEAR_LIB=lib, QLINEAR_ORACLE_LIB=ora,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p",
                          "no:cacheprovider", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
