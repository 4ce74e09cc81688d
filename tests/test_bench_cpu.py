"""CPU tier: bench.py's contract pieces that need no GPU.

It refuses more than one GPU with a message, its per-row figures follow
from their inputs (rate = work / time, fraction = rate / peak), and the
recorded HBM traffic is looked up only for the kernel source it was measured
on.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_row_rate_and_fraction():
    r = bench._row(10.0, 8e7, "GB/s", 8000.0, "hbm", "80 MB in 10 us")
    assert r["achieved"] == 8000.0 and r["frac"] == 1.0 and r["unit"] == "GB/s"
    r = bench._row(2.0, 1e10, "TOPS", 5000.0, "mfma", "1e10 ops in 2 us", oracle_rate=0.5, oracle_sample="s")
    assert r["achieved"] == 5000.0 and r["frac"] == 1.0
    assert r["oracle"] == {"value": 0.5, "unit": "TOPS", "sample": "s"}
    r = bench._row(3.0, 1e6, "TOPS", None, "launch", "tiny")
    assert "frac" not in r and "peak" not in r


def test_recorded_traffic_is_tied_to_the_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# comment line\n"
                 "kernel=k1 src=aaaa fetch_bytes=100 write_bytes=20 fetch_kib_raw=1 write_kib_raw=1 dispatches=3\n"
                 "kernel=k2 src=bbbb fetch_bytes=7 write_bytes=0 fetch_kib_raw=1 write_kib_raw=0 dispatches=1\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("k1", "aaaa") == 120
    assert bench.recorded_traffic("k2", "bbbb") == 7
    assert bench.recorded_traffic("k1", "bbbb") is None      # another source: not this kernel's bytes
    assert bench.recorded_traffic("k3", "aaaa") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic("k1", "aaaa") is None


def test_source_hash_covers_every_listed_file():
    h = bench.kernel_source_hash(bench.GEMM_KERNEL_SOURCES)
    assert len(h) == 16 and h == bench.kernel_source_hash(list(bench.GEMM_KERNEL_SOURCES))
    assert h != bench.kernel_source_hash(bench.GEMM_KERNEL_SOURCES[:-1])
