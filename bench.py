"""Benchmark of the quantized linear layer on one MI355X.

Step: one Q4Linear (A4W4) forward on the 8192^3 workload -- per-tensor 4-bit
quantization of x[8192,8192] and w[8192,8192] (fp16) into packed FP6 E3M2
operands (every 4-bit code is exact in E3M2), then the FP6 matrix-core product
with exact fp32 accumulation and the fused fp16 epilogue -- the large-M GEMM
that the metric's integer TOPS figure is quoted on.  Inputs are resident in
HBM before the timed region; W untimed warm-up steps precede exactly K timed
steps bracketed by device synchronization.

The same JSON line carries:
  roofline      the FP6 GEMM kernel: algorithmic ops per launch / its mean
                duration from HIP events recorded around it in the timed
                region, against the 10.1 PFLOP/s dense FP6 matrix-core peak
                (the dtype it computes in); `traffic` is the HBM bytes per
                launch measured by rocprofv3 counters for the current kernel
                source, else null.
  cpu_baseline  the CPU oracle timed on this host on a bounded row sample of
                the same forward, scaled to TOPS.
  decode_gemv   the metric's second figure: packed-ternary-weight HBM GB/s of
                the M<=16 decode GEMV (K=8192, N=28672) for M in {1,4,16},
                with the packed weight rotated over copies larger than the
                256 MB last-level cache, launches replayed from a HIP graph;
                each M also with its single-launch latency (one eager launch
                timed alone) and its share of the stream floor: the same
                weight bytes read by a plain HBM read stream
                (qlinear_hbm_read_stream), per launch in the same graph
                rotation, and once over all copies in one launch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only PART]

--only runs one part by itself and prints its figures (no headline line):
the rocprofv3 counter runs recorded under profiles/ use it so that a
counter pass sees only the kernels it is about.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 TOPS (large-M GEMM) + packed-weight HBM GB/s (M≤16 GEMV), % roofline"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 / FP4 MFMA, 10.1 PFLOP/s
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA, 2.5 PFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
GEMM_KERNEL_SOURCES = ["gemm_i8.hip", "gemm_ring.hpp", "ql_device.hpp"]
GEMV_KERNEL_SOURCES = ["gemm_w2a8.hip", "ql_device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_quantized_linear_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(name: str, src_hash: str):
    """HBM bytes per launch measured by rocprofv3 for this kernel source, else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = dict(p.split("=", 1) for p in line.split() if "=" in p)
            if parts.get("kernel") == name and parts.get("src") == src_hash:
                return int(parts["fetch_bytes"]) + int(parts["write_bytes"])
    return None


def cpu_baseline(d, target_s: float = 12.0):
    """The CPU oracle on a row sample of the same forward, scaled to TOPS."""
    import numpy as np
    import oracle

    x = d["x"].float().numpy()
    w = d["w"].float().numpy()
    m, k = x.shape
    n = w.shape[0]
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def run(rows):
        t0 = time.perf_counter()
        qa = oracle.quant_int4_tensor(x[:rows], d["scale_a"], d["eps"])
        qw = oracle.quant_int4_tensor(w, d["scale_w"], d["eps"])
        acc = oracle.gemm_i8(qa, qw, True)
        sa = float(oracle.effective_scale(d["scale_a"], d["eps"]))
        sw = float(oracle.effective_scale(d["scale_w"], d["eps"]))
        y = acc.astype(np.float64) * sa * sw
        oracle.round_f16(y)
        return time.perf_counter() - t0

    # calibrate: a fixed part (quantizing all of w) plus a per-row part
    t8, t24 = run(8), run(24)
    per_row = max((t24 - t8) / 16, 1e-6)
    fixed = max(t8 - 8 * per_row, 0.0)
    rows = int(min(m, max(8, (target_s - fixed) / per_row)))
    rows = max(8, rows // 8 * 8)
    t = run(rows)
    return {"value": 2.0 * rows * n * k / t / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {m} token rows of the A4W4 forward (x-row and full-w 4-bit quantization, "
                      f"integer product over k={k} for all n={n} columns, fp64 dequant, fp16 rounding); "
                      f"{t:.1f} s on {threads} threads"}


def bench_a4w4(args, ql, torch, synthetic):
    dev = "cuda:0"
    m = n = k = 8192
    d = synthetic.a4w4(m, n, k, seed=1005)
    x = d["x"].to(dev)
    w = d["w"].to(dev)
    sa = torch.tensor([d["scale_a"]], dtype=torch.float32, device=dev)
    sw = torch.tensor([d["scale_w"]], dtype=torch.float32, device=dev)
    eps = d["eps"]
    out = torch.empty((m, n), dtype=torch.float16, device=dev)
    ws = torch.empty((ql.qlinear_workspace_bytes(ql.QL_OP_GEMM_A4W4, m, n, k),), dtype=torch.uint8, device=dev)
    xa, wb = ql.a4w4_operands_from_workspace(ws, m, n, k)

    # A plain device copy of known size: the byte counters' calibration kernel.
    cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)

    def step(ev=None):
        # the three launches of qlinear_gemm_a4w4, with events between them
        if ev is not None:
            ev[0].record()
        ql.qlinear_quant_a4w4_operand(x, sa, eps, operand=xa)
        if ev is not None:
            ev[1].record()
        ql.qlinear_quant_a4w4_operand(w, sw, eps, operand=wb)
        if ev is not None:
            ev[2].record()
        ql.qlinear_gemm_a4w4_operands(xa, wb, m, n, k, sa, sw, eps, out_dtype=torch.float16, out=out)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    qx = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    qw = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    gm = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    ops = 2.0 * m * n * k
    ms_per_step = wall * 1e3 / args.steps
    # the int8-code product of the same codes (qlinear_gemm_a4w4_codes), for comparison
    xq = ql.qlinear_quant_int4_tensor(x.view(-1), sa, eps).view(m, k)
    wq = ql.qlinear_quant_int4_tensor(w.view(-1), sw, eps).view(n, k)
    ql.qlinear_gemm_a4w4_codes(xq, wq, sa, sw, eps, out_dtype=torch.float16, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        ql.qlinear_gemm_a4w4_codes(xq, wq, sa, sw, eps, out_dtype=torch.float16, out=out)
    e1.record()
    torch.cuda.synchronize()
    i8 = e0.elapsed_time(e1) / 10
    del xq, wq
    # the same product on two-codes-per-byte operands (qlinear_gemm_a4w4_packed)
    xp = ql.qlinear_quant_a4w4_packed(x, sa, eps)
    wp = ql.qlinear_quant_a4w4_packed(w, sw, eps)
    ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, sa, sw, eps, out_dtype=torch.float16, out=out)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        ql.qlinear_gemm_a4w4_packed(xp, wp, m, n, k, sa, sw, eps, out_dtype=torch.float16, out=out)
    e1.record()
    torch.cuda.synchronize()
    pk = e0.elapsed_time(e1) / 10
    e0.record()
    for _ in range(5):
        ql.qlinear_quant_a4w4_packed(x, sa, eps, operand=xp)
    e1.record()
    torch.cuda.synchronize()
    pq = e0.elapsed_time(e1) / 5
    del xp, wp
    res = {"m": m, "n": n, "k": k, "ops": ops, "ms_per_step": ms_per_step,
           "value": ops / (ms_per_step * 1e-3) / 1e12,
           "kernel_ms": {"quant_x": qx, "quant_w": qw, "gemm": gm},
           "gemm_tops": ops / (gm * 1e-3) / 1e12,
           "int8_codes_gemm": {"ms": round(i8, 4), "TOPS": round(ops / (i8 * 1e-3) / 1e12, 1),
                               "frac_int8_peak": round(ops / (i8 * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                               "kernel": "gemm_i8_big_kernel (qlinear_gemm_a4w4_codes), same codes held in int8"},
           "packed_operands_gemm": {"ms": round(pk, 4), "TOPS": round(ops / (pk * 1e-3) / 1e12, 1),
                                    "frac_fp6_peak": round(ops / (pk * 1e-3) / 1e12 / PEAK_FP6_TOPS, 4),
                                    "quant_ms_per_tensor": round(pq, 4),
                                    "kernel": "gemm_a4w4_packed_kernel (qlinear_gemm_a4w4_packed): operands "
                                              "at two 4-bit codes per byte, expanded to FP6 on the way into LDS"}}
    return res, d


def bench_decode(ql, torch, synthetic, reps: int = 10):
    """Packed-weight GB/s of the M<=16 decode GEMV, weights rotated past the last-level cache."""
    dev = "cuda:0"
    n, k = 28672, 8192
    dd = synthetic.decode((1, 4, 16), n, k, seed=1003)
    packed, gamma = ql.qlinear_pack_ternary(dd["w"].to(dev), ql.QL_W_NK)
    copies = [packed] + [packed.clone() for _ in range(5)]     # 6 x 58.7 MB > 256 MB cache
    packed_bytes = n * k // 4
    res = {}
    for m, x in dd["x"].items():
        xq, pts, rs = ql.qlinear_quant_act(x.to(dev), rmsnorm=True)
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        launches = 4 * len(copies)
        for c in copies:   # warm-up outside capture
            ql.qlinear_gemm_w2a8(xq, pts, rs, c, gamma, n, out=out)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                ql.qlinear_gemm_w2a8(xq, pts, rs, copies[i % len(copies)], gamma, n, out=out)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * launches)
        gbs = packed_bytes / (us * 1e-6) / 1e9
        single = time_single(torch, lambda i: ql.qlinear_gemm_w2a8(xq, pts, rs, copies[i % len(copies)], gamma, n,
                                                                   out=out))
        res[str(m)] = {"us_per_launch": round(us, 3), "packed_weight_GBps": round(gbs, 1),
                       "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "single_launch_us": round(single, 3)}
        del g
    floor = stream_floor(ql, torch, copies, packed_bytes, reps)
    for m in res:
        res[m]["frac_of_stream_floor"] = round(floor["per_launch_us"] / res[m]["us_per_launch"], 4)
    return {"unit": "GB/s", "n": n, "k": k, "packed_weight_bytes": packed_bytes,
            "timing": "per launch, mean over HIP-graph replays of 24 back-to-back launches rotating 6 "
                      "copies of the packed weight (352 MB); single_launch_us: median of 24 eager launches "
                      "each timed alone (events around it, device idle before it)",
            "by_m": res, "stream_floor": floor}


def stream_floor(ql, torch, copies, nbytes: int, reps: int = 10):
    """The HBM read ceiling of the decode weight stream (qlinear_hbm_read_stream).

    One launch over a 6x larger buffer gives the sustained read rate; the same
    HIP-graph rotation as the GEMV, one copy per launch, gives the per-launch
    floor that includes the launch's ramp-up and drain.
    """
    big = torch.empty((len(copies) * nbytes,), dtype=torch.uint8, device=copies[0].device)
    for i, c in enumerate(copies):
        big[i * nbytes:(i + 1) * nbytes].copy_(c.view(torch.uint8))
    sink = torch.zeros((ql.QL_HBM_STREAM_SINK_WORDS,), dtype=torch.int64, device=big.device)
    one = time_single(torch, lambda i: ql.qlinear_hbm_read_stream(big, sink), 9)
    per = time_graph(torch, lambda i: ql.qlinear_hbm_read_stream(copies[i % len(copies)], sink),
                     4 * len(copies), reps)
    del big
    return {"kernel": "hbm_read_stream_kernel (qlinear_hbm_read_stream): 16-byte non-temporal loads",
            "one_launch_bytes": len(copies) * nbytes, "one_launch_us": round(one, 3),
            "one_launch_GBps": round(len(copies) * nbytes / (one * 1e-6) / 1e9, 1),
            "per_launch_us": round(per, 3),
            "per_launch_GBps": round(nbytes / (per * 1e-6) / 1e9, 1)}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_single(torch, launch, count: int = 24) -> float:
    """Median us of one eager launch timed alone: events around it, the device idle before it.

    ``launch(i)`` rotates its inputs, so a launch does not find them in the last-level cache.
    """
    launch(0)
    torch.cuda.synchronize()
    t = []
    for i in range(count):
        e0, e1 = _events(torch)
        e0.record()
        launch(i)
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    t.sort()
    return t[len(t) // 2]


def time_graph(torch, launch, count: int, reps: int = 10) -> float:
    """Mean us per launch: `count` launches captured in one HIP graph, replayed `reps` times."""
    launch(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            launch(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * count)


def time_eager(torch, launch, count: int) -> float:
    """Mean us per call of `count` back-to-back calls on the current stream."""
    launch(0)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for i in range(count):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def time_cpu(fn, min_s: float = 1.0) -> float:
    """Seconds per call of fn (repeated until min_s has passed)."""
    fn()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        t = time.perf_counter() - t0
        if t >= min_s:
            return t / n


def _row(us, work, unit, peak, bound, what, oracle_rate=None, oracle_sample=None):
    rate = work / (us * 1e-6) / (1e9 if unit == "GB/s" else 1e12)
    r = {"us_per_launch": round(us, 3), "achieved": round(rate, 1), "unit": unit, "bound": bound,
         "work_per_launch": what}
    if peak is not None:
        r["peak"] = peak
        r["frac"] = round(rate / peak, 4)
    if oracle_rate:
        r["oracle"] = {"value": round(oracle_rate, 4), "unit": unit, "sample": oracle_sample}
    return r


def _with_floor(row, ql, torch, bufs, count, what):
    """Add the HBM read-stream floor of a row: the same buffers read once each, same rotation."""
    sink = torch.zeros((ql.QL_HBM_STREAM_SINK_WORDS,), dtype=torch.int64, device=bufs[0].device)
    us = time_graph(torch, lambda i: ql.qlinear_hbm_read_stream(bufs[i % len(bufs)], sink), count)
    row["stream_floor"] = {"us_per_launch": round(us, 3), "what": what}
    row["frac_of_stream_floor"] = round(us / row["us_per_launch"], 4)


def bench_rows(ql, torch, synthetic, with_oracle: bool = True):
    """Every step of the path on its own workload, against the roofline that bounds it.

    HBM-bound rows rotate enough input copies (>= 384 MB) that no launch finds its
    input in the 256 MB last-level cache; launch-bound rows replay a HIP graph.
    Each row carries the CPU oracle's rate on a sample of the same work.
    """
    import numpy as np
    import oracle

    dev = "cuda:0"
    rows = {}
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # without the oracle legs every oracle rate below comes out 0 and is left out
    tc = time_cpu if with_oracle else (lambda fn, min_s=1.0: math.inf)

    # a4: per-token W8A8, 16x256x128, fp16 out (launch-bound; no roofline claim).
    d = synthetic.w8a8()
    x, w = d["x"].to(dev), d["w"].to(dev)
    deq, pts = d["deq"].to(dev), d["pts"].to(dev)
    out = torch.empty((16, 128), dtype=torch.float16, device=dev)
    us = time_graph(torch, lambda i: ql.qlinear_gemm_w8a8(x, w, ql.QL_W_KN, deq, pts, out=out), 100)
    xn, wn, dn, pn = (d[key].numpy() for key in ("x", "w", "deq", "pts"))
    t = tc(lambda: oracle.w8a8(xn, wn, False, pn, dn))
    rows["a4_w8a8_16x256x128"] = _row(us, 2.0 * 16 * 256 * 128, "TOPS", None, "launch",
                                      "2*m*n*k ops; HIP-graph replay of 100 launches",
                                      2.0 * 16 * 256 * 128 / t / 1e12, "the whole product")

    # a1 + a5: BitLinear forward, x bf16 [2048,4096] (1% outliers), w [4096,4096] -> bf16.
    m, n, k = 2048, 4096, 4096
    d = synthetic.bitlinear(m, n, k)
    xs = [d["x"].to(dev)] + [d["x"].to(dev) for _ in range(23)]            # 24 x 16.8 MB
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    pts = torch.empty((m,), dtype=torch.float32, device=dev)
    rs = torch.empty((m,), dtype=torch.int32, device=dev)
    us = time_graph(torch, lambda i: ql.qlinear_quant_act(xs[i % len(xs)], rmsnorm=True, q=q,
                                                          per_token_scale=pts, rowsum=rs), 48)
    qbytes = m * k * 2 + m * k + 8 * m
    xf = d["x"].float().numpy()
    sample = 256
    t = tc(lambda: oracle.quant_act(xf[:sample], rmsnorm=True))
    rows["a1_quant_act_2048x4096_bf16_rmsnorm"] = _row(
        us, qbytes, "GB/s", PEAK_HBM_GBS, "hbm", f"{qbytes} B (bf16 read, int8 codes, scale and rowsum)",
        sample * (k * 3 + 8) / t / 1e9, f"{sample} of {m} rows")
    _with_floor(rows["a1_quant_act_2048x4096_bf16_rmsnorm"], ql, torch, xs, 48,
                "plain read of the same bf16 inputs in the same rotation (the codes' writes not included)")
    del xs
    packed, gamma = ql.qlinear_pack_ternary(d["w"].to(dev), ql.QL_W_NK)
    xq, pts, rs = ql.qlinear_quant_act(d["x"].to(dev), rmsnorm=True)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    us = time_graph(torch, lambda i: ql.qlinear_gemm_w2a8(xq, pts, rs, packed, gamma, n, out=out), 20)
    ops = 2.0 * m * n * k
    codes, g = oracle.ternary_quant(d["w"].numpy())
    xqn, ptsn, _ = oracle.quant_act(xf[:32], rmsnorm=True)
    t = tc(lambda: oracle.w2a8(xqn, ptsn, codes, g))
    rows["a5_w2a8_gemm_2048x4096x4096"] = _row(us, ops, "TOPS", PEAK_INT8_TOPS, "mfma", "2*m*n*k int8 ops",
                                               2.0 * 32 * n * k / t / 1e12, f"32 of {m} rows")

    # a2: absmean ternary pack of the decode weight fp32 [28672,8192] (one-time).
    n, k = 28672, 8192
    wd = synthetic.master_weight(n, k, 1003 + 100_000)
    wdev = wd.to(dev)
    pk = torch.empty((n * k // 16,), dtype=torch.int32, device=dev)
    gm = torch.empty((1,), dtype=torch.float64, device=dev)
    ws = torch.empty((ql.qlinear_workspace_bytes(ql.QL_OP_PACK_TERNARY, 0, n, k),), dtype=torch.uint8,
                     device=dev)
    us = time_eager(torch, lambda i: ql.qlinear_pack_ternary(wdev, ql.QL_W_NK, packed=pk, gamma=gm,
                                                             workspace=ws), 5)
    pbytes = 2 * n * k * 4 + n * k // 4
    wn = wd.numpy()
    sample = 2048
    t = tc(lambda: oracle.pack_ternary(oracle.ternary_quant(wn[:sample])[0]))
    rows["a2_pack_ternary_28672x8192_fp32"] = _row(
        us, pbytes, "GB/s", PEAK_HBM_GBS, "hbm",
        f"{pbytes} B (fp32 weight read twice: absmean, then threshold; 2-bit words written)",
        sample * k * (8 + 0.25) / t / 1e9, f"{sample} of {n} rows (their own absmean)")
    del wdev, pk, ws

    # a3 + a7: grouped affine INT4, x fp16 [32,4096], uint4 w [11008,4096], g=128 -> fp16.
    dg = synthetic.grouped_int4()
    m, n, k, gs = 32, 11008, 4096, dg["group_size"]
    qdev = dg["q"].to(dev)
    pw = torch.empty((n * k // 8,), dtype=torch.int32, device=dev)
    us = time_eager(torch, lambda i: ql.qlinear_pack_int4(qdev, ql.QL_INT4_WEIGHT, packed=pw), 20)
    i4bytes = n * k + n * k // 2
    qn = dg["q"].numpy()
    t = tc(lambda: oracle.pack_int4(qn[:1024]))
    rows["a3_pack_int4_11008x4096"] = _row(us, i4bytes, "GB/s", PEAK_HBM_GBS, "hbm",
                                           f"{i4bytes} B (one code byte read, half a byte written per weight)",
                                           1024 * k * 1.5 / t / 1e9, f"1024 of {n} rows")
    pws = [pw] + [pw.clone() for _ in range(15)]                           # 16 x 22.5 MB
    xg = dg["x"].to(dev)
    sc = dg["s"].to(dev)
    pz = ql.qlinear_pack_int4(dg["z"].to(dev), ql.QL_INT4_ZEROS)
    outg = torch.empty((m, n), dtype=torch.float16, device=dev)
    us = time_graph(torch, lambda i: ql.qlinear_gemm_w4a8_grouped(xg, pws[i % len(pws)], sc, pz, gs, n,
                                                                  out=outg), 48)
    gbytes = n * k // 2 + n * (k // gs) * 2 + n * (k // gs) // 2 + m * k * 2 + m * n * 2
    xgn, sn = dg["x"].float().numpy(), dg["s"].float().numpy()
    zn = dg["z"].numpy()
    t = tc(lambda: oracle.grouped_int4(xgn, qn[:512], sn[:512], zn[:512], gs))
    rows["a7_grouped_int4_32x4096x11008_g128"] = _row(
        us, gbytes, "GB/s", PEAK_HBM_GBS, "hbm",
        f"{gbytes} B (packed weight, fp16 scales, packed zeros, fp16 x, fp16 out)",
        (512 * k // 2 + 512 * (k // gs) * 2.5 + m * k * 2 + m * 512 * 2) / t / 1e9, f"512 of {n} columns")
    rows["a7_grouped_int4_32x4096x11008_g128"]["single_launch_us"] = round(time_single(
        torch, lambda i: ql.qlinear_gemm_w4a8_grouped(xg, pws[i % len(pws)], sc, pz, gs, n, out=outg)), 3)
    _with_floor(rows["a7_grouped_int4_32x4096x11008_g128"], ql, torch, pws, 48,
                "plain read of the same packed weight copies in the same rotation (scales, zero-points, x "
                "and out not included)")
    xqg, ptsg, _ = ql.qlinear_quant_act(xg)
    us = time_graph(torch, lambda i: ql.qlinear_gemm_w4a8_grouped(xqg, pws[i % len(pws)], sc, pz, gs, n, out=outg,
                                                                  per_token_scale=ptsg), 48)
    gbytes8 = n * k // 2 + n * (k // gs) * 2 + n * (k // gs) // 2 + m * k + 4 * m + m * n * 2
    xqn, ptsn, _ = oracle.quant_act(xgn)
    t = tc(lambda: oracle.grouped_int4_i8(xqn, ptsn, qn[:512], sn[:512], zn[:512], gs))
    rows["a7i8_grouped_int4_int8_act_32x4096x11008_g128"] = _row(
        us, gbytes8, "GB/s", PEAK_HBM_GBS, "hbm",
        f"{gbytes8} B (packed weight, fp16 scales, packed zeros, int8 x codes and scales, fp16 out)",
        (512 * k // 2 + 512 * (k // gs) * 2.5 + m * k + m * 512 * 2) / t / 1e9, f"512 of {n} columns")
    del pws, xg, outg

    # next-4: Q4Linear backward, 8192^3 fp16 (grad_x, grad_w, grad_scale_a);
    # two fp16 matrix-core products of 2*m*n*k flops each plus the operand
    # transposes and the range-masked epilogues
    m = n = k = 8192
    r = np.random.Generator(np.random.PCG64(1007))
    xb = torch.from_numpy(r.normal(0, 1, (m, k)).astype(np.float16)).to(dev)
    wb = torch.from_numpy((0.02 * r.normal(0, 1, (n, k))).astype(np.float16)).to(dev)
    gb = torch.from_numpy(r.normal(0, 1, (m, n)).astype(np.float16)).to(dev)
    sab = (xb.abs().max().float() / 7).reshape(1)
    swb = (wb.abs().max().float() / 7).reshape(1)
    gxb = torch.empty((m, k), dtype=torch.float32, device=dev)
    gwb = torch.empty((n, k), dtype=torch.float32, device=dev)
    gsb = torch.empty((1,), dtype=torch.float32, device=dev)
    wsb = torch.empty((ql.qlinear_workspace_bytes(ql.QL_OP_Q4_BACKWARD, m, n, k),), dtype=torch.uint8, device=dev)
    us = time_eager(torch, lambda i: ql.qlinear_q4_backward(gb, xb, wb, sab, swb, 1e-5, grad_x=gxb, grad_w=gwb,
                                                            grad_scale_a=gsb, workspace=wsb), 5)
    flops = 2 * 2.0 * m * n * k
    gn, xn, wn = gb[:8].float().cpu().numpy(), xb[:8].float().cpu().numpy(), wb.float().cpu().numpy()
    t = tc(lambda: oracle.q4_backward(gn, xn, wn, float(sab.item()), float(swb.item()), 1e-5), min_s=0.5)
    rows["next4_q4_backward_8192x8192x8192_fp16"] = _row(
        us, flops, "TFLOP/s", PEAK_FP16_TFLOPS, "mfma",
        "2 x 2*m*n*k fp16 flops (grad_x = G Wh, grad_w = G^T Xh) with transposes and masked epilogues; "
        "one qlinear_q4_backward call, eager, mean of 5",
        2 * 2.0 * 8 * n * k / t / 1e12, "8 of 8192 token rows (their grad_x and their share of grad_w)")
    del xb, wb, gb, gxb, gwb, wsb
    return {"threads_oracle": threads, "rows": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["a4w4", "decode", "rows"], default=None,
                    help="run one part alone (for counter runs): the A4W4 step, the decode GEMV, or the path rows")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_linear_quant_amd as ql
    import synthetic

    ql.lib()
    if args.only is not None:
        if args.only == "a4w4":
            part = bench_a4w4(args, ql, torch, synthetic)[0]
        elif args.only == "decode":
            part = bench_decode(ql, torch, synthetic)
        else:
            part = bench_rows(ql, torch, synthetic, with_oracle=False)
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "result": part}), flush=True)
        return
    res, d = bench_a4w4(args, ql, torch, synthetic)
    gemv = bench_decode(ql, torch, synthetic)
    gemv_src = kernel_source_hash(GEMV_KERNEL_SOURCES)
    for m_str, key in (("1", "w2a8_gemv_m1_28672x8192"), ("4", "w2a8_gemv_m4_28672x8192"),
                       ("16", "w2a8_gemv_m16_28672x8192")):
        gemv["by_m"][m_str]["traffic"] = recorded_traffic(key, gemv_src)
    gemm_src = kernel_source_hash(GEMM_KERNEL_SOURCES)
    traffic = recorded_traffic("gemm_a4w4_f6_8192", gemm_src)
    achieved = res["gemm_tops"]
    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6",
        "data": "synthetic",
        "config": {"workload": "A4W4 Q4Linear forward: fp16 x[8192,8192] N(0,1), fp16 w[8192,8192] "
                               "N(0,0.02^2), per-tensor scales max|t|/7, eps 1e-5, 4-bit codes packed as "
                               "FP6 E3M2 operands, FP6 MFMA product with exact fp32 accumulation, fp16 out",
                   "m": res["m"], "n": res["n"], "k": res["k"], "global_batch": res["m"],
                   "parallelism": "single GPU"},
        "kernel_ms": {key: round(v, 4) for key, v in res["kernel_ms"].items()},
        "int8_codes_gemm": res["int8_codes_gemm"],
        "packed_operands_gemm": res["packed_operands_gemm"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP6_TOPS, "unit": "TOPS",
                     "frac": round(achieved / PEAK_FP6_TOPS, 4), "traffic": traffic,
                     "kernel": "gemm_a4w4_f6_kernel (qlinear_gemm_a4w4_operands)",
                     "work_per_launch": f"2*m*n*k = {int(res['ops'])} ops on 4-bit codes"},
        "decode_gemv": gemv,
    }
    line["path_rows"] = bench_rows(ql, torch, synthetic)
    torch.cuda.synchronize()
    line["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
