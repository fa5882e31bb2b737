#!/usr/bin/env python3
"""Benchmark of the normalization hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the whole hot path over resident synthetic inputs:
  1. rmsnorm_fwd on x[16384, 16384] bf16 (N(0,1), w ~ U(0.5, 1.5), eps 1e-6),
     the shape the RMSNorm bandwidth table of "[Inductor] Codegen Gluon"
     (section 3.1) peaks at;
  2. qk_norm_rope_fwd on qkv[256, (32+8+8)*128] bf16 (full-rotary fused
     QK-norm + RoPE, "[pretuned] Optimize fused_qk_norm_rope on B200").
Each launch records its own start and end in HIP events (hipExtLaunchKernel,
on the stream it runs on); `value` is the RMSNorm's achieved HBM bandwidth,
algorithmic bytes (2*M*N*2 + 2*N) divided by the mean of its durations, in
GB/s (1e9 B/s). Prints one JSON line.

The CPU baseline is the fp64 oracle run on the host over row blocks of the
same RMSNorm workload (512 rows each), on up to 16 threads and on one.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from probe import HipTimingEvents, kernel_source_hash  # noqa: E402

HBM_PEAK_GBPS = 8000.0
RMS_WORKLOAD = "rms_16384x16384"
QK_WORKLOAD = "qk_256"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "rmsnorm_16384x16384_hbm_traffic.txt")
def measured_traffic(algorithmic_bytes: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none, it covers another workload, or the kernel source changed
    since it was taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    src = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    tot = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    algo = re.search(r"algorithmic_bytes_per_launch:\s*(\d+)", text)
    if not src or not tot or not algo or src.group(1) != kernel_source_hash():
        return None
    if int(algo.group(1)) != algorithmic_bytes:
        return None
    return float(tot.group(1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def streaming_copy_reference(x, y, stream, steps: int, warmup: int):
    """The best 50/50 read/write stream measured on this part -- the
    hand-written copy of libmbn_stream.so with 4 KiB per workgroup (16-byte
    non-temporal loads and stores, the row-norm kernels' accesses) -- timed
    the same way as the RMSNorm (the kernel's own start and end, recorded in
    events by hipExtLaunchKernel) on the same 512 MiB buffers: the reference
    roofline.frac is read against. probe.py compiles libmbn_stream.so when it
    is missing; None when that fails."""
    try:
        from probe import stream_lib

        sl = stream_lib()
    except (RuntimeError, OSError):
        return None
    nbytes = x.numel() * x.element_size()
    sp = stream.cuda_stream

    timer = HipTimingEvents(stream)

    def launch(a, b):
        rc = sl.mbn_stream_copy_timed(x.data_ptr(), y.data_ptr(), nbytes, 256, 1, sp, a, b)
        if rc != 0:
            raise RuntimeError(f"mbn_stream_copy_timed status {rc}")

    spare = (timer.new(), timer.new())
    for _ in range(warmup):
        launch(*spare)
    ev = [(timer.new(), timer.new()) for _ in range(steps)]
    for a, b in ev:
        launch(a, b)
    import torch

    torch.cuda.synchronize()
    us = [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
    timer.close()
    mean = sum(us) / len(us)
    return {"kernel": "stream_copy<256, 1> (4 KiB per workgroup, libmbn_stream.so)",
            "bytes_per_launch": 2 * nbytes, "mean_us": round(mean, 2),
            "GBps": round(2 * nbytes / mean / 1e3, 1),
            "frac": round(2 * nbytes / mean / 1e3 / HBM_PEAK_GBPS, 4)}


def host_threads() -> int:
    """Host threads for the CPU baseline: the CPUs this process may run on,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(x_bits, w_bits, eps, n: int, budget_s: float):
    """Time the oracle over row blocks of the workload: on `host_threads()`
    threads (NumPy releases the GIL inside its array operations) until
    `budget_s` is used, and on one thread over a quarter of that budget."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import rmsnorm_fwd as oracle_rmsnorm

    block = 512
    m = x_bits.shape[0]

    def run(rows):
        oracle_rmsnorm(x_bits[rows : rows + block], w_bits, eps)
        return min(block, m - rows)

    threads = host_threads()
    rows_done = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as pool:
        while rows_done < m and time.perf_counter() - t0 < budget_s:
            starts = list(range(rows_done, min(m, rows_done + threads * block), block))
            rows_done += sum(pool.map(run, starts))
    dt = time.perf_counter() - t0

    rows_one = 0
    t1 = time.perf_counter()
    while rows_one < m and time.perf_counter() - t1 < budget_s / 4:
        rows_one += run(rows_one)
    dt1 = time.perf_counter() - t1

    def rate(rows, sec):
        return round((2 * rows * n * 2 + 2 * n) / sec / 1e9, 4)

    return {
        "value": rate(rows_done, dt),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows_done} of {m} rows of x[16384, 16384] in {block}-row blocks, numpy fp64, "
        f"{threads} threads, {dt:.1f} s on {cpu_model()} ({os.cpu_count()} logical CPUs)",
        "single_thread": {"value": rate(rows_one, dt1), "rows": rows_one, "seconds": round(dt1, 2)},
    }


def suite(steps: int, warmup: int) -> int:
    """Per-workload timing table (one JSON line per workload): all five inputs,
    the pages' 3 x 3 RMSNorm shape grid, fp16 storage, widths that are not
    whole 16-byte chunks, a view at an element offset, small launches, widths
    between powers of two, and the rest of the norm family.

    Workloads whose footprint is under 1 GiB rotate over enough copies of their
    buffers that successive launches cannot be served from the 256 MiB Infinity
    Cache; the median and best of per-launch event times are reported.
    """
    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from workloads import QK_WORKLOADS, RMS_WORKLOADS, make_qk_inputs, make_rms_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    # The part runs slower for its first few hundred milliseconds of sustained
    # load: ~0.5 s of the 16384 x 16384 launch before the first timed workload.
    xw = torch.randn(16384, 16384, device=dev).to(torch.bfloat16)
    ww = torch.ones(16384, dtype=torch.bfloat16, device=dev)
    for _ in range(3000):
        mbn.rmsnorm_fwd(xw, ww, xw, eps=1e-6)
    torch.cuda.synchronize()
    del xw, ww

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def timed(fn, nrot):
        """(median, best) of per-launch event pairs, and the mean of a back-to-back batch."""
        timer = HipTimingEvents(stream)
        for i in range(warmup):
            fn(i % nrot)
        torch.cuda.synchronize()
        ev = [(timer.new(), timer.new()) for _ in range(steps)]
        for i in range(steps):
            timer.record(ev[i][0])
            fn(i % nrot)
            timer.record(ev[i][1])
        torch.cuda.synchronize()
        us = sorted(timer.elapsed_ms(a, b) * 1e3 for a, b in ev)
        b0, b1 = timer.new(), timer.new()
        timer.record(b0)
        for i in range(steps):
            fn(i % nrot)
        timer.record(b1)
        torch.cuda.synchronize()
        timed.batch_us = timer.elapsed_ms(b0, b1) * 1e3 / steps
        timer.close()
        return us[len(us) // 2], us[0]

    def report(workload, kernel, nrot, med, best, b, **shape):
        """One JSON line: the median and best per-launch times and the batch
        mean against b algorithmic bytes per launch."""
        print(json.dumps({"workload": workload, "kernel": kernel, **shape, "algorithmic_bytes": b,
                          "rotating_sets": nrot, "median_us": round(med, 2), "best_us": round(best, 2),
                          "GBps_median": round(b / med / 1e3, 1),
                          "pct_of_8TBps_median": round(b / med / 1e3 / 80.0, 2),
                          "batch_mean_us": round(timed.batch_us, 2),
                          "pct_of_8TBps_batch": round(b / timed.batch_us / 1e3 / 80.0, 2)}), flush=True)

    # The plain 4 KiB-per-workgroup streaming copy (libmbn_stream.so) of the
    # same bytes between the same rotating buffers follows each RMSNorm
    # workload ("<workload>_copy"): what a 50/50 stream of that size reaches
    # on this part, launch ramp and drain included.
    try:
        from probe import stream_lib

        sl = stream_lib()
    except (RuntimeError, OSError):
        sl = None
    sp = stream.cuda_stream

    def copy(src, dst):
        rc = sl.mbn_stream_copy(src.data_ptr(), dst.data_ptr(), src.numel() * 2, 256, 1, sp)
        if rc != 0:
            raise RuntimeError(f"mbn_stream_copy status {rc}")

    for name, wl in RMS_WORKLOADS.items():
        x_bits, w_bits, eps = make_rms_inputs(wl)
        x0, w = to_dev(x_bits), to_dev(w_bits)
        pair = 2 * x0.numel() * 2
        nrot = max(1, -(-(1 << 30) // pair))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
        b = wl.algorithmic_bytes
        report(name, "rmsnorm_fwd", nrot, med, best, b, M=wl.M, N=wl.N)
        if sl is not None:
            med, best = timed(lambda i: copy(xs[i], ys[i]), nrot)
            report(name + "_copy", "stream_copy", nrot, med, best, pair, M=wl.M, N=wl.N)
        del xs, ys, x0
        torch.cuda.empty_cache()
    # The RMSNorm benchmark grid of "[Inductor] Codegen Gluon", section 3.1
    # (M, N in {4096, 8192, 16384}): the leading M x N block of the 16384 x
    # 16384 workload's x and the first N weights. The smaller shapes run on the
    # persistent kernel where its launch tables select it.
    wl = RMS_WORKLOADS["rms_16384x16384"]
    x_bits, w_bits, eps = make_rms_inputs(wl)
    x_full, w_full = to_dev(x_bits), to_dev(w_bits)
    del x_bits, w_bits
    for M in (4096, 8192, 16384):
        for N in (4096, 8192, 16384):
            x0 = x_full[:M, :N].contiguous()
            w = w_full[:N].contiguous()
            nrot = max(1, -(-(1 << 30) // (2 * M * N * 2)))
            xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
            ys = [torch.empty_like(x0) for _ in range(nrot)]
            med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
            b = 2 * M * N * 2 + 2 * N
            report(f"grid_{M}x{N}", "rmsnorm_fwd", nrot, med, best, b, M=M, N=N)
            del xs, ys, x0
    # fp16 storage: the same kernels with the F16 traits, same input in fp16.
    for name in ("rms_16384x16384", "rms_8192x8192"):
        wl16 = RMS_WORKLOADS[name]
        M, N = wl16.M, wl16.N
        x0 = x_full[:M, :N].to(torch.float16).contiguous()
        w = w_full[:N].to(torch.float16).contiguous()
        nrot = max(1, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
        b = 2 * M * N * 2 + 2 * N
        report(f"{name}_f16", "rmsnorm_fwd_f16", nrot, med, best, b, M=M, N=N)
        del xs, ys, x0

    # Widths that are not whole 16-byte chunks (the any-width kernels: 4-, 2-
    # and 1-element accesses), from the same input.
    for N in (16380, 16382, 16383):
        M = 16384
        x0 = x_full[:, :N].contiguous()
        w = w_full[:N].contiguous()
        nrot = max(1, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
        b = 2 * M * N * 2 + 2 * N
        report(f"any_{M}x{N}", "rmsnorm_fwd", nrot, med, best, b, M=M, N=N)
        del xs, ys, x0
    # A view at an element offset of 1 (rows start 2 bytes into a 16-byte
    # block): the 16-byte staged any-width kernel.
    M = N = 16384
    nrot = 2
    bufs = [torch.empty(M * N + 8, dtype=torch.bfloat16, device=dev) for _ in range(2 * nrot)]
    for i in range(nrot):
        bufs[i][1:1 + M * N].copy_(x_full.view(-1))
    xs = [bufs[i][1:1 + M * N].view(M, N) for i in range(nrot)]
    ys = [bufs[nrot + i][1:1 + M * N].view(M, N) for i in range(nrot)]
    med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w_full, ys[i], eps=eps), nrot)
    b = 2 * M * N * 2 + 2 * N
    report(f"view_{M}x{N}_o1", "rmsnorm_fwd", nrot, med, best, b, M=M, N=N)
    del xs, ys, bufs
    # Small launches (row windows of the launch tables), leading blocks of the
    # same input.
    for M, N in ((256, 16384), (1024, 8192), (1024, 16384), (2048, 2048)):
        x0 = x_full[:M, :N].contiguous()
        w = w_full[:N].contiguous()
        nrot = max(1, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
        b = 2 * M * N * 2 + 2 * N
        report(f"small_{M}x{N}", "rmsnorm_fwd", nrot, med, best, b, M=M, N=N)
        del xs, ys, x0
    # Widths between powers of two (the RMSNorm sub-band entries of the
    # launch tables), M * N = 2^27: the same input tiled to M x N (its
    # leading rows and columns repeated past 16384).
    for N in (5120, 12288, 14336, 18432):
        M = (1 << 27) // N
        cols = x_full if N <= 16384 else torch.cat([x_full, x_full[:, :N - 16384]], dim=1)
        x0 = torch.cat([cols[:, :N]] * -(-M // 16384))[:M].contiguous()
        del cols
        assert x0.shape == (M, N)
        w = torch.cat([w_full, w_full])[:N].contiguous()
        nrot = max(1, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        med, best = timed(lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), nrot)
        report(f"width_{M}x{N}", "rmsnorm_fwd", nrot, med, best, 2 * M * N * 2 + 2 * N, M=M, N=N)
        del xs, ys, x0
    # The other norms at widths with entries of their own between powers of
    # two (r: the rows of x in reverse order; bias: the weights reversed).
    for kname, N in (("add_rmsnorm_fwd", 5120), ("layernorm_fwd", 12288), ("l2norm_fwd", 12288)):
        M = (1 << 27) // N
        x0 = torch.cat([x_full[:, :N]] * -(-M // 16384))[:M].contiguous()
        w = w_full[:N].contiguous()
        bias = w_full[:N].flip(0).contiguous()
        streams = 4 if kname == "add_rmsnorm_fwd" else 2
        nrot = max(1, -(-(1 << 30) // (streams * M * N * 2)))
        xs = [x0] + [x0.clone() for _ in range(nrot - 1)]
        rs = [x.flip(0).contiguous() for x in xs] if kname == "add_rmsnorm_fwd" else None
        hs = [torch.empty_like(x0) for _ in range(nrot)] if kname == "add_rmsnorm_fwd" else None
        ys = [torch.empty_like(x0) for _ in range(nrot)]
        fn = {"add_rmsnorm_fwd": lambda i: mbn.add_rmsnorm_fwd(xs[i], rs[i], w, h=hs[i], y=ys[i], eps=eps),
              "layernorm_fwd": lambda i: mbn.layernorm_fwd(xs[i], w, bias, y=ys[i], eps=1e-5),
              "l2norm_fwd": lambda i: mbn.l2norm_fwd(xs[i], y=ys[i], eps=1e-12)}[kname]
        b = streams * M * N * 2 + {"add_rmsnorm_fwd": 2, "layernorm_fwd": 4, "l2norm_fwd": 0}[kname] * N
        med, best = timed(fn, nrot)
        report(f"width_{M}x{N}", kname, nrot, med, best, b, M=M, N=N)
        del xs, rs, hs, ys, x0
    del x_full, w_full
    torch.cuda.empty_cache()

    from workloads import make_norm_family_inputs

    for name in ("rms_8192x8192", "rms_16384x16384"):
        wl = RMS_WORKLOADS[name]
        x_bits, w_bits, r_bits, b_bits, eps = make_norm_family_inputs(wl)
        x, w, r, bb = to_dev(x_bits), to_dev(w_bits), to_dev(r_bits), to_dev(b_bits)
        mn, n = wl.M * wl.N, wl.N
        nrot = max(1, -(-(1 << 30) // (2 * mn * 2)))
        xs = [x] + [x.clone() for _ in range(nrot - 1)]
        rs = [r] + [r.clone() for _ in range(nrot - 1)]
        hs = [torch.empty_like(x) for _ in range(nrot)]
        ys = [torch.empty_like(x) for _ in range(nrot)]
        cases = [
            ("add_rmsnorm_fwd", 8 * mn + 2 * n,
             lambda i: mbn.add_rmsnorm_fwd(xs[i], rs[i], w, h=hs[i], y=ys[i], eps=eps)),
            ("layernorm_fwd", 4 * mn + 4 * n, lambda i: mbn.layernorm_fwd(xs[i], w, bb, y=ys[i], eps=eps)),
            ("l2norm_fwd", 4 * mn, lambda i: mbn.l2norm_fwd(xs[i], y=ys[i], eps=1e-12)),
        ]
        for kname, b, fn in cases:
            med, best = timed(fn, nrot)
            report(name.replace("rms_", "family_"), kname, nrot, med, best, b, M=wl.M, N=wl.N)
        del xs, rs, hs, ys, x, r
        torch.cuda.empty_cache()
    for name, wl in QK_WORKLOADS.items():
        qkv_bits, qw_bits, kw_bits, pos, eps, theta = make_qk_inputs(wl)
        q0 = to_dev(qkv_bits)
        nrot = max(1, -(-(1 << 30) // (q0.numel() * 2)))
        qs = [q0] + [q0.clone() for _ in range(nrot - 1)]
        q_w, k_w = to_dev(qw_bits), to_dev(kw_bits)
        p = torch.from_numpy(pos).to(dev)
        med, best = timed(lambda i: mbn.qk_norm_rope_fwd(qs[i], q_w, k_w, p, wl.n_q_heads, wl.n_kv_heads,
                                                         wl.head_dim, eps=eps, theta=theta), nrot)
        b = wl.algorithmic_bytes
        report(name, "qk_norm_rope_fwd", nrot, med, best, b, T=wl.T)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The part runs ~1.7% slower for the first few hundred milliseconds of
    # sustained load (measured: 171.4 us per launch fresh, 168.5 us after 2000
    # launches, 171 us again after 3 s idle); 2000 warm-up steps (~0.4 s) start
    # the timed steps in the steady state.
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true",
                    help="time every workload (one JSON line each) instead of the benchmark step")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(
            "bench.py measures one GPU only: the kernels run on one MI355X's share of the "
            "rows; multi-GPU runs are not supported.",
            file=sys.stderr,
        )
        return 2

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from workloads import QK_WORKLOADS, RMS_WORKLOADS, make_qk_inputs, make_rms_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    mbn.lib()  # fail loudly if the HIP library is missing
    if args.suite:
        return suite(args.steps, args.warmup)

    dev = torch.device("cuda:0")
    wl = RMS_WORKLOADS[RMS_WORKLOAD]
    qwl = QK_WORKLOADS[QK_WORKLOAD]
    x_bits, w_bits, eps = make_rms_inputs(wl)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = to_dev(x_bits)
    w = to_dev(w_bits)
    y = torch.empty_like(x)
    qkv_bits, qw_bits, kw_bits, pos, qeps, theta = make_qk_inputs(qwl)
    qkv0 = to_dev(qkv_bits)
    qkv = qkv0.clone()
    q_w, k_w = to_dev(qw_bits), to_dev(kw_bits)
    positions = torch.from_numpy(pos).to(dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)

    timer = HipTimingEvents(stream)

    # One step: the RMSNorm, then the QK-norm + RoPE, each through its timed
    # entry point, which records the kernel's own start and end in the step's
    # events (ev[0], ev[1]: RMSNorm; ev[2], ev[3]: QK). Warm-up steps take the
    # same path with a spare set of events.
    def step(ev):
        mbn.rmsnorm_fwd_timed(x, w, ev[0], ev[1], y=y, eps=eps)
        mbn.qk_norm_rope_fwd_timed(qkv, q_w, k_w, positions, qwl.n_q_heads, qwl.n_kv_heads,
                                   ev[2], ev[3], head_dim=qwl.head_dim, eps=qeps, theta=theta)

    spare = [timer.new() for _ in range(4)]
    for _ in range(args.warmup):
        step(spare)
    torch.cuda.synchronize()

    evs = [[timer.new() for _ in range(4)] for _ in range(args.steps)]
    region = (timer.new(), timer.new())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    timer.record(region[0])
    for i in range(args.steps):
        step(evs[i])
    timer.record(region[1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    rms_ms = [timer.elapsed_ms(e[0], e[1]) for e in evs]
    qk_ms = [timer.elapsed_ms(e[2], e[3]) for e in evs]
    region_us = timer.elapsed_ms(*region) * 1e3 / args.steps
    timer.close()
    rms_mean_s = sum(rms_ms) / len(rms_ms) / 1e3
    qk_mean_s = sum(qk_ms) / len(qk_ms) / 1e3
    rms_bytes = wl.algorithmic_bytes
    achieved = rms_bytes / rms_mean_s / 1e9

    traffic = measured_traffic(rms_bytes)
    out = {
        "metric": "achieved HBM GB/s and % of 8 TB/s peak, bf16 RMSNorm M=N=16384",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy, see workloads/)",
        "config": {
            "workload": "bf16 RMSNorm x[16384,16384] + fused QK-norm+RoPE qkv[256,48*128]",
            "io_dtype": "bf16",
            "rmsnorm": {"M": wl.M, "N": wl.N, "eps": wl.eps},
            "qk_norm_rope": {"T": qwl.T, "n_q_heads": qwl.n_q_heads, "n_kv_heads": qwl.n_kv_heads,
                             "head_dim": qwl.head_dim, "theta": qwl.theta, "eps": qwl.eps},
        },
        "pct_of_peak": round(100.0 * achieved / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_calibration": "FETCH_SIZE and WRITE_SIZE per launch, each scaled by the same counter's "
                                   "reading for a plain 512 MiB device copy (copy-relative, not absolute); "
                                   "profiles/rmsnorm_16384x16384_hbm_traffic.txt",
            "kernel": "rmsnorm_fwd",
            "algorithmic_bytes_per_launch": rms_bytes,
            "mean_us": round(rms_mean_s * 1e6, 2),
            "best_us": round(min(rms_ms) * 1e3, 2),
            "timing": "kernel start to end, recorded in HIP events by hipExtLaunchKernel "
                      "(rmsnorm_fwd_timed) on the launch stream; mean over the timed steps",
            "timed_region_us_per_step": round(region_us, 2),
        },
        "qk_norm_rope": {
            "mean_us": round(qk_mean_s * 1e6, 2),
            "best_us": round(min(qk_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": qwl.algorithmic_bytes,
            "GBps": round(qwl.algorithmic_bytes / qk_mean_s / 1e9, 1),
            "note": "2.5 MiB in place; stays in L2/MALL across steps; launch-latency bound",
        },
    }
    # Context for roofline.frac, measured after the timed steps (it overwrites y).
    copy_ref = streaming_copy_reference(x, y, stream, args.steps, min(args.warmup, 500))
    if copy_ref is not None:
        copy_ref["rmsnorm_over_copy"] = round(achieved / copy_ref["GBps"], 4)
        out["roofline"]["streaming_copy_reference"] = copy_ref
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x_bits, w_bits, eps, wl.N, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
