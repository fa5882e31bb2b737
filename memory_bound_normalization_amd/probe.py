"""Short GPU program for hardware-counter runs, and the summarizer of their output.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe run
    rocprofv3 --pmc WRITE_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe run
    python -m memory_bound_normalization_amd.probe summarize <fetch_dir> <write_dir> [workload]

`run [workload]` launches rmsnorm_fwd on x[16384, 16384] (the benchmark
workload; or another RMSNorm workload of `workloads`, e.g. rms_4096x32768) a
few times, then a plain device-to-device copy of the same x (torch's copy
kernel) as the calibration: the counters of the copy, whose true HBM traffic is
known (x's bytes read and written), give the factor that converts each counter
reading into bytes. `summarize` prints the per-launch HBM traffic of the
RMSNorm kernel from the two runs' counter CSV files.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe qk-run
    rocprofv3 --pmc WRITE_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe qk-run
    python -m memory_bound_normalization_amd.probe qk-summarize <fetch_dir> <write_dir>

`qk-run` does the same for qk_norm_rope_fwd on 65536 tokens of 32 q + 8 k + 8 v
heads of 128 (768 MiB, more than the Infinity Cache), calibrated by torch's
device copy of a separate 512 MiB buffer (the RMSNorm runs' calibration
kernel and size);
`qk-summarize` prints its per-launch traffic beside the
algorithmic bytes (q and k heads read and written, v heads untouched).

    rocprofv3 --kernel-trace --stats -d <dir> -o run -- python -m memory_bound_normalization_amd.probe ceiling
    python -m memory_bound_normalization_amd.probe ceiling-summary <dir>

    rocprofv3 --kernel-trace -d <dir> -o run -- python -m memory_bound_normalization_amd.probe small
    python -m memory_bound_normalization_amd.probe small-summary <dir>

`small` launches the two small workloads (RMSNorm on x[1024, 4096], QK-norm +
RoPE on 256 tokens) beside plain copies of the same bytes and a one-workgroup
write; `small-summary` gives their GPU durations, the floor such launches sit
on.

`ceiling` times plain streaming kernels on the same 512 MiB buffers beside
rmsnorm_fwd: torch's (read only: a sum; write only: a fill; read + write: a
copy and a scale) and the hand-written ones of libmbn_stream.so (read only,
write only and copy with the row-norm kernels' 16-byte non-temporal accesses,
at per-workgroup footprints of 4 to 64 KiB), each over two alternating buffer
sets (1 GiB apart, so nothing is served from the 256 MiB Infinity Cache);
`ceiling-summary` turns the kernel trace into GB/s per kernel. It measures what
the memory system gives a pure-read, a pure-write and a 50/50 read/write stream
on this part, the reference for the RMSNorm kernel's fraction of peak.
"""

from __future__ import annotations

import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LAUNCHES = 5
COPY_BYTES = 16384 * 16384 * 2


DEFAULT_WORKLOAD = "rms_16384x16384"


def run(workload: str = DEFAULT_WORKLOAD) -> None:
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from workloads import RMS_WORKLOADS, make_rms_inputs

    wl = RMS_WORKLOADS[workload]
    x_bits, w_bits, eps = make_rms_inputs(wl)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        mbn.rmsnorm_fwd(x, w, y, eps=eps)
        torch.cuda.synchronize()
        print(f"rmsnorm launch {i} done", flush=True)
    z = torch.empty_like(x)
    for i in range(LAUNCHES):
        z.copy_(x)
        torch.cuda.synchronize()
        print(f"copy launch {i} done", flush=True)


QK_TOKENS, QK_HQ, QK_HKV, QK_D = 65536, 32, 8, 128


def qk_algorithmic_bytes(T: int = QK_TOKENS) -> int:
    """q and k heads read and written, the two weights and the positions."""
    return 2 * T * (QK_HQ + QK_HKV) * QK_D * 2 + 2 * QK_D * 2 + 8 * T


def qk_run() -> None:
    sys.path.insert(0, ROOT)
    import torch

    import memory_bound_normalization_amd as mbn

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    width = (QK_HQ + 2 * QK_HKV) * QK_D
    # the calibration copy's source (512 MiB), created before qkv
    n = COPY_BYTES // 2
    src = torch.randn(n, device=dev, generator=g).to(torch.bfloat16)
    qkv = torch.randn(QK_TOKENS, width, device=dev, generator=g).to(torch.bfloat16)
    q_w = (torch.rand(QK_D, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    k_w = (torch.rand(QK_D, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    pos = torch.arange(QK_TOKENS, device=dev, dtype=torch.int64)
    torch.cuda.synchronize()
    for i in range(LAUNCHES):
        mbn.qk_norm_rope_fwd(qkv, q_w, k_w, pos, QK_HQ, QK_HKV, QK_D, eps=1e-6, theta=1e6)
        torch.cuda.synchronize()
        print(f"qk_norm_rope launch {i} done", flush=True)
    # calibration: torch's device copy of 512 MiB, the kernel and footprint of
    # the RMSNorm calibration
    z = torch.empty(n, dtype=src.dtype, device=dev)
    for i in range(LAUNCHES):
        z.copy_(src)
        torch.cuda.synchronize()
        print(f"copy launch {i} done", flush=True)


def qk_summarize(fetch_dir: str, write_dir: str) -> None:
    copy_bytes = COPY_BYTES  # the calibration copy's bytes, each way
    # torch's input set-up launches elementwise kernels too: only the copy counts
    f = _per_kernel(fetch_dir, "FETCH_SIZE", "qk_norm_rope", "copyBuffer")
    w = _per_kernel(write_dir, "WRITE_SIZE", "qk_norm_rope", "copyBuffer")
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    f_k, f_c = mean(f["rmsnorm"]), mean(f["copy"])
    w_k, w_c = mean(w["rmsnorm"]), mean(w["copy"])
    fetch_b = f_k * copy_bytes / f_c
    write_b = w_k * copy_bytes / w_c
    qk = QK_TOKENS * (QK_HQ + QK_HKV) * QK_D * 2
    print(f"qk_norm_rope FETCH_SIZE per launch (raw): {f_k:.1f}  over {len(f['rmsnorm'])} launches")
    print(f"qk_norm_rope WRITE_SIZE per launch (raw): {w_k:.1f}  over {len(w['rmsnorm'])} launches")
    print(f"tokens {QK_TOKENS}, heads {QK_HQ} q + {QK_HKV} k + {QK_HKV} v of {QK_D}")
    print(f"copy    FETCH_SIZE per launch (raw): {f_c:.1f}   WRITE_SIZE: {w_c:.1f}   true bytes each way: {copy_bytes}")
    print(f"calibration factors (bytes per counter unit): fetch {copy_bytes / f_c:.3f}  write {copy_bytes / w_c:.3f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}  (q and k heads: {qk}, x{fetch_b / qk:.4f})")
    print(f"write_bytes_per_launch: {write_b:.0f}  (q and k heads: {qk}, x{write_b / qk:.4f})")
    print(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}  algorithmic_bytes_per_launch: {qk_algorithmic_bytes()}"
          f"  (x{(fetch_b + write_b) / qk_algorithmic_bytes():.4f})")


CEIL_REPS = 20

# (case, bytes moved per launch, kind, lanes, chunks): kind "torch-*" is one of
# torch's kernels, "read" / "write" / "copy" a libmbn_stream.so kernel with
# workgroups of `lanes` lanes moving `chunks` 16-byte chunks each.
CEILING_CASES = [
    ("read only (torch sum)", COPY_BYTES, "torch-sum", 0, 0),
    ("write only (torch fill)", COPY_BYTES, "torch-fill", 0, 0),
    ("copy (torch copy_)", 2 * COPY_BYTES, "torch-copy", 0, 0),
    ("read + write (torch scale)", 2 * COPY_BYTES, "torch-scale", 0, 0),
    ("read only, 4 KiB/WG", COPY_BYTES, "read", 256, 1),
    ("read only, 32 KiB/WG", COPY_BYTES, "read", 256, 8),
    ("write only, 4 KiB/WG", COPY_BYTES, "write", 256, 1),
    ("write only, 32 KiB/WG", COPY_BYTES, "write", 256, 8),
    ("copy, 4 KiB/WG", 2 * COPY_BYTES, "copy", 256, 1),
    ("copy, 8 KiB/WG", 2 * COPY_BYTES, "copy", 512, 1),
    ("copy, 16 KiB/WG", 2 * COPY_BYTES, "copy", 1024, 1),
    ("copy, 16 KiB/WG (4 per lane)", 2 * COPY_BYTES, "copy", 256, 4),
    ("copy, 32 KiB/WG", 2 * COPY_BYTES, "copy", 256, 8),
    ("copy, 32 KiB/WG (1024 lanes)", 2 * COPY_BYTES, "copy", 1024, 2),
    ("copy, 64 KiB/WG", 2 * COPY_BYTES, "copy", 256, 16),
    ("rmsnorm_fwd", 2 * COPY_BYTES + 2 * 16384, "rmsnorm", 0, 0),
]


def stream_lib():
    """ctypes handle of libmbn_stream.so (the streaming reference kernels)."""
    import ctypes

    from memory_bound_normalization_amd.build import STREAM_LIB_PATH

    if not os.path.exists(STREAM_LIB_PATH):
        raise RuntimeError(f"{STREAM_LIB_PATH} is missing: run `python -m memory_bound_normalization_amd.build`")
    h = ctypes.CDLL(STREAM_LIB_PATH)
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
    h.mbn_stream_copy.argtypes = [vp, vp, sz, i32, i32, vp]
    h.mbn_stream_read.argtypes = [vp, vp, sz, i32, i32, vp]
    h.mbn_stream_write.argtypes = [vp, sz, i32, i32, u32, vp]
    for f in (h.mbn_stream_copy, h.mbn_stream_read, h.mbn_stream_write):
        f.restype = i32
    return h


def ceiling() -> None:
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from memory_bound_normalization_amd.timing import HipTimingEvents
    from workloads import RMS_WORKLOADS, make_rms_inputs

    wl = RMS_WORKLOADS["rms_16384x16384"]
    x_bits, w_bits, eps = make_rms_inputs(wl)
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    xs = [x0, x0.clone()]
    ys = [torch.empty_like(x0), torch.empty_like(x0)]
    sink = torch.empty(1024 * 16, dtype=torch.uint8, device=dev)
    sl = stream_lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"libmbn_stream status {rc}")

    def fn_for(kind, lanes, chunks):
        if kind == "torch-sum":
            return lambda i: xs[i].sum(dtype=torch.float32)
        if kind == "torch-fill":
            return lambda i: ys[i].fill_(1.0)
        if kind == "torch-copy":
            return lambda i: ys[i].copy_(xs[i])
        if kind == "torch-scale":
            return lambda i: torch.mul(xs[i], 2.0, out=ys[i])
        if kind == "read":
            return lambda i: ok(sl.mbn_stream_read(xs[i].data_ptr(), sink.data_ptr(), COPY_BYTES, lanes, chunks, sp))
        if kind == "write":
            return lambda i: ok(sl.mbn_stream_write(ys[i].data_ptr(), COPY_BYTES, lanes, chunks, 0x3F803F80, sp))
        if kind == "copy":
            return lambda i: ok(sl.mbn_stream_copy(xs[i].data_ptr(), ys[i].data_ptr(), COPY_BYTES, lanes, chunks, sp))
        return lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps)

    # the copy kernel copies (checked before the timed cases)
    ok(sl.mbn_stream_copy(xs[0].data_ptr(), ys[0].data_ptr(), COPY_BYTES, 256, 8, sp))
    torch.cuda.synchronize()
    if not torch.equal(ys[0].view(torch.int16), xs[0].view(torch.int16)):
        raise RuntimeError("stream copy produced a different buffer")

    timer = HipTimingEvents(stream)
    for name, nbytes, kind, lanes, chunks in CEILING_CASES:
        fn = fn_for(kind, lanes, chunks)
        for i in range(3):
            fn(i % 2)
        torch.cuda.synchronize()
        ev = [(timer.new(), timer.new()) for _ in range(CEIL_REPS)]
        for i, (a, b) in enumerate(ev):
            timer.record(a)
            fn(i % 2)
            timer.record(b)
        torch.cuda.synchronize()
        us = sorted(timer.elapsed_ms(a, b) * 1e3 for a, b in ev)
        timer.close()
        med = us[len(us) // 2]
        print(json.dumps({"case": name, "bytes": nbytes, "median_us": round(med, 2),
                          "GBps": round(nbytes / med / 1e3, 1), "pct_of_8TBps": round(nbytes / med / 1e3 / 80, 2)}),
              flush=True)


def ceiling_summary(d: str) -> None:
    """GB/s per kernel from a rocprofv3 kernel trace of `ceiling`."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    # dispatches of >= 20 us are the 512 MiB kernels: the last ones come in
    # blocks of 3 warm-up + CEIL_REPS per case, in the order of CEILING_CASES
    # (before them: the clone that makes the second buffer set and the check
    # of the copy kernel)
    big = [r for r in rows if int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) > 20000]
    per = 3 + CEIL_REPS
    n = len(CEILING_CASES)
    if len(big) < per * n:
        raise SystemExit(f"expected {per * n} large dispatches, found {len(big)}")
    big = big[len(big) - per * n :]
    for k, (name, nb, *_rest) in enumerate(CEILING_CASES):
        grp = big[k * per + 3 : (k + 1) * per]
        d_us = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
        med = d_us[len(d_us) // 2]
        kname = grp[0]["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
        kname = kname.removeprefix("void ")[:60]
        print(f"{name:<30} {med:9.2f} us {nb / med / 1e3:8.0f} GB/s {nb / med / 1e3 / 80:6.1f}%   {kname}")


# The small workloads beside a plain copy of the same bytes: (case, bytes per
# launch, kind, lanes, chunks) as in CEILING_CASES; "rms-small" is rmsnorm_fwd
# on x[1024, 4096], "qk" qk_norm_rope_fwd on 256 tokens of 32 + 8 + 8 heads.
SMALL_RMS_BYTES = 1024 * 4096 * 2
SMALL_QK_BYTES = 256 * 40 * 128 * 2
SMALL_CASES = [
    ("copy 8 MiB, 4 KiB/WG", 2 * SMALL_RMS_BYTES, "copy", 256, 1),
    ("copy 8 MiB, 8 KiB/WG", 2 * SMALL_RMS_BYTES, "copy", 512, 1),
    ("copy 8 MiB, 16 KiB/WG", 2 * SMALL_RMS_BYTES, "copy", 1024, 1),
    ("rmsnorm_fwd 1024x4096", 2 * SMALL_RMS_BYTES + 2 * 4096, "rms-small", 0, 0),
    ("copy 2.5 MiB, 4 KiB/WG", 2 * SMALL_QK_BYTES, "copy", 256, 1),
    ("copy 2.5 MiB, 8 KiB/WG", 2 * SMALL_QK_BYTES, "copy", 512, 1),
    ("qk_norm_rope_fwd 256 tokens", 2 * SMALL_QK_BYTES + 512 + 8 * 256, "qk", 0, 0),
    ("write 4 KiB (one workgroup)", 4096, "write-tiny", 256, 1),
]
SMALL_REPS = 200


def small() -> None:
    """Times the small workloads and plain copies of their bytes, buffers
    rotated over >= 1 GiB (cold) except the in-place QK tensor set (64 copies,
    160 MiB); read the durations from a kernel trace (`small-summary`)."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from workloads import QK_WORKLOADS, RMS_WORKLOADS, make_qk_inputs, make_rms_inputs

    dev = torch.device("cuda:0")
    sl = stream_lib()
    sp = torch.cuda.current_stream(dev).cuda_stream

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"libmbn_stream status {rc}")

    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    x_bits, w_bits, eps = make_rms_inputs(RMS_WORKLOADS["rms_1024x4096"])
    nrot = (1 << 30) // (2 * SMALL_RMS_BYTES)
    xs = [up(x_bits) for _ in range(nrot)]
    ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
    w = up(w_bits)
    qwl = QK_WORKLOADS["qk_256"]
    qkv_bits, qw_bits, kw_bits, pos, qeps, theta = make_qk_inputs(qwl)
    qs = [up(qkv_bits) for _ in range(64)]
    qw, kw = up(qw_bits), up(kw_bits)
    posg = torch.from_numpy(pos).to(dev)
    qrot = 64
    # the copies of the QK case move the q and k heads' bytes, one tensor per launch
    qk_src = [torch.empty(SMALL_QK_BYTES // 2, dtype=torch.bfloat16, device=dev) for _ in range(qrot)]
    qk_dst = [torch.empty_like(qk_src[0]) for _ in range(qrot)]
    torch.cuda.synchronize()
    for name, nbytes, kind, lanes, chunks in SMALL_CASES:
        for i in range(SMALL_REPS + 20):
            if kind == "copy" and nbytes == 2 * SMALL_RMS_BYTES:
                ok(sl.mbn_stream_copy(xs[i % nrot].data_ptr(), ys[i % nrot].data_ptr(), SMALL_RMS_BYTES, lanes, chunks, sp))
            elif kind == "copy":
                ok(sl.mbn_stream_copy(qk_src[i % qrot].data_ptr(), qk_dst[i % qrot].data_ptr(), SMALL_QK_BYTES, lanes,
                                      chunks, sp))
            elif kind == "rms-small":
                mbn.rmsnorm_fwd(xs[i % nrot], w, ys[i % nrot], eps=eps)
            elif kind == "qk":
                mbn.qk_norm_rope_fwd(qs[i % qrot], qw, kw, posg, qwl.n_q_heads, qwl.n_kv_heads, qwl.head_dim,
                                     eps=qeps, theta=theta)
            else:
                ok(sl.mbn_stream_write(ys[0].data_ptr(), 4096, lanes, chunks, 0, sp))
        torch.cuda.synchronize()
        print(f"{name}: {SMALL_REPS + 20} launches", flush=True)


def small_summary(d: str) -> None:
    """Median GPU duration of each `small` case (its last SMALL_REPS launches)."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ours = [r for r in rows if any(k in r["Kernel_Name"] for k in ("stream_", "rownorm", "qk_norm_rope"))]
    per = SMALL_REPS + 20
    if len(ours) < per * len(SMALL_CASES):
        raise SystemExit(f"expected {per * len(SMALL_CASES)} dispatches, found {len(ours)}")
    ours = ours[len(ours) - per * len(SMALL_CASES):]
    for k, (name, nb, *_rest) in enumerate(SMALL_CASES):
        grp = ours[k * per + 20 : (k + 1) * per]
        d_us = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
        med = d_us[len(d_us) // 2]
        kname = grp[0]["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
        kname = kname.removeprefix("void ").replace("mbn::", "")[:48]
        print(f"{name:<30} {med:8.2f} us  p10 {d_us[len(d_us) // 10]:7.2f}  {nb / med / 1e3:7.0f} GB/s "
              f"{nb / med / 1e3 / 80:6.1f}%   {kname}")


def _rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _per_kernel(d: str, counter: str, kernel: str = "rownorm_kernel", copy: str | None = None):
    """{'rmsnorm': [values...], 'copy': [values...]} for one counter (summed over
    its instances); 'rmsnorm' holds the kernels whose name contains `kernel`,
    'copy' those whose name contains `copy` (default: torch's copy or
    elementwise kernels)."""
    acc = {}
    for r in _rows(d):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    res = {"rmsnorm": [], "copy": []}
    for (_, name), v in sorted(acc.items(), key=lambda kv: int(kv[0][0])):
        if kernel in name:
            res["rmsnorm"].append(v)
        elif (copy in name) if copy else ("copy" in name.lower() or "elementwise" in name.lower()):
            res["copy"].append(v)
    return res


def summarize(fetch_dir: str, write_dir: str, workload: str = DEFAULT_WORKLOAD) -> None:
    sys.path.insert(0, ROOT)
    from workloads import RMS_WORKLOADS

    wl = RMS_WORKLOADS[workload]
    copy_bytes = wl.M * wl.N * 2  # the calibration copy moves x once each way
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    f_r, f_c = mean(f["rmsnorm"]), mean(f["copy"])
    w_r, w_c = mean(w["rmsnorm"]), mean(w["copy"])
    f_scale = copy_bytes / f_c
    w_scale = copy_bytes / w_c
    fetch_b = f_r * f_scale
    write_b = w_r * w_scale
    print(f"rmsnorm FETCH_SIZE per launch (raw, KiB units): {f_r:.1f}  over {len(f['rmsnorm'])} launches")
    print(f"rmsnorm WRITE_SIZE per launch (raw, KiB units): {w_r:.1f}  over {len(w['rmsnorm'])} launches")
    print(f"workload: {workload}  algorithmic_bytes_per_launch: {wl.algorithmic_bytes}")
    print(f"copy    FETCH_SIZE per launch (raw): {f_c:.1f}   WRITE_SIZE: {w_c:.1f}   true bytes each way: {copy_bytes}")
    print(f"calibration factors (bytes per counter unit): fetch {f_scale:.3f}  write {w_scale:.3f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"write_bytes_per_launch: {write_b:.0f}")
    print(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}")


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "ceiling":
        ceiling()
    elif len(sys.argv) >= 3 and sys.argv[1] == "ceiling-summary":
        ceiling_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "small":
        small()
    elif len(sys.argv) == 3 and sys.argv[1] == "small-summary":
        small_summary(sys.argv[2])
    elif len(sys.argv) in (2, 3) and sys.argv[1] == "run":
        run(*sys.argv[2:])
    elif len(sys.argv) == 2 and sys.argv[1] == "qk-run":
        qk_run()
    elif len(sys.argv) == 4 and sys.argv[1] == "qk-summarize":
        qk_summarize(sys.argv[2], sys.argv[3])
    elif len(sys.argv) in (4, 5) and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
