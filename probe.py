"""Short GPU program for hardware-counter runs, and the summarizer of their output.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python probe.py run
    rocprofv3 --pmc WRITE_SIZE -d <dir> -o run -- python probe.py run
    python probe.py summarize <fetch_dir> <write_dir> [workload]

`run [workload]` launches rmsnorm_fwd on x[16384, 16384] (the benchmark
workload; or another RMSNorm workload of `workloads`, e.g. rms_4096x32768) a
few times, then a plain device-to-device copy of the same x (torch's copy
kernel) as the calibration: the counters of the copy, whose true HBM traffic is
known (x's bytes read and written), give the factor that converts each counter
reading into bytes. `summarize` prints the per-launch HBM traffic of the
RMSNorm kernel from the two runs' counter CSV files.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python probe.py qk-run
    rocprofv3 --pmc WRITE_SIZE -d <dir> -o run -- python probe.py qk-run
    python probe.py qk-summarize <fetch_dir> <write_dir>

`qk-run` does the same for qk_norm_rope_fwd on 65536 tokens of 32 q + 8 k + 8 v
heads of 128 (768 MiB, more than the Infinity Cache), calibrated by torch's
device copy of a separate 512 MiB buffer (the RMSNorm runs' calibration
kernel and size);
`qk-summarize` prints its per-launch traffic beside the
algorithmic bytes (q and k heads read and written, v heads untouched).

    rocprofv3 --kernel-trace --stats -d <dir> -o run -- python probe.py ceiling
    python probe.py ceiling-summary <dir>

    rocprofv3 --kernel-trace -d <dir> -o run -- python probe.py small
    python probe.py small-summary <dir>

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
on this part, the reference for the RMSNorm kernel's fraction of peak. The
copies are also timed with other cache policies on their stores (nt sc1, sc1,
sc0 sc1).

    python probe.py store-policy > <log>
    python probe.py store-policy-summary <log>

`store-policy` times the library's RMSNorm on x[16384, 16384] against the same
kernel compiled with those store policies on its output stores
(probe_csrc/store_policy.hip, built on first use), after checking that every
variant's output equals the library's bit for bit.

    python probe.py staging > <log>
    python probe.py staging-summary <log>
    python probe.py late-weights > <log>
    python probe.py late-weights-summary <log>

`staging` times rmsnorm_fwd where its launch tables hold each lane's chunks
of the row in VGPRs (N = 32768 and 65536) against the staged-row (LDS) kernel
those widths used before; `late-weights` the N <= 8192 band's entry, which
loads the weight after the reduction, against the band's previous entry. The
prior entries are the library's own kernels, compiled from its source by
probe_csrc/prior_entries.hip; same data, outputs compared first.

    python probe.py qk-pattern > <log>
    python probe.py qk-pattern-summary <log>
    python probe.py qk-ab > <log>
    python probe.py qk-ab-summary <log>
    python probe.py any-width-ab [N:offset,...] > <log>
    python probe.py any-width-summary <log>

`qk-pattern` times qk_norm_rope_fwd against its memory access pattern with no
arithmetic (the q and k bytes of each token read and written back in place).
`qk-ab` times qk_norm_rope_fwd against the prior QK kernel
(probe_csrc/prior_qk_norm_rope.hip) over token and head counts.
`any-width-ab` times the any-width row norms against the prior any-width path
(probe_csrc/prior_any_width.hip).

The other commands, each the source of a committed summary: `timeline`,
`timeline-summary` (per-workgroup timelines), `variants`, `claim`, `stream`,
`sizes`, `experiments-summary` (the geometry, claimed-tail, pipelined-kernel
and size experiments), `trace-summary`, `suite-summary` (kernel-trace
summaries of the bench commands).
"""

from __future__ import annotations

import csv
import ctypes
import glob
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PROBE_CSRC = os.path.join(ROOT, "probe_csrc")
STREAM_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_stream.so")
LAUNCHES = 5
COPY_BYTES = 16384 * 16384 * 2


DEFAULT_WORKLOAD = "rms_16384x16384"


class HipTimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence.

    A default event record performs a system-scope release (an L2 writeback and
    invalidate) when it completes; the HIP header documents this flag for
    events used only to measure time, to avoid that cost and its effect on
    the following work. Measured on MI355X around each 170 us RMSNorm launch:
    default events (torch's) read 170.8 us, these 169.1 us, the rocprofv3
    kernel trace 166.4 us. Recorded on the stream the kernels run on.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream):
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")  # already loaded by torch
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.events = []

    def new(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(e)
        return e

    def record(self, e):
        rc = self.hip.hipEventRecord(e, self.stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


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
    ("copy, 4 KiB/WG, stores nt (inline asm)", 2 * COPY_BYTES, "copy-pol0", 256, 1),
    ("copy, 4 KiB/WG, stores nt sc1", 2 * COPY_BYTES, "copy-pol1", 256, 1),
    ("copy, 4 KiB/WG, stores sc1", 2 * COPY_BYTES, "copy-pol2", 256, 1),
    ("copy, 4 KiB/WG, stores sc0 sc1", 2 * COPY_BYTES, "copy-pol3", 256, 1),
    ("copy, 32 KiB/WG, stores nt (inline asm)", 2 * COPY_BYTES, "copy-pol0", 256, 8),
    ("copy, 32 KiB/WG, stores nt sc1", 2 * COPY_BYTES, "copy-pol1", 256, 8),
    ("rmsnorm_fwd", 2 * COPY_BYTES + 2 * 16384, "rmsnorm", 0, 0),
]


def build_stream(verbose: bool = False) -> str:
    """Compile probe_csrc/stream.hip into probe_csrc/libmbn_stream.so (the
    streaming reference kernels; not part of the library); always rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=STREAM_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "stream.hip")])


def stream_lib():
    """ctypes handle of libmbn_stream.so (the streaming reference kernels),
    compiled first when it is not there."""
    import ctypes

    if not os.path.exists(STREAM_LIB_PATH):
        build_stream()
    h = ctypes.CDLL(STREAM_LIB_PATH)
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
    h.mbn_stream_copy.argtypes = [vp, vp, sz, i32, i32, vp]
    h.mbn_stream_read.argtypes = [vp, vp, sz, i32, i32, vp]
    h.mbn_stream_write.argtypes = [vp, sz, i32, i32, u32, vp]
    h.mbn_stream_copy_policy.argtypes = [vp, vp, sz, i32, i32, vp]
    h.mbn_stream_copy_timed.argtypes = [vp, vp, sz, i32, i32, vp, vp, vp]
    h.mbn_stream_qk_pattern.argtypes = [vp, ctypes.c_int64, i32, i32, vp]
    for f in (h.mbn_stream_copy, h.mbn_stream_read, h.mbn_stream_write, h.mbn_stream_copy_policy,
              h.mbn_stream_qk_pattern, h.mbn_stream_copy_timed):
        f.restype = i32
    return h


def ceiling() -> None:
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
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
        if kind.startswith("copy-pol"):
            pol = int(kind[len("copy-pol"):])
            return lambda i: ok(sl.mbn_stream_copy_policy(xs[i].data_ptr(), ys[i].data_ptr(), COPY_BYTES, chunks, pol,
                                                          sp))
        return lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps)

    # the copy kernels copy (checked before the timed cases)
    copies = [lambda: ok(sl.mbn_stream_copy(xs[0].data_ptr(), ys[0].data_ptr(), COPY_BYTES, 256, 8, sp))]
    copies += [lambda c=c, p=p: ok(sl.mbn_stream_copy_policy(xs[0].data_ptr(), ys[0].data_ptr(), COPY_BYTES, c, p, sp))
               for c in (1, 8) for p in range(4)]
    for copy in copies:
        ys[0].zero_()
        copy()
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
        print(f"{name:<40} {med:9.2f} us {nb / med / 1e3:8.0f} GB/s {nb / med / 1e3 / 80:6.1f}%   {kname}")


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


# The one-shot row-norm kernels (staged rows, rows in VGPRs) by name.
ROW_KERNELS = ("rownorm_kernel", "rownorm_regs_kernel")


def _per_kernel(d: str, counter: str, kernel: str | tuple = ROW_KERNELS, copy: str | None = None):
    """{'rmsnorm': [values...], 'copy': [values...]} for one counter (summed over
    its instances); 'rmsnorm' holds the kernels whose name contains `kernel`
    (or one of them), 'copy' those whose name contains `copy` (default: torch's
    copy or elementwise kernels)."""
    kernels = (kernel,) if isinstance(kernel, str) else kernel
    acc = {}
    for r in _rows(d):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    res = {"rmsnorm": [], "copy": []}
    for (_, name), v in sorted(acc.items(), key=lambda kv: int(kv[0][0])):
        if any(k in name for k in kernels):
            res["rmsnorm"].append(v)
        elif (copy in name) if copy else ("copy" in name.lower() or "elementwise" in name.lower()):
            res["copy"].append(v)
    return res


KERNEL_SOURCES = [os.path.join(ROOT, "memory_bound_normalization_amd", "csrc", f) for f in ("rownorm.hip", "device.h")]


def kernel_source_hash() -> str:
    """First 16 hex digits of sha256(csrc/rownorm.hip + csrc/device.h): the
    row-norm kernels' source, recorded with their counter summaries."""
    import hashlib

    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summarize(fetch_dir: str, write_dir: str, workload: str = DEFAULT_WORKLOAD) -> None:
    """Print the HBM-traffic summary of rmsnorm_fwd on `workload` from the
    FETCH_SIZE and WRITE_SIZE runs of `run` (the text committed under
    profiles/)."""
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
    rd = wl.M * wl.N * 2 + 2 * wl.N
    wr = wl.M * wl.N * 2
    arg = "" if workload == DEFAULT_WORKLOAD else f" {workload}"
    title = f"rmsnorm_fwd HBM traffic per launch, x[{wl.M}, {wl.N}] bf16, MI355X (gfx950)"
    print(title)
    print("=" * len(title))
    print()
    print("Commands (from the repository root, TMPDIR=/tmp), one counter per run:")
    print(f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o run -- \\")
    print(f"      python -u probe.py run{arg}")
    print(f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o run -- \\")
    print(f"      python -u probe.py run{arg}")
    print(f"  python probe.py summarize {fetch_dir} {write_dir}{arg}")
    print()
    print(f"The probe launches rmsnorm_fwd {LAUNCHES} times on the workload, then torch's device copy")
    print(f"of the same {copy_bytes:,} B {LAUNCHES} times (the calibration kernel: true traffic")
    print(f"{copy_bytes:,} B read and {copy_bytes:,} B written per launch). The figures are")
    print("therefore relative to that copy: an over-fetch a plain copy shares would not show.")
    print()
    print("Raw counters (mean per dispatch, as rocprofv3 reports them):")
    print(f"  rmsnorm  FETCH_SIZE {f_r:.1f}   WRITE_SIZE {w_r:.1f}   ({len(f['rmsnorm'])} / {len(w['rmsnorm'])} dispatches)")
    print(f"  copy     FETCH_SIZE {f_c:.1f}   WRITE_SIZE {w_c:.1f}   ({len(f['copy'])} / {len(w['copy'])} dispatches)")
    print(f"Calibration (true bytes / copy counter): fetch x{f_scale:.3f}, write x{w_scale:.3f}")
    print()
    print("Per rmsnorm launch:")
    print(f"  fetch_bytes_per_launch: {fetch_b:.0f}   (algorithmic read {rd:,}: {100 * (fetch_b / rd - 1):+.3f}%)")
    print(f"  write_bytes_per_launch: {write_b:.0f}   (algorithmic write {wr:,}: {100 * (write_b / wr - 1):+.3f}%)")
    print(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}")
    print(f"algorithmic_bytes_per_launch: {wl.algorithmic_bytes}   (traffic / algorithmic = "
          f"{(fetch_b + write_b) / wl.algorithmic_bytes:.4f})")
    print()
    print(f"kernel_source_sha256_16: {kernel_source_hash()}")
    print("(sha256 of csrc/rownorm.hip + csrc/device.h, first 16 hex digits; bench.py")
    print("reports roofline.traffic only while this matches the current source.)")


TL_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_tl.so")
TL_MAGIC = 0x74696D65
TICKS_PER_US = 100.0  # s_memrealtime: 100 MHz constant-rate clock


def build_timeline(verbose: bool = False) -> str:
    """Compile probe_csrc/timeline.hip (the library's row-norm source with its
    timeline marks defined, and a marked copy) into probe_csrc/libmbn_tl.so."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=TL_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "timeline.hip")])


def timeline_lib():
    import ctypes

    if not os.path.exists(TL_LIB_PATH):
        build_timeline()
    h = ctypes.CDLL(TL_LIB_PATH)
    vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    h.mbn_tl_rmsnorm.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, vp]
    h.mbn_tl_copy.argtypes = [vp, vp, sz, i32, vp]
    h.mbn_tl_clear.argtypes = [i64]
    h.mbn_tl_fetch.argtypes = [vp, i64]
    for f in (h.mbn_tl_rmsnorm, h.mbn_tl_copy, h.mbn_tl_clear, h.mbn_tl_fetch, h.mbn_tl_max_blocks):
        f.restype = i32
    return h


def timeline_metrics(rec, total_bytes: float) -> dict:
    """Launch metrics from per-workgroup records [nblocks, 8] (start, landed,
    last store issued, stores done, XCC_ID, HW_ID, block, magic).

    Reads are counted when a workgroup's data has landed, writes when its
    stores have completed; `steady` is the rate between 20% and 80% of the
    launch's bytes, `head` / `tail` the time lost before / after that
    stretch against the steady rate, `xcd_end_spread` the gap between the first
    and the last XCD to finish.
    """
    import numpy as np

    ok = rec[:, 7] == TL_MAGIC
    r = rec[ok].astype(np.float64)
    n = int(ok.sum())
    t0 = r[:, 0].min()
    start, landed, issued, done = ((r[:, i] - t0) / TICKS_PER_US for i in range(4))
    xcc = rec[ok, 4].astype(np.int64) & 0xF
    span = float(done.max())
    half = total_bytes / 2 / n
    ev_t = np.concatenate([landed, done])
    order = np.argsort(ev_t, kind="stable")
    cum = np.cumsum(np.full(2 * n, half))
    ts = ev_t[order]

    def t_at(frac):
        return float(ts[np.searchsorted(cum, frac * total_bytes)])

    t20, t80 = t_at(0.2), t_at(0.8)
    steady = 0.6 * total_bytes / (t80 - t20) / 1e3  # GB/s (bytes per us / 1e3)
    ideal = total_bytes / steady / 1e3
    xcd_end = {int(k): float(done[xcc == k].max()) for k in np.unique(xcc)}
    ends = np.array(list(xcd_end.values()))
    # resident workgroups over time
    edges = np.concatenate([start, done])
    delta = np.concatenate([np.ones(n), -np.ones(n)])
    occ = np.cumsum(delta[np.argsort(edges, kind="stable")])
    # end of a workgroup -> start of the next one on the same CU (HW_ID: CU
    # bits 11:8, SH bit 12, SE bits 15:13; with the XCD that names the CU)
    hw = rec[ok, 5].astype(np.int64)
    cu = xcc * 4096 + ((hw >> 13) & 7) * 256 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 15)
    gaps = []
    for k in np.unique(cu):
        m = cu == k
        ss = np.sort(start[m])
        j = np.searchsorted(ss, done[m])
        gaps.append((ss[j[j < len(ss)]] - done[m][j < len(ss)]))
    gaps = np.concatenate(gaps) if gaps else np.zeros(1)
    return {
        "blocks": n,
        "cus": int(len(np.unique(cu))),
        "gap_us_median": round(float(np.median(gaps)), 2),
        "gap_us_p90": round(float(np.percentile(gaps, 90)), 2),
        "span_us": round(span, 2),
        "GBps_span": round(total_bytes / span / 1e3, 1),
        "steady_GBps": round(steady, 1),
        "steady_pct": round(100 * steady / 8000.0, 2),
        "ideal_us_at_steady": round(ideal, 2),
        "overhead_us": round(span - ideal, 2),
        "head_us": round(t20 - 0.2 * ideal, 2),
        "tail_us": round(span - t80 - 0.2 * ideal, 2),
        "last_start_us": round(float(start.max()), 2),
        "drain_us": round(span - float(start.max()), 2),
        "first_end_us": round(float(done.min()), 2),
        "xcd_end_us": {k: round(v, 2) for k, v in sorted(xcd_end.items())},
        "xcd_end_spread_us": round(float(ends.max() - ends.min()), 2),
        "xcd_blocks": {int(k): int((xcc == k).sum()) for k in np.unique(xcc)},
        "max_resident_wgs": int(occ.max()),
        "wg_life_us_median": round(float(np.median(done - start)), 2),
        "wg_land_us_median": round(float(np.median(landed - start)), 2),
        "wg_store_us_median": round(float(np.median(done - landed)), 2),
    }


def _timeline_total(name: str) -> int:
    """Algorithmic bytes of a timeline case: rmsnorm_MxN or a copy of 512 MiB."""
    if name.startswith("rmsnorm_"):
        m, n = (int(v) for v in name.split("_")[1].split("x"))
        return 2 * m * n * 2 + 2 * n
    return 2 * 16384 * 16384 * 2


TIMELINE_SHAPES = [(16384, 16384), (8192, 8192), (4096, 32768)]


def timeline(out_dir: str = "probe_out/timeline", launches: int = 4) -> None:
    """Per-workgroup timelines of rmsnorm_fwd (the library's kernel with its
    marks compiled in) at x[16384, 16384], x[8192, 8192] and x[4096, 32768],
    and of the streaming copy of 512 MiB (4 KiB and 32 KiB per workgroup).
    Records are saved per traced launch (.npz, times relative to the launch's
    first workgroup start).
    Before each traced launch the part runs ~40 ms of back-to-back library
    launches at 16384 x 16384 (1 GiB each, so the traced launch's data is not
    in the 256 MiB Infinity Cache); records saved as .npy, one JSON line of
    metrics per traced launch."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    os.makedirs(out_dir, exist_ok=True)
    tl = timeline_lib()
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    bufs = {}
    for M, N in TIMELINE_SHAPES:
        x = torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16)
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        bufs[(M, N)] = (x, w, torch.empty_like(x))
    x, w, y = bufs[(16384, 16384)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    nbytes = x.numel() * 2
    for _ in range(2400):
        mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
    torch.cuda.synchronize()
    timer = HipTimingEvents(stream)
    ev = [(timer.new(), timer.new()) for _ in range(200)]
    for a, b in ev:
        timer.record(a)
        mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
        timer.record(b)
    torch.cuda.synchronize()
    lib_us = [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
    print(json.dumps({"kernel": "library rmsnorm_fwd 16384x16384 (no marks)", "launches": len(lib_us),
                      "mean_us": round(sum(lib_us) / len(lib_us), 2), "min_us": round(min(lib_us), 2)}), flush=True)
    rmax = tl.mbn_tl_max_blocks()

    def rms_case(M, N):
        xm, wm, ym = bufs[(M, N)]
        return lambda: tl.mbn_tl_rmsnorm(xm.data_ptr(), wm.data_ptr(), ym.data_ptr(), M, N, 1e-6, sp)

    cases = [(f"rmsnorm_{M}x{N}", rms_case(M, N)) for M, N in TIMELINE_SHAPES]
    cases += [("copy_4KiB_per_wg", lambda: tl.mbn_tl_copy(x.data_ptr(), y.data_ptr(), nbytes, 1, sp)),
              ("copy_32KiB_per_wg", lambda: tl.mbn_tl_copy(x.data_ptr(), y.data_ptr(), nbytes, 8, sp))]
    for name, fn in cases:
        total = _timeline_total(name)
        for i in range(launches):
            for _ in range(240):
                mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
            torch.cuda.synchronize()
            if tl.mbn_tl_clear(rmax) != 0:
                raise RuntimeError("mbn_tl_clear failed")
            a, b = timer.new(), timer.new()
            timer.record(a)
            rc = fn()
            timer.record(b)
            if rc != 0:
                raise RuntimeError(f"{name}: launch status {rc}")
            torch.cuda.synchronize()
            rec = np.zeros((rmax, 8), dtype=np.uint64)
            if tl.mbn_tl_fetch(rec.ctypes.data, rmax) != 0:
                raise RuntimeError("mbn_tl_fetch failed")
            rec = rec[rec[:, 7] == TL_MAGIC]
            rec[:, :4] -= rec[:, 0].min()  # times relative to the first start (compresses well)
            np.savez_compressed(os.path.join(out_dir, f"{name}_{i}.npz"), rec=rec)
            m = timeline_metrics(rec, total)
            m.update({"case": name, "launch": i, "event_us": round(timer.elapsed_ms(a, b) * 1e3, 2)})
            print(json.dumps(m), flush=True)
    timer.close()


def timeline_summary(d: str) -> None:
    """Median metrics per case over the saved launches, and the bandwidth over
    time (4 us bins) of the median-span launch of rmsnorm_16384x16384 and
    copy_4KiB_per_wg."""
    import numpy as np

    names = sorted({os.path.basename(f).rsplit("_", 1)[0] for f in glob.glob(os.path.join(d, "*_*.npz"))})
    for name in names:
        total = _timeline_total(name)
        files = sorted(glob.glob(os.path.join(d, f"{name}_*.npz")))
        if not files:
            continue
        recs = [np.load(f)["rec"] for f in files]
        ms = [timeline_metrics(r, total) for r in recs]
        keys = ["span_us", "GBps_span", "steady_GBps", "steady_pct", "overhead_us", "head_us", "tail_us",
                "gap_us_median", "gap_us_p90",
                "drain_us", "xcd_end_spread_us", "max_resident_wgs", "wg_life_us_median", "wg_land_us_median",
                "wg_store_us_median", "first_end_us"]
        print(f"{name}: {len(ms)} launches, {ms[0]['blocks']} workgroups")
        for k in keys:
            v = [m[k] for m in ms]
            print(f"  {k:22s} median {np.median(v):9.2f}   min {min(v):9.2f}   max {max(v):9.2f}")
        print("  XCD finish times (us after the first workgroup start), per launch:")
        for m in ms:
            e = m["xcd_end_us"]
            print("    " + " ".join(f"{e[k]:7.2f}" for k in sorted(e)) + f"   spread {m['xcd_end_spread_us']:.2f}")
        if name not in ("rmsnorm_16384x16384", "copy_4KiB_per_wg"):
            continue
        med = sorted(range(len(ms)), key=lambda i: ms[i]["span_us"])[len(ms) // 2]
        r = recs[med][recs[med][:, 7] == TL_MAGIC].astype(np.float64)
        t0 = r[:, 0].min()
        landed, done = (r[:, 1] - t0) / TICKS_PER_US, (r[:, 3] - t0) / TICKS_PER_US
        n = len(r)
        half = total / 2 / n
        bins = np.arange(0.0, done.max() + 4.0, 4.0)
        rd = np.histogram(landed, bins)[0] * half / 4.0 / 1e3
        wr = np.histogram(done, bins)[0] * half / 4.0 / 1e3
        print(f"  GB/s per 4 us bin (launch {med}): rows landed + rows written = total, % of 8 TB/s")
        for i in range(len(bins) - 1):
            tot = rd[i] + wr[i]
            print(f"    {bins[i]:6.1f}-{bins[i + 1]:6.1f} us  {rd[i]:7.0f} + {wr[i]:7.0f} = {tot:7.0f}  {100 * tot / 8000:5.1f}%")


def sizes() -> None:
    """Kernel time against size at N = 16384: the library's rmsnorm_fwd and the
    4 KiB-per-workgroup streaming copy of the same bytes, M = 8192 ... 131072
    (event mean of 100 launches after 50), and a least-squares line per kernel:
    its slope is the steady-state rate, its intercept the per-launch overhead."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    N = 16384
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sl = stream_lib()
    timer = HipTimingEvents(stream)
    Ms = [8192, 16384, 32768, 65536, 131072]
    xbig = torch.empty(max(Ms), N, dtype=torch.bfloat16, device=dev).normal_()
    ybig = torch.empty_like(xbig)
    w = torch.ones(N, dtype=torch.bfloat16, device=dev)
    for _ in range(2400):
        mbn.rmsnorm_fwd(xbig[:16384], w, ybig[:16384], eps=1e-6)
    torch.cuda.synchronize()
    res = {"rmsnorm": [], "copy": []}
    for M in Ms:
        x, y = xbig[:M], ybig[:M]
        fns = {"rmsnorm": lambda: mbn.rmsnorm_fwd(x, w, y, eps=1e-6),
               "copy": lambda: sl.mbn_stream_copy(x.data_ptr(), y.data_ptr(), M * N * 2, 256, 1, sp)}
        for name, fn in fns.items():
            for _ in range(50):
                fn()
            ev = [(timer.new(), timer.new()) for _ in range(100)]
            for a, b in ev:
                timer.record(a)
                fn()
                timer.record(b)
            torch.cuda.synchronize()
            us = float(np.mean([timer.elapsed_ms(a, b) * 1e3 for a, b in ev]))
            nb = 2 * M * N * 2 + (2 * N if name == "rmsnorm" else 0)
            res[name].append((nb, us))
            print(json.dumps({"kernel": name, "M": M, "N": N, "bytes": nb, "mean_us": round(us, 2),
                              "pct": round(100 * nb / us / 1e3 / 8000, 2)}), flush=True)
            timer.close()
    for name, pts in res.items():
        b = np.array([p[0] for p in pts], dtype=np.float64)
        t = np.array([p[1] for p in pts])
        slope, icpt = np.polyfit(b, t, 1)
        print(json.dumps({"fit": name, "steady_GBps": round(1 / slope / 1e3, 1),
                          "steady_pct": round(100 / slope / 1e3 / 8000, 2), "intercept_us": round(icpt, 2)}),
              flush=True)


VARIANTS = {
    0: "N=16384: 2 lane sets x 128 lanes, 1 row each, cap 2, XCD group 4 (the table's entry)",
    1: "N=16384: 128 lanes, 1 row, cap 4, group 4",
    2: "N=16384: 128 lanes, 1 row, cap 2, group 4",
    3: "N=16384: 256 lanes, 1 row, cap 4, group 4",
    4: "N=16384: 2 x 128 lanes, cap 2, group 0",
    5: "N=16384: 128 lanes, 1 row, cap 5, group 4",
    6: "N=16384: 2 x 128 lanes, cap 2, group 8",
    7: "N=16384: 128 lanes, 2 rows per lane set, cap 2, group 4",
    8: "N=16384: 256 lanes, 1 row, cap 3, group 4",
    9: "N=16384: 2 x 128 lanes, cap 1, group 4",
    10: "N=32768: 1024 lanes, 1 row, no cap, group 0 (the staged-row entry)",
    11: "N=32768: 512 lanes, cap 2, group 0",
    12: "N=32768: 256 lanes, cap 2, group 0",
    13: "N=32768: 512 lanes, cap 2, group 4",
    14: "N=32768: 1024 lanes, no cap, group 4",
    15: "N=32768: 256 lanes, cap 2, group 4",
}


def variants(out_dir: str = "probe_out/variants", rounds: int = 3, launches: int = 60) -> None:
    """Geometry variants of the library's one-shot RMSNorm kernel (timeline
    marks compiled in) at x[16384, 16384] (variants 0-9) and x[4096, 32768]
    (10-15): event median over `launches` launches per round, rounds
    interleaved, plus one traced launch per variant (saved as .npz)."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    os.makedirs(out_dir, exist_ok=True)
    tl = timeline_lib()
    tl.mbn_tl_rmsnorm_variant.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                                                  ctypes.c_void_p, ctypes.c_int]
    tl.mbn_tl_rmsnorm_variant.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(12)
    shapes = {16384: (16384, 16384), 32768: (4096, 32768)}
    bufs = {}
    for n, (M, N) in shapes.items():
        x = torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16)
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        bufs[n] = (M, N, x, w, torch.empty_like(x), torch.empty_like(x))
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    M0, N0, x0, w0, y0, _ = bufs[16384]
    for _ in range(2400):
        mbn.rmsnorm_fwd(x0, w0, y0, eps=1e-6)
    torch.cuda.synchronize()
    for v in VARIANTS:  # first launch of each kernel (module load) outside the timing
        M, N, x, w, y, y2 = bufs[16384 if v < 10 else 32768]
        if tl.mbn_tl_rmsnorm_variant(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, 1e-6, sp, v) != 0:
            raise RuntimeError(f"variant {v}: launch failed")
    torch.cuda.synchronize()
    timer = HipTimingEvents(stream)
    res = {v: [] for v in VARIANTS}
    lib_res = {16384: [], 32768: []}
    for rnd in range(rounds):
        for n in (16384, 32768):
            M, N, x, w, y, y2 = bufs[n]
            ev = [(timer.new(), timer.new()) for _ in range(launches)]
            for i, (a, b) in enumerate(ev):
                timer.record(a)
                mbn.rmsnorm_fwd(x, w, y if i % 2 else y2, eps=1e-6)
                timer.record(b)
            torch.cuda.synchronize()
            lib_res[n] += [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
            timer.close()
        for v in VARIANTS:
            M, N, x, w, y, y2 = bufs[16384 if v < 10 else 32768]
            ev = [(timer.new(), timer.new()) for _ in range(launches)]
            for i, (a, b) in enumerate(ev):
                timer.record(a)
                rc = tl.mbn_tl_rmsnorm_variant(x.data_ptr(), w.data_ptr(), (y if i % 2 else y2).data_ptr(), M, N,
                                               1e-6, sp, v)
                timer.record(b)
                if rc != 0:
                    raise RuntimeError(f"variant {v}: status {rc}")
            torch.cuda.synchronize()
            res[v] += [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
            timer.close()
        print(f"round {rnd} done", flush=True)
    rmax = tl.mbn_tl_max_blocks()
    for n in (16384, 32768):
        M, N = shapes[n]
        nb = 2 * M * N * 2 + 2 * N
        us = float(np.median(lib_res[n]))
        print(json.dumps({"variant": "library", "N": n, "median_us": round(us, 2),
                          "pct": round(100 * nb / us / 1e3 / 8000, 2)}), flush=True)
    for v, desc in VARIANTS.items():
        M, N, x, w, y, y2 = bufs[16384 if v < 10 else 32768]
        nb = 2 * M * N * 2 + 2 * N
        us = float(np.median(res[v]))
        for _ in range(100):
            mbn.rmsnorm_fwd(x0, w0, y0, eps=1e-6)
        torch.cuda.synchronize()
        tl.mbn_tl_clear(rmax)
        if tl.mbn_tl_rmsnorm_variant(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, 1e-6, sp, v) != 0:
            raise RuntimeError(f"variant {v}: launch failed")
        torch.cuda.synchronize()
        rec = np.zeros((rmax, 8), dtype=np.uint64)
        tl.mbn_tl_fetch(rec.ctypes.data, rmax)
        rec = rec[rec[:, 7] == TL_MAGIC]
        rec[:, :4] -= rec[:, 0].min()
        np.savez_compressed(os.path.join(out_dir, f"variant{v}.npz"), rec=rec)
        m = timeline_metrics(rec, nb)
        keep = {k: m[k] for k in ("span_us", "steady_pct", "overhead_us", "gap_us_median", "gap_us_p90",
                                  "xcd_end_spread_us", "max_resident_wgs", "wg_land_us_median",
                                  "wg_store_us_median")}
        print(json.dumps({"variant": v, "desc": desc, "median_us": round(us, 2),
                          "pct": round(100 * nb / us / 1e3 / 8000, 2), **keep}), flush=True)


SP_POLICIES = {0: "nt (inline asm)", 1: "nt sc1", 2: "sc1", 3: "sc0 sc1"}


def sp_lib_path(policy: int) -> str:
    return os.path.join(PROBE_CSRC, f"libmbn_sp{policy}.so")


def store_policy_source() -> str:
    """The library's csrc/rownorm.hip with the one-shot kernel's output store
    (pass 2 of rownorm_block: its only store_nt_16 of y) replaced by
    MBN_STORE_Y, which probe_csrc/store_policy.hip defines."""
    with open(os.path.join(ROOT, "memory_bound_normalization_amd", "csrc", "rownorm.hip")) as f:
        text = f.read()
    start = text.index("rownorm_block(const RowNormArgs")
    end = text.index(") rownorm_kernel(RowNormArgs a)", start)  # the body ends before the kernel that calls it
    store = "store_nt_16(yrow + k, o);"
    if text.count(store, start, end) != 1:
        raise RuntimeError("rownorm.hip: expected exactly one output store in rownorm_block")
    i = text.index(store, start, end)
    return text[:i] + "MBN_STORE_Y(yrow + k, o);" + text[i + len(store):]


def build_store_policy(verbose: bool = False) -> None:
    """Compile probe_csrc/store_policy.hip once per store policy (the library's
    row-norm source with another cache policy on pass 2's stores) into
    probe_csrc/libmbn_sp<policy>.so; always rebuilds."""
    sys.path.insert(0, ROOT)
    from concurrent.futures import ThreadPoolExecutor

    from memory_bound_normalization_amd.build import build

    csrc = os.path.join(ROOT, "memory_bound_normalization_amd", "csrc")
    gen = os.path.join(PROBE_CSRC, "gen")
    os.makedirs(gen, exist_ok=True)
    with open(os.path.join(gen, "rownorm_store_policy.hip"), "w") as f:
        f.write(store_policy_source())
    src = [os.path.join(PROBE_CSRC, "store_policy.hip")]
    with ThreadPoolExecutor(len(SP_POLICIES)) as ex:
        list(ex.map(lambda p: build(verbose=verbose, out=sp_lib_path(p),
                                    extra=["-I", gen, "-I", csrc, f"-DMBN_PROBE_POLICY={p}"], sources_=src),
                    SP_POLICIES))


def store_policy(rounds: int = 4, launches: int = 60) -> None:
    """The library's RMSNorm at x[16384, 16384] against the same kernel with
    other cache policies on its output stores (libmbn_sp<policy>.so): every
    output checked bit for bit against the library's, then event medians over
    `launches` launches per round, rounds interleaved (order reversed every
    other round), two buffer sets alternating."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    if not all(os.path.exists(sp_lib_path(p)) for p in SP_POLICIES):
        build_store_policy()
    libs = {}
    for p in SP_POLICIES:
        h = ctypes.CDLL(sp_lib_path(p))
        h.mbn_sp_rmsnorm.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                                             ctypes.c_void_p]
        h.mbn_sp_rmsnorm.restype = ctypes.c_int
        libs[p] = h
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(21)
    M = N = 16384
    xs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(2)]
    w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    ys = [torch.empty_like(xs[0]) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    nb = 2 * M * N * 2 + 2 * N

    def call(k, i):
        if k == "library":
            mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=1e-6)
            return
        rc = libs[k].mbn_sp_rmsnorm(xs[i].data_ptr(), w.data_ptr(), ys[i].data_ptr(), M, N, 1e-6, sp)
        if rc != 0:
            raise RuntimeError(f"store policy {k}: status {rc}")

    kinds = ["library", *SP_POLICIES]
    call("library", 0)
    torch.cuda.synchronize()
    ref = ys[0].clone()
    for k in SP_POLICIES:
        ys[0].zero_()
        call(k, 0)
        torch.cuda.synchronize()
        if not torch.equal(ys[0].view(torch.int16), ref.view(torch.int16)):
            raise RuntimeError(f"store policy {k}: output differs from the library's")
    del ref
    print(json.dumps({"check": "every policy's output equals the library's bit for bit"}), flush=True)
    for _ in range(2400):
        call("library", 0)
    torch.cuda.synchronize()
    timer = HipTimingEvents(stream)
    res = {k: [] for k in kinds}
    for rnd in range(rounds):
        for k in (kinds if rnd % 2 == 0 else kinds[::-1]):
            for i in range(6):
                call(k, i % 2)
            torch.cuda.synchronize()
            ev = [(timer.new(), timer.new()) for _ in range(launches)]
            for i, (a, b) in enumerate(ev):
                timer.record(a)
                call(k, i % 2)
                timer.record(b)
            torch.cuda.synchronize()
            res[k].append(float(np.median([timer.elapsed_ms(a, b) * 1e3 for a, b in ev])))
            timer.close()
        print(f"round {rnd} done", flush=True)
    for k in kinds:
        us = float(np.median(res[k]))
        print(json.dumps({"kernel": k if k == "library" else f"policy {k}",
                          "stores": "nt (compiler)" if k == "library" else SP_POLICIES[k],
                          "median_us": round(us, 2), "pct": round(100 * nb / us / 1e3 / 8000, 2),
                          "rounds_us": [round(t, 2) for t in res[k]]}), flush=True)


def store_policy_summary(log: str) -> None:
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    print("RMSNorm x[16384, 16384], the library's kernel with other cache policies on its output stores")
    print("(event medians; per round: median of 60 launches; reported: median of the round medians):")
    print(f"  {'kernel':<12} {'stores':<18} {'median_us':>9} {'% of 8 TB/s':>12}  rounds")
    for r in rows:
        if "check" in r:
            continue
        print(f"  {r['kernel']:<12} {r['stores']:<18} {r['median_us']:>9.2f} {r['pct']:>12.2f}  "
              + " ".join(f"{t:.1f}" for t in r["rounds_us"]))
    if any("check" in r for r in rows):
        print("  every policy's output equals the library's bit for bit")


PRIOR_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_prior.so")
STAGING_SHAPES = [(1024, 32768), (4096, 32768), (8192, 32768), (512, 65536), (2048, 65536), (4096, 65536)]


def build_prior(verbose: bool = False) -> str:
    """Compile probe_csrc/prior_entries.hip (launch-table entries the library
    used before: the staged-row kernel at N = 32768 and 65536, the N <= 8192
    band's early-weight entry) into probe_csrc/libmbn_prior.so; always
    rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=PRIOR_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "prior_entries.hip")])


def prior_lib():
    if not os.path.exists(PRIOR_LIB_PATH):
        build_prior()
    h = ctypes.CDLL(PRIOR_LIB_PATH)
    for f in (h.mbn_lds_rmsnorm, h.mbn_early_w_rmsnorm):
        f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
        f.restype = ctypes.c_int
    return h


def _ab_prior(shapes, new_name, old_name, old_fn, eps, same_bits, seed, rounds=6, launches=60) -> None:
    """rmsnorm_fwd against a prior launch-table entry (old_fn(h, x, w, y, M,
    N, eps, stream) through libmbn_prior.so) on the same data: outputs
    compared (within one bf16 ulp; bit for bit where same_bits(N)), then, per
    round and in alternating order, the median of `launches` individually
    timed launches and the mean over about 0.2 s of back-to-back launches,
    over buffer sets rotated through >= 1 GiB. One JSON line per shape,
    kernel and timing."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    import memory_bound_normalization_amd as mbn

    h = prior_lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(seed)
    for M, N in shapes:
        n = max(2, -(-(1 << 30) // (M * N * 4)))
        xs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        ys = [torch.empty_like(xs[0]) for _ in range(n)]
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)

        def old(i):
            rc = old_fn(h, xs[i].data_ptr(), w.data_ptr(), ys[i].data_ptr(), M, N, eps, sp)
            if rc != 0:
                raise RuntimeError(f"{old_name}: status {rc}")

        fns = {new_name: lambda i: mbn.rmsnorm_fwd(xs[i], w, ys[i], eps=eps), old_name: old}
        outs = []
        for fn in fns.values():
            ys[0].zero_()
            fn(0)
            torch.cuda.synchronize()
            outs.append(ys[0].clone())
        a, b2 = outs[0].float(), outs[1].float()
        if not bool(((a - b2).abs() <= b2.abs() * 2.0 ** -7 + 1e-6).all()):
            raise RuntimeError(f"{M}x{N}: the two kernels' outputs differ by more than one bf16 ulp")
        same = float((outs[0].view(torch.int16) == outs[1].view(torch.int16)).float().mean())
        if same_bits(N) and same != 1.0:
            raise RuntimeError(f"{M}x{N}: the two kernels' outputs differ")
        del outs, a, b2
        nb = 2 * M * N * 2 + 2 * N
        sustained_n = max(200, int(0.2e6 / (nb / 6.4e6)))
        res = {(k, m): [] for k in fns for m in ("events", "sustained")}
        for _ in range(200):
            fns[new_name](0)
        torch.cuda.synchronize()
        for rnd in range(rounds):
            for k in (list(fns) if rnd % 2 == 0 else list(fns)[::-1]):
                fn = fns[k]
                for i in range(20):
                    fn(i % n)
                torch.cuda.synchronize()
                ev = [(timer.new(), timer.new()) for _ in range(launches)]
                for i, (a, b) in enumerate(ev):
                    timer.record(a)
                    fn(i % n)
                    timer.record(b)
                torch.cuda.synchronize()
                us = sorted(timer.elapsed_ms(a, b) * 1e3 for a, b in ev)
                timer.close()
                res[(k, "events")].append(us[len(us) // 2])
                e0, e1 = timer.new(), timer.new()
                timer.record(e0)
                for i in range(sustained_n):
                    fn(i % n)
                timer.record(e1)
                torch.cuda.synchronize()
                res[(k, "sustained")].append(timer.elapsed_ms(e0, e1) * 1e3 / sustained_n)
                timer.close()
        for (k, m), t in res.items():
            us = sorted(t)[len(t) // 2]
            print(json.dumps({"M": M, "N": N, "kernel": k, "timing": m, "buffer_sets": n, "median_us": round(us, 2),
                              "pct": round(100 * nb / us / 1e3 / 8000, 2), "rounds_us": [round(v, 2) for v in t]}),
                  flush=True)
        print(json.dumps({"check": f"{M}x{N}: outputs within one bf16 ulp, {100 * same:.4f}% bit-identical"}),
              flush=True)
        del xs, ys
        torch.cuda.empty_cache()


def staging() -> None:
    """rmsnorm_fwd, rows held in VGPRs at N = 32768 and 65536, against the
    staged-row kernel those widths used before. At 32768 both use 1024 lanes
    per row (same sums in the same order: same bits); at 65536 512 against
    1024 lanes, so the outputs agree to one ulp."""
    _ab_prior(STAGING_SHAPES, "registers (library)", "LDS (before)",
              lambda h, *args: h.mbn_lds_rmsnorm(*args), 1e-5, lambda N: N == 32768, 23)


LATE_W_SHAPES = [(M, N) for N in (8192, 7680, 6656) for M in (4096, 8192, 16384, 32768)]


def late_weights() -> None:
    """rmsnorm_fwd in the N <= 8192 band (512 lanes per row, weight loaded
    after the reduction) against the band's previous entry (256 lanes, weight
    loaded with the row copy); the lane mappings differ, so the outputs agree
    to one ulp."""
    _ab_prior(LATE_W_SHAPES, "late weight (library)", "early weight (before)",
              lambda h, *args: h.mbn_early_w_rmsnorm(*args), 1e-6, lambda N: False, 29)


WIDE_ROWS_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_wide.so")
# probe_csrc/wide_rows.hip, variant: (lanes per row, occupancy cap, XCD row run,
# when the weight is loaded); variant 1 is the launch table's entry.
WIDE_ROW_VARIANTS = {
    1: (1024, 4, 4, "with the row"),
    2: (1024, 4, 4, "after the reduction"),
    3: (1024, 4, 0, "after the reduction"),
    4: (1024, 4, 8, "after the reduction"),
    5: (512, 4, 4, "with the row"),
    6: (512, 2, 4, "with the row"),
    7: (512, 4, 4, "after the reduction"),
    8: (512, 3, 4, "after the reduction"),
    9: (512, 0, 4, "after the reduction"),
    10: (512, 4, 0, "after the reduction"),
    11: (256, 4, 4, "after the reduction"),
    12: (256, 8, 4, "after the reduction"),
}
WIDE_ROW_SHAPES = [(4096, 32768), (8192, 32768)]


def build_wide_rows(verbose: bool = False) -> str:
    """Compile probe_csrc/wide_rows.hip (register-row RMSNorm geometries at
    N = 32768, with the library's row-norm source) into
    probe_csrc/libmbn_wide.so; always rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=WIDE_ROWS_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "wide_rows.hip")])


def wide_rows_lib():
    if not os.path.exists(WIDE_ROWS_LIB_PATH):
        build_wide_rows()
    h = ctypes.CDLL(WIDE_ROWS_LIB_PATH)
    h.mbn_wide_rows_variant.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_float, ctypes.c_int] + [
        ctypes.c_void_p] * 3
    h.mbn_wide_rows_variant.restype = ctypes.c_int
    return h


def _timed_rounds(cases, nrot, timer, rounds, launches):
    """Median per round of `launches` launches of each case (f(i, start, stop)
    records the kernel's own start and end), rounds in alternating order.
    Destroys every event the timer holds (the caller's too) as it goes."""
    import statistics

    import torch

    spare = (timer.new(), timer.new())
    res = {k: [] for k, _ in cases}
    for rnd in range(rounds):
        for k, f in (cases if rnd % 2 == 0 else cases[::-1]):
            for i in range(4):
                f(i % nrot, *spare)
            ev = [(timer.new(), timer.new()) for _ in range(launches)]
            for i, (a, b) in enumerate(ev):
                f(i % nrot, a, b)
            torch.cuda.synchronize()
            res[k].append(statistics.median(timer.elapsed_ms(a, b) * 1e3 for a, b in ev))
            timer.close()
            spare = (timer.new(), timer.new())
    return res


def wide_rows(rounds: int = 6, launches: int = 40) -> None:
    """rmsnorm_fwd at N = 32768 (rows in VGPRs) against the register-row
    geometries of probe_csrc/wide_rows.hip on the same data (x ~ 0.5 N(0, 1),
    w ~ U(0.5, 1.5), eps 1e-5, buffer sets rotated through >= 1 GiB). Each
    variant's output is compared with the library's (same lanes per row: same
    bits; otherwise within one ulp); then per round, in alternating order, the
    median of `launches` launches timed by the kernels' own start and end.
    One JSON line per shape and case."""
    sys.path.insert(0, ROOT)
    import json
    import statistics

    import torch

    import memory_bound_normalization_amd as mbn

    h = wide_rows_lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(3)
    for M, N in WIDE_ROW_SHAPES:
        spare = (timer.new(), timer.new())  # _timed_rounds destroys the timer's events
        nrot = max(2, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [(torch.randn(M, N, device=dev, generator=g) * 0.5).to(torch.bfloat16) for _ in range(nrot)]
        ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        ref = mbn.rmsnorm_fwd(xs[0], w, eps=1e-5)

        def variant(v):
            def f(i, a, b):
                rc = h.mbn_wide_rows_variant(xs[i].data_ptr(), w.data_ptr(), ys[i].data_ptr(), M, 1e-5, v, sp, a, b)
                if rc != 0:
                    raise RuntimeError(f"wide-row variant {v}: status {rc}")
            return f

        def library(i, a, b):
            mbn.rmsnorm_fwd_timed(xs[i], w, a, b, y=ys[i], eps=1e-5)

        for v in WIDE_ROW_VARIANTS:
            variant(v)(0, *spare)
            torch.cuda.synchronize()
            d = (ys[0].view(torch.int16).int() - ref.view(torch.int16).int()).abs()
            print(json.dumps({"check": v, "M": M, "N": N, "bit_identical": float((d == 0).float().mean()),
                              "max_bits": int(d.max())}), flush=True)
            if int(d.max()) > 1:
                raise RuntimeError(f"wide-row variant {v}: outputs differ from the library's by more than one ulp")
        for i in range(2000 * 4096 // M):
            library(i % nrot, *spare)
        torch.cuda.synchronize()
        cases = [("library", library)] + [(v, variant(v)) for v in WIDE_ROW_VARIANTS]
        res = _timed_rounds(cases, nrot, timer, rounds, launches)
        nb = 2 * M * N * 2 + 2 * N
        for k, _ in cases:
            med = statistics.median(res[k])
            print(json.dumps({"kernel": k, "M": M, "N": N, "median_us": round(med, 2),
                              "pct": round(nb / med / 1e3 / 80, 2), "rounds": [round(r, 2) for r in res[k]]}),
                  flush=True)
        del xs, ys
        torch.cuda.empty_cache()


def wide_rows_summary(log: str) -> None:
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    print("rmsnorm_fwd at N = 32768 (rows in VGPRs) against register-row geometries, MI355X (gfx950), one GPU")
    print("=" * 98)
    print()
    print("Commands (from the repository root; probe.py builds probe_csrc/libmbn_wide.so from")
    print("probe_csrc/wide_rows.hip on first use):")
    print(f"  python -u probe.py wide-rows > {log}")
    print(f"  python probe.py wide-rows-summary {log}")
    print()
    print("Each variant holds the row in VGPRs as the library's rownorm_regs_kernel does (16-byte")
    print("non-temporal loads and stores, one cross-wave LDS step), with the lanes per row, the")
    print("occupancy cap (resident workgroups per CU, through the dynamic LDS request; 0 = none),")
    print("the XCD row run (0 = dispatch order) and the point where the weight is loaded chosen")
    print("per variant. Variant 1 is the launch table's entry. Same data (x ~ 0.5 N(0,1), buffer")
    print("sets rotated through >= 1 GiB), outputs checked against the library's; per round, in")
    print("alternating order, the median of 40 launches timed by the kernels' own start and end;")
    print("the median over 6 rounds; % of 8 TB/s on the algorithmic bytes.")
    for M, N in sorted({(r["M"], r["N"]) for r in rows if "kernel" in r}):
        print()
        lib = next(r for r in rows if r.get("kernel") == "library" and r["M"] == M)
        print(f"  x[{M}, {N}]")
        print(f"  {'case':<58} {'median_us':>9} {'%':>6} {'vs library':>10} {'same bits':>9}")
        print(f"  {'library rmsnorm_fwd':<58} {lib['median_us']:>9.2f} {lib['pct']:>6.2f} {1.0:>10.3f} {'':>9}")
        for r in rows:
            if r.get("kernel") in WIDE_ROW_VARIANTS and r["M"] == M:
                lanes, cap, run, wt = WIDE_ROW_VARIANTS[r["kernel"]]
                chk = next(c for c in rows if c.get("check") == r["kernel"] and c["M"] == M)
                desc = f"{r['kernel']}: {lanes} lanes, cap {cap}, XCD run {run}, weight {wt}"
                print(f"  {desc:<58} {r['median_us']:>9.2f} {r['pct']:>6.2f} {lib['median_us'] / r['median_us']:>10.3f} "
                      f"{100 * chk['bit_identical']:>8.4f}%")


SMALL_REGS_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_small_regs.so")
SMALL_REGS_WIDTHS = (2048, 4096, 8192, 16384)
SMALL_REGS_ROWS = (256, 384, 512, 768, 1024, 1536, 2048)


def build_small_regs(verbose: bool = False) -> str:
    """Compile probe_csrc/small_regs.hip into probe_csrc/libmbn_small_regs.so;
    always rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=SMALL_REGS_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "small_regs.hip")])


def small_regs_lib():
    if not os.path.exists(SMALL_REGS_LIB_PATH):
        build_small_regs()
    h = ctypes.CDLL(SMALL_REGS_LIB_PATH)
    vp = ctypes.c_void_p
    h.mbn_small_regs.argtypes = [ctypes.c_int] + [vp] * 6 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                                            ctypes.c_int] + [vp] * 3
    h.mbn_small_regs.restype = ctypes.c_int
    h.mbn_small_regs_geometry.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    h.mbn_small_regs_geometry.restype = ctypes.c_int
    return h


def small_regs_geometries(h):
    out = {}
    g = (ctypes.c_int * 3)()
    for v in range(h.mbn_small_regs_count()):
        if h.mbn_small_regs_geometry(v, g) != 0:
            raise RuntimeError("mbn_small_regs_geometry failed")
        out[v] = (g[0], g[1], g[2])
    return out


# op: (kernel mode, eps)
SMALL_REGS_OPS = {"rms": (0, 1e-6), "add": (1, 1e-6), "layer": (2, 1e-5), "l2": (3, 1e-12)}


def small_regs(ops: str = "rms", width: str = "", rows: str = "", rounds: int = 8, launches: int = 60) -> None:
    """Small row-norm launches (N = 2048 ... 16384, M = 256 ... 2048, or the
    one width `width` at the comma-separated row counts `rows`) through the
    library and through the register-row geometries of
    probe_csrc/small_regs.hip of the same width, on the same data, buffer sets
    rotated through >= 1 GiB, for each op of `ops` (comma-separated: rms, add,
    layer, l2). Meant to run under rocprofv3 --kernel-trace: every group of
    back-to-back launches is announced by a JSON line {"block": [op, N, M,
    case, launches]} in launch order, so that small-regs-summary can attribute
    the traced kernels. Outputs are compared with the library's first (within
    twice the one-ulp tolerance, the sums being taken in another order; the
    residual sum h bit for bit)."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    import memory_bound_normalization_amd as mbn

    h = small_regs_lib()
    geo = small_regs_geometries(h)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    L = mbn.lib()
    g = torch.Generator(device=dev).manual_seed(17)

    def block(op, N, M, case, n):
        print(json.dumps({"block": [op, N, M, case, n]}), flush=True)

    widths = (int(width),) if width else SMALL_REGS_WIDTHS
    row_counts = tuple(int(m) for m in rows.split(",")) if rows else SMALL_REGS_ROWS
    print(json.dumps({"small_regs": {"ops": ops, "width": width, "rows": rows, "rounds": rounds,
                                     "launches": launches}}), flush=True)
    for op in ops.split(","):
        mode, eps = SMALL_REGS_OPS[op]
        for N in widths:
            vs = [v for v, (wpr, _, maxc) in geo.items() if 64 * wpr * maxc * 8 == N]
            w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
            b = (torch.rand(N, device=dev, generator=g) - 0.5).to(torch.bfloat16)
            for M in row_counts:
                nrot = max(2, -(-(1 << 30) // ((4 if op == "add" else 2) * M * N * 2)))
                xs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(nrot)]
                rs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(nrot)] \
                    if op == "add" else [None] * nrot
                ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
                hs = [torch.empty_like(xs[0]) for _ in range(nrot)] if op == "add" else [None] * nrot

                def ptr(t):
                    return None if t is None else t.data_ptr()

                def run(case, i):
                    # both through ctypes straight to C, so that the host paces
                    # the library's launches and the variants' alike
                    if case == "library":
                        x_, y_ = xs[i].data_ptr(), ys[i].data_ptr()
                        if op == "rms":
                            st = L.rmsnorm_fwd(x_, w.data_ptr(), y_, M, N, eps, sp)
                        elif op == "add":
                            st = L.add_rmsnorm_fwd(x_, rs[i].data_ptr(), w.data_ptr(), hs[i].data_ptr(), y_, M, N,
                                                   eps, sp)
                        elif op == "layer":
                            st = L.layernorm_fwd(x_, w.data_ptr(), b.data_ptr(), y_, M, N, eps, sp)
                        else:
                            st = L.l2norm_fwd(x_, y_, M, N, eps, sp)
                        if st != 0:
                            raise RuntimeError(f"small-regs {op} library: {mbn.mbn_strerror(st)}")
                    elif h.mbn_small_regs(mode, xs[i].data_ptr(), ptr(rs[i]), None if op == "l2" else w.data_ptr(),
                                          b.data_ptr() if op == "layer" else None, ptr(hs[i]), ys[i].data_ptr(),
                                          M, N, eps, case, sp, None, None) != 0:
                        raise RuntimeError(f"small-regs {op} variant {case}: launch failed")

                block(op, N, M, "library", 1)
                run("library", 0)
                torch.cuda.synchronize()
                ref_y = ys[0].clone()
                ref_h = hs[0].clone() if op == "add" else None
                for v in vs:
                    block(op, N, M, v, 1)
                    run(v, 0)
                    torch.cuda.synchronize()
                    # each within one bf16 ulp + 1e-6 of the exact result, so
                    # within twice that of each other (LayerNorm outputs near
                    # zero may differ in more than their last bit)
                    a_, b_ = ys[0].float(), ref_y.float()
                    bad = not bool(((a_ - b_).abs() <= 2.0 ** -6 * b_.abs() + 2e-6).all())
                    if op == "add":
                        bad = bad or not torch.equal(hs[0].view(torch.int16), ref_h.view(torch.int16))
                    if bad:
                        raise RuntimeError(f"small-regs {op} variant {v}: outputs differ from the library's")
                cases = ["library"] + vs
                for rnd in range(rounds):
                    for case in (cases if rnd % 2 == 0 else cases[::-1]):
                        block(op, N, M, case, launches)
                        for i in range(launches):
                            run(case, (i * 7) % nrot)
                        torch.cuda.synchronize()
                del xs, rs, ys, hs
                torch.cuda.empty_cache()


def small_regs_summary(trace_dir: str, log: str) -> None:
    """Per width and row count, the median kernel duration of the library and
    of each register-row geometry, from the kernel trace (trace_dir) of
    `python -u probe.py small-regs > log`."""
    import json
    import statistics

    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ks = [r for r in rows if "rownorm" in r["Kernel_Name"]]
    blocks = [json.loads(x)["block"] for x in open(log) if x.startswith('{"block"')]
    blocks = [b if len(b) == 5 else ["rms"] + b for b in blocks]  # logs without the op are RMSNorm
    if sum(b[4] for b in blocks) != len(ks):
        raise SystemExit(f"{len(ks)} traced row-norm dispatches, {sum(b[4] for b in blocks)} announced")
    dur = {}
    kname = {}
    i = 0
    for op, N, M, case, n in blocks:
        grp = ks[i:i + n]
        i += n
        if n > 1:  # timed groups (single launches are the output checks)
            dur.setdefault((op, N, M, case), []).extend(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
            kname[(op, N, M, case)] = _short_kernel(grp[0]["Kernel_Name"])
    ops = [o for o in SMALL_REGS_OPS if any(b[0] == o for b in blocks)]
    args = [json.loads(x)["small_regs"] for x in open(log) if x.startswith('{"small_regs"')]
    args = args[0] if args else {"width": "", "rows": "", "rounds": 8, "launches": 60}
    arg = "" if ops == ["rms"] and not args["width"] else " " + ",".join(ops)
    if args["width"]:
        arg += f" {args['width']} {args['rows']}"
    print("Small row-norm launches: the library against register-row geometries, MI355X (gfx950), one GPU")
    print("=" * 96)
    print()
    print("Commands (from the repository root, TMPDIR=/tmp; probe.py builds probe_csrc/libmbn_small_regs.so")
    print("from probe_csrc/small_regs.hip on first use):")
    print(f"  rocprofv3 --kernel-trace --output-format csv -d {trace_dir} -o run -- \\")
    print(f"      python -u probe.py small-regs{arg} > {log}")
    print(f"  python probe.py small-regs-summary {trace_dir} {log}")
    print()
    print(f"Kernel durations from the trace: median over {args['rounds']} rounds x {args['launches']} "
          "launches per case (rounds in")
    print("alternating order, buffer sets rotated through >= 1 GiB); every variant's output within")
    print("twice the one-ulp tolerance of the library's (the residual sum h bit for bit).")
    print("rownorm_regs_kernel<mode, W, R, C, true>: 64 * W lanes per row, R rows per workgroup,")
    print("C chunks of 16 bytes per lane, rows held in VGPRs (mode 0 RMSNorm, 1 residual add +")
    print("RMSNorm, 2 LayerNorm, 3 L2Norm).")
    names = {"rms": "RMSNorm", "add": "residual add + RMSNorm", "layer": "LayerNorm", "l2": "L2Norm"}
    for op in [o for o in SMALL_REGS_OPS if any(k[0] == o for k in dur)]:
        for N in sorted({k[1] for k in dur if k[0] == op}):
            for M in sorted({k[2] for k in dur if k[:2] == (op, N)}):
                lib = statistics.median(dur[(op, N, M, "library")])
                print()
                print(f"  {names[op]} x[{M}, {N}]: library {kname[(op, N, M, 'library')]}: {lib:.2f} us")
                cases = sorted((statistics.median(v), c) for (o_, n_, m_, c), v in dur.items()
                               if (o_, n_, m_) == (op, N, M) and c != "library")
                for med, c in cases:
                    print(f"    {kname[(op, N, M, c)][:52]:<52} {med:7.2f} us  {lib / med:6.3f} x library")


def _small_regs_table(path: str) -> dict:
    """{(op name, N, M): (library us, library kernel, {variant kernel: us})}
    from a small-regs-summary text."""
    out, cur = {}, None
    for line in open(path):
        m = re.match(r"\s+(?:(\S.*?) )?x\[(\d+), (\d+)\]: library (.*): ([\d.]+) us", line)
        if m:  # summaries of RMSNorm-only runs name no op
            cur = (m.group(1) or "RMSNorm", int(m.group(3)), int(m.group(2)))
            out[cur] = (float(m.group(5)), m.group(4), {})
            continue
        m = re.match(r"\s+(rownorm_regs_kernel<[^>]*>)\s+([\d.]+) us", line)
        if m and cur:
            out[cur][2][m.group(1)] = float(m.group(2))
    return out


def small_regs_compare(before: str, after: str) -> None:
    """Per op, width and row count: the library's kernel time in two
    small-regs-summary texts (before and after a change of the launch tables)
    and the best register-row geometry of the second."""
    import math

    b, a = _small_regs_table(before), _small_regs_table(after)
    print(f"  {'op':<24} {'N':>6} {'M':>5}  {'before_us':>9} {'after_us':>8} {'speedup':>7}  "
          f"{'best_variant_us':>15}  after: kernel")
    ratios = []
    for k in sorted(a, key=lambda k: (k[0], k[1], k[2])):
        if k not in b:
            continue
        t0, t1 = b[k][0], a[k][0]
        best = min(a[k][2].values()) if a[k][2] else float("nan")
        ratios.append(t0 / t1)
        print(f"  {k[0]:<24} {k[1]:>6} {k[2]:>5}  {t0:>9.2f} {t1:>8.2f} {t0 / t1:>7.3f}  {best:>15.2f}  "
              f"{a[k][1][:48]}")
    if ratios:
        print(f"  geometric mean speedup over {len(ratios)} launches: "
              f"{math.exp(sum(map(math.log, ratios)) / len(ratios)):.3f}")


QK_ANGLE_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_qk_angle.so")
QK_ANGLE_MODES = {0: "library path: wave 0 forms the angles, LDS table, barrier",
                  1: "every wave forms the angles, ds_bpermute, no barrier",
                  3: "as 1, rotation products in fp32"}


def build_qk_angle(verbose: bool = False) -> str:
    """Compile probe_csrc/qk_angle_paths.hip into probe_csrc/libmbn_qk_angle.so;
    always rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=QK_ANGLE_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "qk_angle_paths.hip")])


def qk_angles(rounds: int = 8, launches: int = 100) -> None:
    """qk_norm_rope_fwd on 256 tokens (32 q + 8 k heads, full rotary, theta
    1e6) beside the angle-path variants of probe_csrc/qk_angle_paths.hip, in
    rounds of `launches` back-to-back launches per case (alternating order),
    qkv buffers rotated through >= 1 GiB. Meant to run under rocprofv3
    --kernel-trace (qk-angles-summary reads the durations by kernel name).
    Modes 0, 1 and 3 are checked against the library first (mode 3 to one
    ulp, the others bit for bit)."""
    sys.path.insert(0, ROOT)
    import torch

    import memory_bound_normalization_amd as mbn

    if not os.path.exists(QK_ANGLE_LIB_PATH):
        build_qk_angle()
    h = ctypes.CDLL(QK_ANGLE_LIB_PATH)
    vp = ctypes.c_void_p
    h.mbn_qk_angle_path.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    vp, vp]
    h.mbn_qk_angle_path.restype = ctypes.c_int
    T, hq, hk = 256, 32, 8
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(5)
    width = (hq + 2 * hk) * 128
    n = max(2, -(-(1 << 30) // (T * width * 2)))
    qkv = [torch.randn(T, width, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
    qw = (torch.rand(128, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    kw = (torch.rand(128, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    pos = torch.arange(T, device=dev, dtype=torch.int64)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    ev = (timer.new(), timer.new())

    def library(i):
        mbn.qk_norm_rope_fwd(qkv[i], qw, kw, pos, hq, hk, eps=1e-6, theta=1e6)

    def mode(m):
        def f(i):
            if h.mbn_qk_angle_path(qkv[i].data_ptr(), qw.data_ptr(), kw.data_ptr(), pos.data_ptr(), T, hq, hk, m,
                                   sp, *ev) != 0:
                raise RuntimeError(f"qk angle path {m}: launch failed")
        return f

    src = qkv[0].clone()
    qkv[0].copy_(src)
    library(0)
    torch.cuda.synchronize()
    ref = qkv[0].clone()
    for m in (0, 1, 3):
        qkv[0].copy_(src)
        mode(m)(0)
        torch.cuda.synchronize()
        d = (qkv[0].view(torch.int16).int() - ref.view(torch.int16).int()).abs()
        if int(d.max()) > (1 if m == 3 else 0):
            raise RuntimeError(f"qk angle path {m}: outputs differ from the library's")
    qkv[0].copy_(src)
    cases = [library] + [mode(m) for m in QK_ANGLE_MODES]
    for i in range(500):
        library(i % n)
    torch.cuda.synchronize()
    for rnd in range(rounds):
        for f in (cases if rnd % 2 == 0 else cases[::-1]):
            for i in range(launches):
                f((i * 7) % n)
            torch.cuda.synchronize()
    timer.close()


def qk_angles_summary(trace_dir: str) -> None:
    import statistics

    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    lib, modes = [], {m: [] for m in QK_ANGLE_MODES}
    for r in rows:
        n, d = r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        m = re.search(r"qkx_kernel<[^,]+, (\d)>", n)
        if m:
            modes[int(m.group(1))].append(d)
        elif "qk_norm_rope_kernel" in n:
            lib.append(d)
    lib = lib[-800:]  # the timed rounds (the warm-up launches come first)
    print("qk_norm_rope_fwd on 256 tokens: what the angle work adds, MI355X (gfx950), one GPU")
    print("==================================================================================")
    print()
    print("Commands (from the repository root, TMPDIR=/tmp; probe.py builds probe_csrc/libmbn_qk_angle.so")
    print("from probe_csrc/qk_angle_paths.hip on first use):")
    print(f"  rocprofv3 --kernel-trace --output-format csv -d {trace_dir} -o run -- python -u probe.py qk-angles")
    print(f"  python probe.py qk-angles-summary {trace_dir}")
    print()
    print("qkv[256, 48 * 128] bf16 (32 q + 8 k heads of 128), full rotary, theta 1e6, positions 0..255,")
    print("buffers rotated through >= 1 GiB; 8 rounds x 100 back-to-back launches per case in")
    print("alternating order; kernel durations from the trace (median, 10th percentile). The")
    print("variants are the library's kernel body for one head row per wave with the angle work")
    print("done another way; modes 0 and 1 give the library's bits, mode 3 within one ulp.")
    print()
    print(f"  {'case':<64} {'median_us':>9} {'p10_us':>7}")

    def line(name, d):
        print(f"  {name:<64} {statistics.median(d):>9.2f} {sorted(d)[len(d) // 10]:>7.2f}")

    line("library qk_norm_rope_fwd", lib)
    for m, d in modes.items():
        line(f"{m}: {QK_ANGLE_MODES[m]}", d)


LAUNCH_MODE_SHAPES = [(2560, 4096), (768, 16384), (4096, 4096), (16384, 16384)]
LAUNCH_MODES = {"plain": "rmsnorm_fwd",
                "ev_nofence": "rmsnorm_fwd_timed, events created with hipEventDisableSystemFence",
                "ev_default": "rmsnorm_fwd_timed, events created with default flags"}


def launch_modes(rounds: int = 6, launches: int = 40) -> None:
    """rmsnorm_fwd launched plainly and through rmsnorm_fwd_timed (two kinds of
    events), in rounds of back-to-back launches per mode (alternating order),
    for each shape of LAUNCH_MODE_SHAPES (10 launches per round at 16384 x
    16384), buffer sets rotated through >= 1 GiB, all through ctypes. Prints a
    JSON line {"block": [M, N, mode, launches]} before each group, so that
    launch-modes-summary can attribute a kernel trace, and per shape the
    median over rounds of (region events around the group) / launches."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    import memory_bound_normalization_amd as mbn

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    L = mbn.lib()
    timer = HipTimingEvents(stream)
    hip = timer.hip
    g = torch.Generator(device=dev).manual_seed(3)
    for M, N in LAUNCH_MODE_SHAPES:
        nrot = max(2, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(nrot)]
        ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        n = launches if M * N < (1 << 26) else 10
        nofence = [timer.new() for _ in range(2 * n)]
        default = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), 0) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            default.append(e)
        r0, r1 = timer.new(), timer.new()
        res = {}
        modes = list(LAUNCH_MODES)
        for rnd in range(rounds):
            for mode in (modes if rnd % 2 == 0 else modes[::-1]):
                print(json.dumps({"block": [M, N, mode, n]}), flush=True)
                timer.record(r0)
                for i in range(n):
                    j = (i * 7) % nrot
                    if mode == "plain":
                        st = L.rmsnorm_fwd(xs[j].data_ptr(), w.data_ptr(), ys[j].data_ptr(), M, N, 1e-6, sp)
                    else:
                        ev = nofence if mode == "ev_nofence" else default
                        st = L.rmsnorm_fwd_timed(xs[j].data_ptr(), w.data_ptr(), ys[j].data_ptr(), M, N, 1e-6, sp,
                                                 ev[2 * i], ev[2 * i + 1])
                    if st != 0:
                        raise RuntimeError(f"launch-modes {mode}: {mbn.mbn_strerror(st)}")
                timer.record(r1)
                torch.cuda.synchronize()
                res.setdefault(mode, []).append(timer.elapsed_ms(r0, r1) * 1e3 / n)
        print(json.dumps({"region": [M, N, {k: sorted(v)[len(v) // 2] for k, v in res.items()}]}), flush=True)
        for e in default:
            hip.hipEventDestroy(e)
        del xs, ys
        torch.cuda.empty_cache()
    timer.close()


def launch_modes_summary(trace_dir: str, log: str, plain_log: str) -> None:
    """Per shape and launch mode: the median kernel duration and the median
    idle time between consecutive kernels of a group from the kernel trace
    (trace_dir) of `python -u probe.py launch-modes > log`, the region time
    per launch of that run, and of a run without the profiler (plain_log)."""
    import json
    import statistics

    rows = sorted(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))),
                  key=lambda r: int(r["Start_Timestamp"]))
    ks = [r for r in rows if "rownorm" in r["Kernel_Name"]]
    recs = [json.loads(x) for x in open(log) if x.startswith("{")]
    blocks = [r["block"] for r in recs if "block" in r]
    if sum(b[3] for b in blocks) != len(ks):
        raise SystemExit(f"{len(ks)} traced row-norm dispatches, {sum(b[3] for b in blocks)} announced")
    dur, gap, i = {}, {}, 0
    for M, N, mode, n in blocks:
        grp = ks[i:i + n]
        i += n
        dur.setdefault((M, N, mode), []).extend(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
        gap.setdefault((M, N, mode), []).extend(
            (int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3 for a, b in zip(grp, grp[1:]))
    region = {tuple(r["region"][:2]): r["region"][2] for r in recs if "region" in r}
    plain = {tuple(r["region"][:2]): r["region"][2]
             for r in (json.loads(x) for x in open(plain_log) if x.startswith('{"region"'))}
    print("rmsnorm_fwd: what the timed entry point costs between launches, MI355X (gfx950), one GPU")
    print("=========================================================================================")
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print(f"  rocprofv3 --kernel-trace --output-format csv -d {trace_dir} -o run -- \\")
    print(f"      python -u probe.py launch-modes > {log}")
    print(f"  python -u probe.py launch-modes > {plain_log}")
    print(f"  python probe.py launch-modes-summary {trace_dir} {log} {plain_log}")
    print()
    print("Back-to-back launches of one mode per group (6 rounds, alternating order; 40 launches")
    print("per group, 10 at 16384 x 16384), buffer sets rotated through >= 1 GiB, all through ctypes:")
    for k, v in LAUNCH_MODES.items():
        print(f"  {k:<11} {v}")
    print("kernel: median trace duration; gap: median idle time between consecutive kernels of a")
    print("group (trace); region / launch: events around each group / launches (median over rounds),")
    print("under the profiler and in the run without it.")
    print()
    print(f"  {'x[M, N]':<16} {'mode':<11} {'kernel_us':>9} {'gap_us':>7} {'region/launch_us':>16} "
          f"{'without_profiler_us':>19}")
    for (M, N), reg in region.items():
        for mode in LAUNCH_MODES:
            k = (M, N, mode)
            print(f"  {f'x[{M}, {N}]':<16} {mode:<11} {statistics.median(dur[k]):>9.2f} "
                  f"{statistics.median(gap[k]):>7.2f} {reg[mode]:>16.2f} "
                  f"{plain.get((M, N), {}).get(mode, float('nan')):>19.2f}")


# Cache-policy bits of the row copy's LDS-DMA loads (global_load_lds_dwordx4):
# aux operand of __builtin_amdgcn_global_load_lds on gfx950 (sc0 1, nt 2, sc1 16).
LOAD_POLICIES = {0: "none", 16: "sc1", 18: "nt sc1", 17: "sc0 sc1", 3: "nt sc0"}
LOAD_POLICY_SHAPES = [(16384, 16384), (8192, 8192)]


def lp_lib_path(pol: int) -> str:
    return os.path.join(PROBE_CSRC, f"libmbn_lp{pol}.so")


def build_load_policy(verbose: bool = False) -> None:
    """Compile the whole library once per load policy into
    probe_csrc/libmbn_lp<policy>.so, from a copy of its sources in
    probe_csrc/gen/lp<policy>/ whose device.h gives the LDS-DMA loads that
    policy (the library's is nt); always rebuilds."""
    sys.path.insert(0, ROOT)
    import shutil
    from concurrent.futures import ThreadPoolExecutor

    from memory_bound_normalization_amd.build import build

    csrc = os.path.join(ROOT, "memory_bound_normalization_amd", "csrc")
    gen = os.path.join(PROBE_CSRC, "gen")
    os.makedirs(os.path.join(gen, "include"), exist_ok=True)  # csrc/abi.hip includes ../../include/mbn.h
    shutil.copyfile(os.path.join(ROOT, "include", "mbn.h"), os.path.join(gen, "include", "mbn.h"))
    line = "constexpr int kCachePolicyNT = 2;"
    srcs = {}
    for pol in LOAD_POLICIES:
        d = os.path.join(gen, f"lp{pol}", "csrc")
        if os.path.exists(d):
            shutil.rmtree(d)
        shutil.copytree(csrc, d)
        text = open(os.path.join(d, "device.h")).read()
        if text.count(line) != 1:
            raise RuntimeError("device.h: the load policy constant is not where the probe expects it")
        with open(os.path.join(d, "device.h"), "w") as f:
            f.write(text.replace(line, f"constexpr int kCachePolicyNT = {pol};"))
        srcs[pol] = sorted(os.path.join(d, n) for n in os.listdir(d) if n.endswith(".hip"))
    with ThreadPoolExecutor(len(LOAD_POLICIES)) as ex:
        list(ex.map(lambda p: build(verbose=verbose, out=lp_lib_path(p), sources_=srcs[p]), LOAD_POLICIES))


def load_policy(rounds: int = 6, launches: int = 40) -> None:
    """rmsnorm_fwd against the same library built with other cache policies on
    its LDS-DMA row loads (libmbn_lp<policy>.so), at 16384 x 16384 and
    8192 x 8192: outputs compared bit for bit, then per round, in alternating
    order, the median of `launches` launches timed by the kernels' own start
    and end (rmsnorm_fwd_timed of each library), buffer sets rotated through
    >= 1 GiB. One JSON line per shape and case."""
    sys.path.insert(0, ROOT)
    import json
    import statistics

    import torch

    import memory_bound_normalization_amd as mbn

    if not all(os.path.exists(lp_lib_path(p)) for p in LOAD_POLICIES):
        build_load_policy()
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    libs = {"nt (library)": mbn.lib()}
    for p in LOAD_POLICIES:
        h = ctypes.CDLL(lp_lib_path(p))
        h.rmsnorm_fwd_timed.argtypes = [vp, vp, vp, i64, i64, f32, vp, vp, vp]
        h.rmsnorm_fwd_timed.restype = ctypes.c_int
        libs[LOAD_POLICIES[p]] = h
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(4)
    for M, N in LOAD_POLICY_SHAPES:
        spare = (timer.new(), timer.new())  # _timed_rounds destroys the timer's events
        nrot = max(2, -(-(1 << 30) // (2 * M * N * 2)))
        xs = [torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16) for _ in range(nrot)]
        ys = [torch.empty_like(xs[0]) for _ in range(nrot)]
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        ref = mbn.rmsnorm_fwd(xs[0], w, eps=1e-6)

        def mk(h):
            def f(i, a, b):
                rc = h.rmsnorm_fwd_timed(xs[i].data_ptr(), w.data_ptr(), ys[i].data_ptr(), M, N, 1e-6, sp, a, b)
                if rc != 0:
                    raise RuntimeError(f"rmsnorm_fwd_timed: status {rc}")
            return f

        cases = [(k, mk(h)) for k, h in libs.items()]
        for k, f in cases[1:]:
            f(0, *spare)
            torch.cuda.synchronize()
            if not torch.equal(ys[0].view(torch.int16), ref.view(torch.int16)):
                raise RuntimeError(f"load policy {k}: outputs differ from the library's")
        for i in range(2000 * (16384 * 16384) // (M * N)):
            cases[0][1](i % nrot, *spare)
        torch.cuda.synchronize()
        res = _timed_rounds(cases, nrot, timer, rounds, launches)
        nb = 2 * M * N * 2 + 2 * N
        for k, _ in cases:
            med = statistics.median(res[k])
            print(json.dumps({"policy": k, "M": M, "N": N, "median_us": round(med, 2),
                              "pct": round(nb / med / 1e3 / 80, 2), "rounds": [round(r, 2) for r in res[k]]}),
                  flush=True)
        del xs, ys
        torch.cuda.empty_cache()


def load_policy_summary(log: str) -> None:
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    print("rmsnorm_fwd with other cache policies on its LDS-DMA row loads, MI355X (gfx950), one GPU")
    print("=" * 88)
    print()
    print("Commands (from the repository root; probe.py builds probe_csrc/libmbn_lp<policy>.so from")
    print("copies of the library's sources in probe_csrc/gen/ on first use):")
    print(f"  python -u probe.py load-policy > {log}")
    print(f"  python probe.py load-policy-summary {log}")
    print()
    print("The whole library is rebuilt with another cache policy on global_load_lds_dwordx4 (the")
    print("row copy HBM -> LDS); everything else is unchanged. Outputs are bit-identical to the")
    print("library's. Per round, in alternating order, the median of 40 launches timed by the")
    print("kernels' own start and end; the median over 6 rounds; buffer sets rotated through")
    print(">= 1 GiB; % of 8 TB/s on the algorithmic bytes.")
    for M, N in sorted({(r["M"], r["N"]) for r in rows}, reverse=True):
        print()
        lib = next(r for r in rows if r["policy"] == "nt (library)" and r["M"] == M)
        print(f"  x[{M}, {N}]")
        print(f"  {'load policy':<16} {'median_us':>9} {'%':>6} {'vs library':>10}")
        for r in rows:
            if r["M"] == M:
                print(f"  {r['policy']:<16} {r['median_us']:>9.2f} {r['pct']:>6.2f} "
                      f"{lib['median_us'] / r['median_us']:>10.3f}")


PRIOR_ANY_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_prior_any.so")


def build_prior_any(verbose: bool = False) -> str:
    """Compile probe_csrc/prior_any_width.hip (the any-width launch path
    before the staged kernels' weight windows became unconditional loads and
    their tables were re-swept) into probe_csrc/libmbn_prior_any.so; always
    rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=PRIOR_ANY_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "prior_any_width.hip")])


def prior_any_lib():
    if not os.path.exists(PRIOR_ANY_LIB_PATH):
        build_prior_any()
    h = ctypes.CDLL(PRIOR_ANY_LIB_PATH)
    h.mbn_prior_any_rownorm.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6 + [
        ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
    h.mbn_prior_any_rownorm.restype = ctypes.c_int
    return h


# (N, element offset of every row tensor): widths that take the 16-byte staged
# kernels (N % 8 != 0 from 1024 on; below, pointers that are not 8-byte
# aligned), one per band of the tables and a view of an aligned width.
ANY_AB_SHAPES = [(300, 1), (511, 1), (777, 3), (1023, 1), (1523, 0), (2047, 0), (3059, 0), (4095, 0), (8191, 0),
                 (16383, 0), (16384, 1), (24563, 0), (32767, 0), (65521, 0)]
ANY_AB_OPS = ("rms", "add", "layer", "l2")


def any_width_ab(rounds: int = 6, launches: int = 40) -> None:
    """The any-width row norms of the library against the prior any-width
    path (libmbn_prior_any.so) on the same data, per width and op: outputs
    compared (one bf16 ulp, or 2^-14 absolute), then per round, in
    alternating order, the median of `launches` individually timed launches
    over buffer sets rotated through >= 1 GiB (about 256 MiB of rows each).
    One JSON line per width, op and kernel."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    import memory_bound_normalization_amd as mbn

    h = prior_any_lib()
    lib = mbn.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(37)
    mode = {"rms": 0, "add": 1, "layer": 2, "l2": 3}
    for N, off in ANY_AB_SHAPES:
        M = max(1, (1 << 27) // N)
        n = max(2, -(-(1 << 30) // (M * N * 2)))
        size = M * N + off + 8
        xs = [torch.randn(size, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        rs = [torch.randn(size, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        hs = [torch.empty_like(xs[0]) for _ in range(n)]
        ys = [torch.empty_like(xs[0]) for _ in range(n)]
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        b = (torch.rand(N, device=dev, generator=g) - 0.5).to(torch.bfloat16)

        def ptr(t, i):
            return t[i].data_ptr() + 2 * off

        for op in ANY_AB_OPS:
            def new(i, op=op):
                x, y = ptr(xs, i), ptr(ys, i)
                if op == "rms":
                    rc = lib.rmsnorm_fwd(x, w.data_ptr(), y, M, N, 1e-6, sp)
                elif op == "add":
                    rc = lib.add_rmsnorm_fwd(x, ptr(rs, i), w.data_ptr(), ptr(hs, i), y, M, N, 1e-6, sp)
                elif op == "layer":
                    rc = lib.layernorm_fwd(x, w.data_ptr(), b.data_ptr(), y, M, N, 1e-6, sp)
                else:
                    rc = lib.l2norm_fwd(x, y, M, N, 1e-6, sp)
                if rc != 0:
                    raise RuntimeError(f"{op} N={N}: status {rc}")

            def old(i, op=op):
                rc = h.mbn_prior_any_rownorm(mode[op], 0, ptr(xs, i), ptr(rs, i), w.data_ptr(), b.data_ptr(),
                                             ptr(hs, i), ptr(ys, i), M, N, 1e-6, sp)
                if rc != 0:
                    raise RuntimeError(f"prior {op} N={N}: status {rc}")

            fns = {"library": new, "before": old}
            outs = []
            for fn in fns.values():
                ys[0].zero_()
                fn(0)
                torch.cuda.synchronize()
                outs.append(ys[0][off:off + M * N].float().clone())
            a, b2 = outs
            if not bool(((a - b2).abs() <= b2.abs() * 2.0 ** -7 + 2.0 ** -14).all()):
                raise RuntimeError(f"{op} N={N}: the two paths' outputs differ by more than one bf16 ulp")
            del outs, a, b2
            nb = (4 if op == "add" else 2) * M * N * 2
            res = {k: [] for k in fns}
            for fn in fns.values():
                for i in range(20):
                    fn(i % n)
            torch.cuda.synchronize()
            for rnd in range(rounds):
                for k in (list(fns) if rnd % 2 == 0 else list(fns)[::-1]):
                    ev = [(timer.new(), timer.new()) for _ in range(launches)]
                    for i, (e0, e1) in enumerate(ev):
                        timer.record(e0)
                        fns[k](i % n)
                        timer.record(e1)
                    torch.cuda.synchronize()
                    us = sorted(timer.elapsed_ms(e0, e1) * 1e3 for e0, e1 in ev)
                    timer.close()
                    res[k].append(us[len(us) // 2])
            for k, t in res.items():
                us = sorted(t)[len(t) // 2]
                print(json.dumps({"N": N, "M": M, "offset": off, "op": op, "kernel": k, "median_us": round(us, 2),
                                  "pct": round(100 * nb / us / 1e3 / 8000, 2), "rounds_us": [round(v, 2) for v in t]}),
                      flush=True)
        del xs, rs, hs, ys
        torch.cuda.empty_cache()


def any_width_summary(log: str) -> None:
    """Table of an any-width-ab log: library against the prior path per width
    and op, with the ratio before / library."""
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    by = {}
    for r in rows:
        by.setdefault((r["N"], r["offset"], r["M"], r["op"]), {})[r["kernel"]] = r
    print("Any-width row norms: library against the prior any-width path, same data, per-launch median")
    print("of 40 launches, median over rounds; % of 8 TB/s on the algorithmic bytes:")
    print(f"  {'N':>6} {'off':>3} {'M':>6} {'op':<6} {'library us':>10} {'%':>6} {'before us':>9} {'%':>6} {'speedup':>7}")
    for (N, off, M, op), d in by.items():
        new, old = d["library"], d["before"]
        print(f"  {N:>6} {off:>3} {M:>6} {op:<6} {new['median_us']:>10.2f} {new['pct']:>6.1f} "
              f"{old['median_us']:>9.2f} {old['pct']:>6.1f} {old['median_us'] / new['median_us']:>7.3f}")


def ab_summary(log: str) -> None:
    """Table of a staging / late-weights log: the library against the prior
    entry, per shape and timing."""
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    kinds = []
    for r in rows:
        if "kernel" in r and r["kernel"] not in kinds:
            kinds.append(r["kernel"])
    new, old = kinds
    print(f"{new} against {old}, same data; median over rounds (events: per-launch median of 60;")
    print("sustained: mean per launch over ~0.2 s of back-to-back launches):")
    print(f"  {'shape':<14} {'timing':<10} {'library us':>10} {'%':>6} {'before us':>9} {'%':>6} {'ratio':>6}")
    by = {}
    for r in rows:
        if "check" in r:
            continue
        by.setdefault((r["M"], r["N"], r["timing"]), {})[r["kernel"]] = r
    for (M, N, m), d in by.items():
        a, b = d[new], d[old]
        print(f"  {str(M) + 'x' + str(N):<14} {m:<10} {a['median_us']:>10.2f} {a['pct']:>6.2f} {b['median_us']:>9.2f} "
              f"{b['pct']:>6.2f} {a['median_us'] / b['median_us']:>6.3f}")
    for r in rows:
        if "check" in r:
            print("  " + r["check"])


QK_PATTERN_TOKENS = (65536, 4096)


def qk_pattern(rounds: int = 6, launches: int = 40) -> None:
    """qk_norm_rope_fwd (32 q + 8 k + 8 v heads of 128) against its memory
    access pattern with no arithmetic (stream_qk_pattern: the q and k bytes of
    each token read and written back in place, every load before the first
    store), per token count: per-launch event medians, rounds interleaved."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    import memory_bound_normalization_amd as mbn

    sl = stream_lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(67)
    hq, hkv, d = 32, 8, 128
    for T in QK_PATTERN_TOKENS:
        row = (hq + 2 * hkv) * d
        n = max(2, -(-(1 << 30) // (T * row * 2)))
        qkv = [torch.randn(T, row, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        qw = (torch.rand(d, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        kw = (torch.rand(d, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        pos = torch.arange(T, device=dev, dtype=torch.int64)

        def bare(i):
            rc = sl.mbn_stream_qk_pattern(qkv[i].data_ptr(), T, row // 8, (hq + hkv) * d // 8, sp)
            if rc != 0:
                raise RuntimeError(f"qk pattern: status {rc}")

        fns = {"qk_norm_rope_fwd": lambda i: mbn.qk_norm_rope_fwd(qkv[i], qw, kw, pos, hq, hkv, d, eps=1e-6,
                                                                  theta=1e6),
               "access pattern only": bare}
        nb = 2 * T * (hq + hkv) * d * 2
        res = {k: [] for k in fns}
        # the GPU's first sustained load of the process runs slower for a while
        for fn in fns.values():
            for i in range(40):
                fn(i % n)
        torch.cuda.synchronize()
        for rnd in range(rounds):
            for k in (list(fns) if rnd % 2 == 0 else list(fns)[::-1]):
                fn = fns[k]
                for i in range(10):
                    fn(i % n)
                torch.cuda.synchronize()
                ev = [(timer.new(), timer.new()) for _ in range(launches)]
                for i, (a, b) in enumerate(ev):
                    timer.record(a)
                    fn(i % n)
                    timer.record(b)
                torch.cuda.synchronize()
                us = sorted(timer.elapsed_ms(a, b) * 1e3 for a, b in ev)
                timer.close()
                res[k].append(us[len(us) // 2])
        for k, t in res.items():
            us = sorted(t)[len(t) // 2]
            print(json.dumps({"T": T, "kernel": k, "median_us": round(us, 2), "pct": round(100 * nb / us / 1e3 / 8000, 2),
                              "rounds_us": [round(v, 2) for v in t]}), flush=True)
        del qkv
        torch.cuda.empty_cache()


PRIOR_QK_LIB_PATH = os.path.join(PROBE_CSRC, "libmbn_prior_qk.so")


def build_prior_qk(verbose: bool = False) -> str:
    """Compile probe_csrc/prior_qk_norm_rope.hip (the QK kernel before each
    wave kept all of its head rows in flight) into
    probe_csrc/libmbn_prior_qk.so; always rebuilds."""
    sys.path.insert(0, ROOT)
    from memory_bound_normalization_amd.build import build

    return build(verbose=verbose, out=PRIOR_QK_LIB_PATH, sources_=[os.path.join(PROBE_CSRC, "prior_qk_norm_rope.hip")])


def prior_qk_lib():
    if not os.path.exists(PRIOR_QK_LIB_PATH):
        build_prior_qk()
    h = ctypes.CDLL(PRIOR_QK_LIB_PATH)
    h.mbn_prior_qk_norm_rope.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                                 ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    h.mbn_prior_qk_norm_rope.restype = ctypes.c_int
    return h


# (tokens, q heads, kv heads): the bench workload's head counts over the
# launch shapes (one step per wave up to 512 tokens, two up to 1024, three
# beyond), and other head counts.
QK_AB_CASES = [(256, 32, 8), (768, 32, 8), (1024, 32, 8), (4096, 32, 8), (16384, 32, 8), (65536, 32, 8),
               (256, 64, 8), (4096, 64, 8), (16384, 64, 8), (600, 28, 4), (5000, 28, 4), (3000, 96, 8),
               (20000, 96, 8), (4096, 8, 1), (65536, 8, 1), (32768, 16, 4)]


def qk_ab(rounds: int = 6, launches: int = 40) -> None:
    """qk_norm_rope_fwd against the prior QK kernel (libmbn_prior_qk.so) on
    the same data (bf16, full rotary, theta 1e6, random positions below 2^17):
    outputs compared bit for bit, then per round, in alternating order, the
    median of `launches` individually timed launches over buffer sets rotated
    through >= 1 GiB. One JSON line per case and kernel."""
    sys.path.insert(0, ROOT)
    import json

    import torch

    h = prior_qk_lib()
    lib = __import__("memory_bound_normalization_amd").lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = HipTimingEvents(stream)
    g = torch.Generator(device=dev).manual_seed(41)
    for T, hq, hk in QK_AB_CASES:
        width = (hq + 2 * hk) * 128
        n = max(2, -(-(1 << 30) // (T * width * 2)))
        qkv = [torch.randn(T, width, device=dev, generator=g).to(torch.bfloat16) for _ in range(n)]
        qw = (torch.rand(128, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        kw = (torch.rand(128, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        pos = torch.randint(0, 1 << 17, (T,), device=dev, dtype=torch.int64, generator=g)

        def new(i):
            rc = lib.qk_norm_rope_fwd(qkv[i].data_ptr(), qw.data_ptr(), kw.data_ptr(), pos.data_ptr(), T, hq, hk, 128,
                                      1e-6, 1e6, sp)
            if rc != 0:
                raise RuntimeError(f"qk_norm_rope_fwd: status {rc}")

        def old(i):
            rc = h.mbn_prior_qk_norm_rope(qkv[i].data_ptr(), qw.data_ptr(), kw.data_ptr(), pos.data_ptr(), T, hq, hk,
                                          1e-6, 1e6, sp)
            if rc != 0:
                raise RuntimeError(f"prior qk: status {rc}")

        fns = {"library": new, "before": old}
        src = qkv[0].clone()
        outs = []
        for fn in fns.values():
            qkv[0].copy_(src)
            fn(0)
            torch.cuda.synchronize()
            outs.append(qkv[0].clone())
        if not torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)):
            raise RuntimeError(f"T={T} hq={hq} hk={hk}: the two kernels' outputs differ")
        del src, outs
        nb = 2 * T * (hq + hk) * 128 * 2
        res = {k: [] for k in fns}
        for fn in fns.values():
            for i in range(20):
                fn(i % n)
        torch.cuda.synchronize()
        for rnd in range(rounds):
            for k in (list(fns) if rnd % 2 == 0 else list(fns)[::-1]):
                ev = [(timer.new(), timer.new()) for _ in range(launches)]
                for i, (e0, e1) in enumerate(ev):
                    timer.record(e0)
                    fns[k](i % n)
                    timer.record(e1)
                torch.cuda.synchronize()
                us = sorted(timer.elapsed_ms(e0, e1) * 1e3 for e0, e1 in ev)
                timer.close()
                res[k].append(us[len(us) // 2])
        for k, t in res.items():
            us = sorted(t)[len(t) // 2]
            print(json.dumps({"T": T, "n_q": hq, "n_kv": hk, "kernel": k, "median_us": round(us, 2),
                              "pct": round(100 * nb / us / 1e3 / 8000, 2), "rounds_us": [round(v, 2) for v in t]}),
                  flush=True)
        del qkv
        torch.cuda.empty_cache()


def qk_ab_summary(log: str) -> None:
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    by = {}
    for r in rows:
        by.setdefault((r["T"], r["n_q"], r["n_kv"]), {})[r["kernel"]] = r
    print("qk_norm_rope_fwd against the prior QK kernel, same data, outputs bit-identical; per-launch median")
    print("of 40 launches, median over rounds; % of 8 TB/s on 2 x T x (q + kv heads) x 256 B:")
    print(f"  {'T':>6} {'q':>3} {'kv':>3} {'library us':>10} {'%':>6} {'before us':>9} {'%':>6} {'speedup':>7}")
    for (T, hq, hk), d in by.items():
        new, old = d["library"], d["before"]
        print(f"  {T:>6} {hq:>3} {hk:>3} {new['median_us']:>10.2f} {new['pct']:>6.1f} {old['median_us']:>9.2f} "
              f"{old['pct']:>6.1f} {old['median_us'] / new['median_us']:>7.3f}")


def qk_pattern_summary(log: str) -> None:
    import json

    rows = [json.loads(x) for x in open(log) if x.startswith("{")]
    print("qk_norm_rope_fwd against its access pattern with no arithmetic (q and k bytes of each token read")
    print("and written back in place; % of 8 TB/s on 2 x T x 40 x 128 x 2 B):")
    for r in rows:
        print(f"  T={r['T']:<6} {r['kernel']:<22} {r['median_us']:>8.2f} us {r['pct']:>6.2f}%  rounds "
              + " ".join(f"{v:.1f}" for v in r["rounds_us"]))


STREAM_VARIANTS = {
    0: (16384, "128 lanes/row, 2 buffers, 2 WGs/CU"),
    1: (16384, "256 lanes/row, 2 buffers, 2 WGs/CU"),
    2: (16384, "256 lanes/row, 3 buffers, 1 WG/CU"),
    3: (16384, "256 lanes/row, 4 buffers, 1 WG/CU"),
    4: (16384, "512 lanes/row, 4 buffers, 1 WG/CU"),
    5: (16384, "128 lanes/row, 2 buffers, 1 WG/CU"),
    6: (16384, "256 lanes/row, 2 buffers, 1 WG/CU"),
    10: (32768, "512 lanes/row, 2 buffers, 1 WG/CU"),
    11: (32768, "256 lanes/row, 2 buffers, 1 WG/CU"),
    12: (32768, "1024 lanes/row, 2 buffers, 1 WG/CU"),
    20: (8192, "128 lanes/row, 2 buffers, 4 WGs/CU"),
    21: (8192, "128 lanes/row, 3 buffers, 3 WGs/CU"),
    22: (8192, "64 lanes/row, 2 buffers, 4 WGs/CU"),
    23: (8192, "256 lanes/row, 4 buffers, 2 WGs/CU"),
}
STREAM_SHAPES = {16384: (16384, 16384), 32768: (4096, 32768), 8192: (8192, 8192)}


def stream_variants(rounds: int = 3, launches: int = 60) -> None:
    """The pipelined persistent RMSNorm experiment (probe_csrc/timeline.hip)
    against the library's rmsnorm_fwd at the same shapes: every output compared
    with the library's (at most one bf16 ulp apart: the reduction order may
    differ), then event medians over interleaved rounds. Inputs rotate over
    buffer sets of >= 1 GiB so no launch is served from the Infinity Cache."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    tl = timeline_lib()
    tl.mbn_tl_rmsnorm_stream.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                                                 ctypes.c_void_p, ctypes.c_int]
    tl.mbn_tl_rmsnorm_stream.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(13)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    sets = {}
    for n, (M, N) in STREAM_SHAPES.items():
        nset = max(1, -(-(1 << 30) // (2 * M * N * 2)))
        w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
        sets[n] = [(torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16), w,
                    torch.empty(M, N, dtype=torch.bfloat16, device=dev)) for _ in range(nset)]
    x0, w0, y0 = sets[16384][0]
    for _ in range(2400):
        mbn.rmsnorm_fwd(x0, w0, y0, eps=1e-6)
    torch.cuda.synchronize()

    def run_stream(v, x, w, y):
        M, N = x.shape
        rc = tl.mbn_tl_rmsnorm_stream(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, 1e-6, sp, v)
        if rc != 0:
            raise RuntimeError(f"stream variant {v}: status {rc}")

    # correctness against the library, every output
    for v, (n, desc) in STREAM_VARIANTS.items():
        x, w, y = sets[n][0]
        ref = mbn.rmsnorm_fwd(x, w, eps=1e-6)
        y.fill_(0)
        run_stream(v, x, w, y)
        torch.cuda.synchronize()
        d = (y.float() - ref.float()).abs()
        tol = ref.float().abs() * 2.0 ** -7 + 1e-6
        bad = int((d > tol).sum())
        same = float((y.view(torch.int16) == ref.view(torch.int16)).float().mean())
        print(json.dumps({"check": v, "outside_1ulp": bad, "bit_equal_frac": round(same, 6)}), flush=True)
        if bad:
            raise RuntimeError(f"stream variant {v}: {bad} outputs differ from the library by more than 1 ulp")
    timer = HipTimingEvents(stream)
    res = {("lib", n): [] for n in STREAM_SHAPES}
    res.update({v: [] for v in STREAM_VARIANTS})

    def timed(key, fn, n):
        ev = [(timer.new(), timer.new()) for _ in range(launches)]
        for i, (a, b) in enumerate(ev):
            x, w, y = sets[n][i % len(sets[n])]
            timer.record(a)
            fn(x, w, y)
            timer.record(b)
        torch.cuda.synchronize()
        res[key] += [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
        timer.close()

    for rnd in range(rounds):
        for n in STREAM_SHAPES:
            timed(("lib", n), lambda x, w, y: mbn.rmsnorm_fwd(x, w, y, eps=1e-6), n)
            for v, (vn, _) in STREAM_VARIANTS.items():
                if vn == n:
                    timed(v, lambda x, w, y, v=v: run_stream(v, x, w, y), n)
        print(f"round {rnd} done", flush=True)
    for key, us in res.items():
        n = key[1] if isinstance(key, tuple) else STREAM_VARIANTS[key][0]
        M, N = STREAM_SHAPES[n]
        nb = 2 * M * N * 2 + 2 * N
        med = float(np.median(us))
        print(json.dumps({"kernel": "library" if isinstance(key, tuple) else key, "shape": f"{M}x{N}",
                          "desc": "rmsnorm_fwd" if isinstance(key, tuple) else STREAM_VARIANTS[key][1],
                          "median_us": round(med, 2), "mean_us": round(float(np.mean(us)), 2),
                          "pct_median": round(100 * nb / med / 1e3 / 8000, 2)}), flush=True)


CLAIM_CASES = [(0, 512), (256, 512), (512, 512), (1024, 512), (512, 256), (1024, 1024), (2048, 512)]


def claim_variants(rounds: int = 4, launches: int = 50) -> None:
    """The claimed-tail experiment (probe_csrc/timeline.hip, tl_claim_kernel)
    at x[16384, 16384]: (dynamic blocks, claiming workgroups) cases against the
    same geometry without claims (variant 0) and the library's rmsnorm_fwd;
    every output compared with the library's, then event medians over
    interleaved rounds."""
    sys.path.insert(0, ROOT)
    import json

    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn

    tl = timeline_lib()
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    tl.mbn_tl_rmsnorm_claim.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, vp, ctypes.c_uint, ctypes.c_uint]
    tl.mbn_tl_rmsnorm_claim.restype = ctypes.c_int
    tl.mbn_tl_rmsnorm_variant.argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, vp, ctypes.c_int]
    tl.mbn_tl_rmsnorm_variant.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(14)
    M = N = 16384
    x = torch.randn(M, N, device=dev, generator=g).to(torch.bfloat16)
    w = (torch.rand(N, device=dev, generator=g) + 0.5).to(torch.bfloat16)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    for _ in range(2400):
        mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
    torch.cuda.synchronize()
    ref = mbn.rmsnorm_fwd(x, w, eps=1e-6)

    def claim(c):
        rc = tl.mbn_tl_rmsnorm_claim(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, 1e-6, sp, c[0], c[1])
        if rc != 0:
            raise RuntimeError(f"claim {c}: status {rc}")

    for c in CLAIM_CASES:
        for rep in range(2):
            y.fill_(0)
            claim(c)
            torch.cuda.synchronize()
            same = bool(torch.equal(y.view(torch.int16), ref.view(torch.int16)))
            print(json.dumps({"check": list(c), "rep": rep, "bit_equal_to_library": same}), flush=True)
            if not same:
                raise RuntimeError(f"claim {c}: output differs from the library's")
    timer = HipTimingEvents(stream)
    keys = ["library", "variant0"] + [tuple(c) for c in CLAIM_CASES]
    res = {k: [] for k in keys}

    def fn_of(k):
        if k == "library":
            return lambda: mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
        if k == "variant0":
            return lambda: tl.mbn_tl_rmsnorm_variant(x.data_ptr(), w.data_ptr(), y.data_ptr(), M, N, 1e-6, sp, 0)
        return lambda: claim(k)

    for rnd in range(rounds):
        for k in keys:
            fn = fn_of(k)
            ev = [(timer.new(), timer.new()) for _ in range(launches)]
            for a, b in ev:
                timer.record(a)
                fn()
                timer.record(b)
            torch.cuda.synchronize()
            res[k] += [timer.elapsed_ms(a, b) * 1e3 for a, b in ev]
            timer.close()
        print(f"round {rnd} done", flush=True)
    nb = 2 * M * N * 2 + 2 * N
    for k in keys:
        med = float(np.median(res[k]))
        print(json.dumps({"kernel": k if isinstance(k, str) else {"ndyn": k[0], "nclaim": k[1]},
                          "median_us": round(med, 2), "mean_us": round(float(np.mean(res[k])), 2),
                          "pct_median": round(100 * nb / med / 1e3 / 8000, 2)}), flush=True)
    # XCD finish times without and with the claimed tail (timeline records: a
    # claiming workgroup's record is that of the last block it served)
    rmax = tl.mbn_tl_max_blocks()
    for k in ("variant0", (2048, 512)):
        for rep in range(4):
            for _ in range(240):
                mbn.rmsnorm_fwd(x, w, y, eps=1e-6)
            torch.cuda.synchronize()
            tl.mbn_tl_clear(rmax)
            fn_of(k)()
            torch.cuda.synchronize()
            rec = np.zeros((rmax, 8), dtype=np.uint64)
            tl.mbn_tl_fetch(rec.ctypes.data, rmax)
            rec = rec[rec[:, 7] == TL_MAGIC].astype(np.float64)
            t0 = rec[:, 0].min()
            done = (rec[:, 3] - t0) / TICKS_PER_US
            xcc = rec[:, 4].astype(np.int64) & 0xF
            ends = [float(done[xcc == c].max()) for c in range(8)]
            print(json.dumps({"xcd_ends": k if isinstance(k, str) else {"ndyn": k[0], "nclaim": k[1]}, "rep": rep,
                              "span_us": round(max(ends), 2), "xcd_end_us": [round(e, 2) for e in ends],
                              "spread_us": round(max(ends) - min(ends), 2)}), flush=True)


def _short_kernel(n: str) -> str:
    m = re.search(r"stream_copy<[^>]*>", n)
    if m:
        return m.group(0)
    n = n.replace("mbn::(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\(mbn::RowNormArgs\)|\(mbn::RowNormAnyArgs\)|\(RowNormAnyArgs\)|\(unsigned short\*.*", "", n)
    return n.replace("(mbn::Norm)", "").replace("mbn::Bf16, ", "").replace("mbn::", "")


def trace_summary(d: str, bench_json: str) -> None:
    """The headline kernel-trace summary: rocprofv3 --kernel-trace --stats of
    a bench.py run (files in d), beside that run's JSON line (bench_json: a
    file holding it)."""
    import json
    import statistics

    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_trace.csv"))))
    stats = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    rms = sorted((r for r in rows if any(k in r["Kernel_Name"] for k in ROW_KERNELS)),
                 key=lambda r: int(r["Start_Timestamp"]))
    b = [json.loads(line) for line in open(bench_json) if line.startswith("{")][-1]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rms][-b["steps"]:]
    algo = b["roofline"]["algorithmic_bytes_per_launch"]
    r0 = rms[0]
    title = "rmsnorm_fwd, x[16384, 16384] bf16 -> y (bench workload), MI355X (gfx950), one GPU"
    print(title)
    print("=" * len(title))
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print(f"  rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o run -- \\")
    # the command as it was run: the CPU baseline leg is in the JSON unless it
    # was switched off
    flags = "" if "cpu_baseline" in b else " --no-cpu-baseline"
    if (b["warmup"], b["steps"]) != (2000, 200):
        flags = f" --gpus 1 --steps {b['steps']} --warmup {b['warmup']}" + flags
    print(f"      python -u bench.py{flags} > {bench_json}")
    print(f"      ({b['warmup']} warm-up + {b['steps']} timed steps)")
    print(f"  python probe.py trace-summary {d} {bench_json}")
    print()
    print(f"Kernel statistics (run_kernel_stats.csv, every dispatch of the run, warm-up included):")
    print()
    print(f"  {'kernel':<66} {'calls':>5} {'avg_us':>8} {'min_us':>8} {'max_us':>8} {'sd_us':>7}")
    for st in stats:
        kn = _short_kernel(st["Name"])[:66]
        print(f"  {kn:<66} {int(st['Calls']):>5} {float(st['AverageNs']) / 1e3:>8.2f} "
              f"{float(st['MinNs']) / 1e3:>8.2f} {float(st['MaxNs']) / 1e3:>8.2f} {float(st['StdDev']) / 1e3:>7.2f}")
    print()
    print(f"{_short_kernel(r0['Kernel_Name'])}: workgroup {r0['Workgroup_Size_X']} threads, grid "
          f"{int(r0['Grid_Size_X']) // int(r0['Workgroup_Size_X'])} workgroups, VGPR {r0['VGPR_Count']}, "
          f"SGPR {r0['SGPR_Count']}, LDS {r0.get('LDS_Block_Size', r0.get('Lds_Size', '?'))} B")
    print()
    m = statistics.mean(dur)
    print(f"Algorithmic bytes per launch: 2*M*N*2 + 2*N = {algo:,} B.")
    print(f"Mean over the last {len(dur)} dispatches (the timed steps), trace: {m:.2f} us -> "
          f"{algo / m / 1e3:.1f} GB/s = {100 * algo / m / 1e3 / 8000:.2f}% of 8 TB/s.")
    how = ("the kernel's own start and end in HIP events" if "timing" in b["roofline"]
           else "HIP events around each launch")
    print(f"The same run's bench.py line ({how}): mean {b['roofline']['mean_us']} us, "
          f"best {b['roofline']['best_us']} us -> {b['value']} GB/s ({100 * b['roofline']['frac']:.2f}%); "
          f"the means differ by {100 * (b['roofline']['mean_us'] - m) / m:+.2f}%.")
    cr = b["roofline"].get("streaming_copy_reference")
    if cr:
        print(f"Streaming copy of the same buffers in the same run (stream_copy<256, 1>): "
              f"{cr['mean_us']} us, {cr['GBps']} GB/s ({100 * cr['frac']:.2f}%); rmsnorm / copy = "
              f"{cr['rmsnorm_over_copy']}.")


def suite_summary(d: str, suite_log: str, warm: int = 3000) -> None:
    """The all-workloads table from rocprofv3 --kernel-trace of
    `python -u bench.py --suite --steps 50 --warmup 5` (files in d) and that
    run's JSON lines (suite_log). The first `warm` dispatches (the suite's
    initial load) are skipped; each workload then owns an equal run of
    dispatches in order."""
    import json
    import statistics

    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ks = [r for r in rows if any(k in r["Kernel_Name"] for k in ("rownorm", "qk_norm_rope", "stream_copy"))]
    ks = ks[warm:]
    cases = [json.loads(line) for line in open(suite_log) if line.startswith("{")]
    per, rem = divmod(len(ks), len(cases))
    if rem:
        raise SystemExit(f"{len(ks)} dispatches do not split into {len(cases)} workloads")
    title = "Every workload, GPU-side kernel durations, MI355X (gfx950), one GPU"
    print(title)
    print("=" * len(title))
    print()
    print("Commands (from the repository root, TMPDIR=/tmp):")
    print(f"  rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o run -- \\")
    print(f"      python -u bench.py --suite --steps 50 --warmup 5 > {suite_log}")
    print(f"  python probe.py suite-summary {d} {suite_log}")
    print()
    print("bench.py --suite rotates over buffer sets of >= 1 GiB per workload, so no launch")
    print("finds its inputs in the 256 MiB Infinity Cache. Durations are kernel start to")
    print(f"end from the trace ({per} dispatches per workload: warm-up, per-launch-event and")
    print("batch phases); bytes are the algorithmic bytes of one launch; % is of 8 TB/s.")
    print("grid_MxN: the RMSNorm shape grid of the normalization pages (the leading M x N")
    print("block of the 16384 x 16384 input). Template arguments: rownorm_kernel<mode, WPR,")
    print("ROWS, RPL, MAXC, full, chunk wait>, rownorm_regs_kernel<mode, WPR, ROWS, MAXC,")
    print("full> (rows in VGPRs), rownorm_persistent_kernel<mode, WPR, RPL, MAXC, full>")
    print("(mode 0 RMSNorm, 1 residual add + RMSNorm, 2 LayerNorm, 3 L2Norm),")
    print("rownorm_any_kernel / rownorm_s16_kernel (widths that are not whole 16-byte")
    print("chunks). WGs is the grid size (the persistent grid loops over the rows).")
    print()
    if any(c["kernel"] == "stream_copy" for c in cases):
        print("<workload>_copy: the plain streaming copy (stream_copy<256, 1> of libmbn_stream.so,")
        print("4 KiB per workgroup, 16-byte non-temporal loads and stores) of the same input bytes")
        print("between the same buffers; 'of copy' = the copy's median time / the workload's.")
    print()
    print(f"  {'workload':<22} {'op':<20} {'kernel instantiation':<56} {'WGs':>6} {'median_us':>9} {'min_us':>8} "
          f"{'GB/s':>7} {'%':>6} {'of copy':>7}")
    meds = {}
    for i, c in enumerate(cases):
        grp = ks[i * per:(i + 1) * per]
        meds[c["workload"]] = statistics.median(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
    for i, c in enumerate(cases):
        grp = ks[i * per:(i + 1) * per]
        names = {_short_kernel(r["Kernel_Name"]) for r in grp}
        if len(names) != 1:
            raise SystemExit(f"workload {c['workload']}: kernels {names}")
        du = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in grp)
        med = statistics.median(du)
        b = c["algorithmic_bytes"]
        wg = int(grp[0]["Grid_Size_X"]) // int(grp[0]["Workgroup_Size_X"])
        cm = meds.get(c["workload"] + "_copy")
        vs = f"{cm / med:>7.3f}" if cm and c["kernel"] != "stream_copy" else f"{'':>7}"
        print(f"  {c['workload']:<22} {c['kernel']:<20} {names.pop()[:56]:<56} {wg:>6} {med:>9.2f} {du[0]:>8.2f} "
              f"{b / med / 1e3:>7.0f} {b / med / 1e3 / 80:>6.1f} {vs}")


def experiments_summary(sizes_log: str, variants_log: str, claim_log: str, stream_log: str) -> None:
    """Tables of the size sweep, the geometry variants, the claimed-tail and the
    pipelined persistent experiments from their JSON-line outputs."""
    import json

    def lines(p):
        return [json.loads(x) for x in open(p) if x.startswith("{")]

    print("Size sweep at N = 16384 (event mean of 100 launches after 50; copy = stream_copy<256, 1>):")
    print(f"  {'kernel':<8} {'M':>7} {'bytes':>12} {'mean_us':>9} {'% of 8 TB/s':>12}")
    for r in lines(sizes_log):
        if "fit" in r:
            print(f"  least-squares line, {r['fit']}: slope -> {r['steady_GBps']} GB/s ({r['steady_pct']}%), "
                  f"intercept {r['intercept_us']} us")
        else:
            print(f"  {r['kernel']:<8} {r['M']:>7} {r['bytes']:>12} {r['mean_us']:>9.2f} {r['pct']:>12.2f}")
    print()
    print("Geometry variants of the one-shot kernel (timeline marks compiled in; event median of 180")
    print("launches in interleaved rounds; the trace columns are from one traced launch):")
    print(f"  {'variant':<82} {'med_us':>7} {'%':>6} {'steady%':>7} {'gap':>5} {'gap90':>5} {'xcd':>5} {'land':>5}")
    for r in lines(variants_log):
        if r["variant"] == "library":
            print(f"  {'library rmsnorm_fwd, N = ' + str(r['N']) + ' (no marks)':<82} {r['median_us']:>7.2f} {r['pct']:>6.2f}")
            continue
        print(f"  {str(r['variant']) + ': ' + r['desc']:<82} {r['median_us']:>7.2f} {r['pct']:>6.2f} "
              f"{r['steady_pct']:>7.2f} {r['gap_us_median']:>5.2f} {r['gap_us_p90']:>5.2f} "
              f"{r['xcd_end_spread_us']:>5.2f} {r['wg_land_us_median']:>5.2f}")
    print("  (gap: us from a workgroup's end to the next start on its CU, median / p90; xcd: spread of")
    print("  the XCD finish times; land: median us from a workgroup's start until its rows are reduced)")
    print()
    print("Claimed tail at x[16384, 16384] (the table's geometry; ndyn row blocks claimed from a device")
    print("counter by nclaim workgroups dispatched after the static ones; event median of 200 launches):")
    for r in lines(claim_log):
        if "check" in r:
            continue
        if "xcd_ends" in r:
            k = r["xcd_ends"]
            name = k if isinstance(k, str) else f"ndyn {k['ndyn']}, nclaim {k['nclaim']}"
            print(f"  traced {name:<21} span {r['span_us']:7.2f} us  XCD finish spread {r['spread_us']:5.2f} us  "
                  f"(" + " ".join(f"{e:.1f}" for e in r["xcd_end_us"]) + ")")
            continue
        k = r["kernel"]
        name = k if isinstance(k, str) else f"ndyn {k['ndyn']}, nclaim {k['nclaim']}"
        print(f"  {name:<28} {r['median_us']:>8.2f} us  {r['pct_median']:>6.2f}%")
    print()
    print("Pipelined persistent kernel (rows g, g + G, ... per workgroup, NB LDS row buffers in a ring,")
    print("the next row's copy issued as soon as pass 2 has read a buffer; event median of 180 launches):")
    for r in lines(stream_log):
        if "check" in r:
            continue
        name = "library rmsnorm_fwd" if r["kernel"] == "library" else f"{r['kernel']}: {r['desc']}"
        print(f"  {r['shape']:<12} {name:<50} {r['median_us']:>8.2f} us  {r['pct_median']:>6.2f}%")


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
    elif len(sys.argv) in (2, 3) and sys.argv[1] == "timeline":
        timeline(*sys.argv[2:])
    elif len(sys.argv) == 3 and sys.argv[1] == "timeline-summary":
        timeline_summary(sys.argv[2])
    elif len(sys.argv) in (2, 3) and sys.argv[1] == "variants":
        variants(*sys.argv[2:])
    elif len(sys.argv) == 4 and sys.argv[1] == "trace-summary":
        trace_summary(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 4 and sys.argv[1] == "suite-summary":
        suite_summary(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 6 and sys.argv[1] == "experiments-summary":
        experiments_summary(*sys.argv[2:])
    elif len(sys.argv) == 2 and sys.argv[1] == "claim":
        claim_variants()
    elif len(sys.argv) == 2 and sys.argv[1] == "stream":
        stream_variants()
    elif len(sys.argv) == 2 and sys.argv[1] == "sizes":
        sizes()
    elif len(sys.argv) == 2 and sys.argv[1] == "staging":
        staging()
    elif len(sys.argv) in (2, 3) and sys.argv[1] == "any-width-ab":
        if len(sys.argv) == 3:  # N:offset,... instead of the default widths
            ANY_AB_SHAPES[:] = [tuple(int(v) for v in c.split(":")) for c in sys.argv[2].split(",")]
        any_width_ab()
    elif len(sys.argv) == 3 and sys.argv[1] == "any-width-summary":
        any_width_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "qk-ab":
        qk_ab()
    elif len(sys.argv) == 3 and sys.argv[1] == "qk-ab-summary":
        qk_ab_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "qk-pattern":
        qk_pattern()
    elif len(sys.argv) == 3 and sys.argv[1] == "qk-pattern-summary":
        qk_pattern_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "wide-rows":
        wide_rows()
    elif len(sys.argv) == 3 and sys.argv[1] == "wide-rows-summary":
        wide_rows_summary(sys.argv[2])
    elif len(sys.argv) in (2, 3, 5) and sys.argv[1] == "small-regs":
        small_regs(*sys.argv[2:])
    elif len(sys.argv) == 4 and sys.argv[1] == "small-regs-summary":
        small_regs_summary(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 4 and sys.argv[1] == "small-regs-compare":
        small_regs_compare(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 2 and sys.argv[1] == "qk-angles":
        qk_angles()
    elif len(sys.argv) == 2 and sys.argv[1] == "launch-modes":
        launch_modes()
    elif len(sys.argv) == 5 and sys.argv[1] == "launch-modes-summary":
        launch_modes_summary(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) == 3 and sys.argv[1] == "qk-angles-summary":
        qk_angles_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "load-policy":
        load_policy()
    elif len(sys.argv) == 3 and sys.argv[1] == "load-policy-summary":
        load_policy_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "late-weights":
        late_weights()
    elif len(sys.argv) == 3 and sys.argv[1] in ("staging-summary", "late-weights-summary"):
        ab_summary(sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "store-policy":
        store_policy()
    elif len(sys.argv) == 3 and sys.argv[1] == "store-policy-summary":
        store_policy_summary(sys.argv[2])
    elif len(sys.argv) in (4, 5) and sys.argv[1] == "summarize":
        summarize(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
