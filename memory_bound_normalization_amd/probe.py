"""Short GPU program for hardware-counter runs, and the summarizer of their output.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe run
    rocprofv3 --pmc WRITE_SIZE -d <dir> -o run -- python -m memory_bound_normalization_amd.probe run
    python -m memory_bound_normalization_amd.probe summarize <fetch_dir> <write_dir>

`run` launches rmsnorm_fwd on x[16384, 16384] (the benchmark workload) a few
times, then a plain device-to-device copy of the same 512 MiB (torch's copy
kernel) as the calibration: the counters of the copy, whose true HBM traffic is
known (512 MiB read, 512 MiB written), give the factor that converts each
counter reading into bytes. `summarize` prints the per-launch HBM traffic of the
RMSNorm kernel from the two runs' counter CSV files.
"""

from __future__ import annotations

import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LAUNCHES = 5
COPY_BYTES = 16384 * 16384 * 2


def run() -> None:
    sys.path.insert(0, ROOT)
    import numpy as np
    import torch

    import memory_bound_normalization_amd as mbn
    from workloads import RMS_WORKLOADS, make_rms_inputs

    wl = RMS_WORKLOADS["rms_16384x16384"]
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


def _rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def _per_kernel(d: str, counter: str):
    """{'rmsnorm': [values...], 'copy': [values...]} for one counter (summed over its instances)."""
    acc = {}
    for r in _rows(d):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    res = {"rmsnorm": [], "copy": []}
    for (_, name), v in sorted(acc.items(), key=lambda kv: int(kv[0][0])):
        if "rownorm_kernel" in name:
            res["rmsnorm"].append(v)
        elif "copy" in name.lower() or "elementwise" in name.lower():
            res["copy"].append(v)
    return res


def summarize(fetch_dir: str, write_dir: str) -> None:
    f = _per_kernel(fetch_dir, "FETCH_SIZE")
    w = _per_kernel(write_dir, "WRITE_SIZE")
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    f_r, f_c = mean(f["rmsnorm"]), mean(f["copy"])
    w_r, w_c = mean(w["rmsnorm"]), mean(w["copy"])
    f_scale = COPY_BYTES / f_c
    w_scale = COPY_BYTES / w_c
    fetch_b = f_r * f_scale
    write_b = w_r * w_scale
    print(f"rmsnorm FETCH_SIZE per launch (raw, KiB units): {f_r:.1f}  over {len(f['rmsnorm'])} launches")
    print(f"rmsnorm WRITE_SIZE per launch (raw, KiB units): {w_r:.1f}  over {len(w['rmsnorm'])} launches")
    print(f"copy    FETCH_SIZE per launch (raw): {f_c:.1f}   WRITE_SIZE: {w_c:.1f}   true bytes each way: {COPY_BYTES}")
    print(f"calibration factors (bytes per counter unit): fetch {f_scale:.3f}  write {w_scale:.3f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"write_bytes_per_launch: {write_b:.0f}")
    print(f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}")


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
