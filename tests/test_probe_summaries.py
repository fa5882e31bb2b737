"""CPU tests of the hardware-counter summarizers of probe.py (the measurement tools next to bench.py).

The summarizers turn rocprofv3 counter CSV files into bytes per launch, with a
device copy of known size as the calibration. These tests feed them small
synthetic CSV files (no GPU) and check which dispatches count as the measured
kernel and which as the calibration copy.
"""

import csv
import os

import pytest

import probe

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows, start=1):
            # two counter instances per dispatch, summed by the summarizer
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})


def _qk_rows(qk_value, copy_value):
    return ([("void at::native::vectorized_elementwise_kernel<4, float>", 7.0e5)]  # input set-up
            + [("void mbn::qk_norm_rope_kernel<mbn::Bf16>", qk_value)] * 3
            + [("__amd_rocclr_copyBuffer", copy_value)] * 3)


def test_qk_summary_uses_only_the_copy_kernel(tmp_path, capsys):
    copy_bytes = probe.COPY_BYTES
    qk = probe.QK_TOKENS * (probe.QK_HQ + probe.QK_HKV) * probe.QK_D * 2
    # counters in the units the copy calibrates: fetch 2 KiB, write 1 KiB per unit
    _write(tmp_path / "f", "FETCH_SIZE", _qk_rows(qk / 2048, copy_bytes / 2048))
    _write(tmp_path / "w", "WRITE_SIZE", _qk_rows(qk / 1024, copy_bytes / 1024))
    probe.qk_summarize(str(tmp_path / "f"), str(tmp_path / "w"))
    out = capsys.readouterr().out
    assert "calibration factors (bytes per counter unit): fetch 2048.000  write 1024.000" in out
    assert f"fetch_bytes_per_launch: {qk}" in out
    assert f"write_bytes_per_launch: {qk}" in out


def test_default_copy_filter_keeps_torch_copies(tmp_path):
    rows = [("void mbn::rownorm_kernel<0>", 10.0), ("__amd_rocclr_copyBuffer", 4.0),
            ("void at::native::vectorized_elementwise_kernel<4, copy>", 6.0)]
    _write(tmp_path / "f", "FETCH_SIZE", rows)
    res = probe._per_kernel(str(tmp_path / "f"), "FETCH_SIZE")
    assert res["rmsnorm"] == [pytest.approx(10.0)]
    assert res["copy"] == [pytest.approx(4.0), pytest.approx(6.0)]
    res = probe._per_kernel(str(tmp_path / "f"), "FETCH_SIZE", copy="copyBuffer")
    assert res["copy"] == [pytest.approx(4.0)]


def test_qk_algorithmic_bytes():
    T = probe.QK_TOKENS
    assert probe.qk_algorithmic_bytes() == 2 * T * 40 * 128 * 2 + 512 + 8 * T == 1342702080


def test_timing_events_bind_without_a_gpu():
    """bench.py's timing events bind the HIP runtime's event calls (no call is
    made until an event is created)."""

    class _Stream:
        cuda_stream = 0

    t = probe.HipTimingEvents(_Stream())
    assert t.events == [] and t.hip.hipEventRecord is not None


def test_timeline_metrics_on_a_synthetic_schedule():
    """Workgroups started every 0.1 us, landing 5 us and finishing 10 us
    later, on 8 XCDs round robin: the steady rate is one workgroup's bytes per
    0.1 us, the overhead one workgroup lifetime, the XCD finish spread 0.7 us."""
    import numpy as np

    n, per_wg = 800, 65536 * 2
    rec = np.zeros((n, 8), dtype=np.uint64)
    for i in range(n):
        s = 1000 + 10 * i  # ticks of 10 ns
        rec[i] = [s, s + 500, s + 990, s + 1000, i % 8, 0, i, probe.TL_MAGIC]
    rec[5, 7] = 0  # a record that was not written is ignored ...
    m = probe.timeline_metrics(rec, (n - 1) * per_wg)
    assert m["blocks"] == n - 1
    rec[5, 7] = probe.TL_MAGIC
    m = probe.timeline_metrics(rec, n * per_wg)
    assert m["blocks"] == n
    assert m["steady_GBps"] == pytest.approx(per_wg / 0.1 / 1e3, rel=1e-3)
    assert m["ideal_us_at_steady"] == pytest.approx(80.0, rel=1e-3)
    assert m["span_us"] == pytest.approx(89.9)
    assert m["overhead_us"] == pytest.approx(9.9, abs=0.05)
    assert m["xcd_end_spread_us"] == pytest.approx(0.7)
    assert m["xcd_blocks"] == {k: 100 for k in range(8)}
    assert m["max_resident_wgs"] == 101
    assert m["wg_land_us_median"] == pytest.approx(5.0) and m["wg_store_us_median"] == pytest.approx(5.0)


def test_store_policy_source_replaces_only_the_one_shot_output_store():
    src = probe.store_policy_source()
    with open(os.path.join(probe.ROOT, "memory_bound_normalization_amd", "csrc", "rownorm.hip")) as f:
        lib = f.read()
    assert src.count("MBN_STORE_Y(yrow + k, o);") == 1
    assert src.replace("MBN_STORE_Y(yrow + k, o);", "store_nt_16(yrow + k, o);") == lib
    # the replaced store is pass 2 of the one-shot body, not another kernel's
    assert src.index("rownorm_block(const RowNormArgs") < src.index("MBN_STORE_Y") < src.index(
        ") rownorm_kernel(RowNormArgs a)")


def test_ceiling_summary_groups_dispatches_per_case(tmp_path, capsys):
    d = tmp_path / "trace"
    d.mkdir()
    per = 3 + probe.CEIL_REPS
    rows, t = [], 0
    # a short set-up dispatch, then per case: 3 warm-up + CEIL_REPS timed launches
    for k in range(len(probe.CEILING_CASES)):
        for j in range(per):
            dur = 100_000 + 1000 * k + (50_000 if j < 3 else 0)  # warm-ups slower, excluded
            rows.append({"Kernel_Name": f"void k{k}(int)", "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 10
    rows.insert(0, {"Kernel_Name": "setup", "Start_Timestamp": -5000, "End_Timestamp": -4000})
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    probe.ceiling_summary(str(d))
    out = capsys.readouterr().out.strip().split("\n")
    assert len(out) == len(probe.CEILING_CASES)
    for k, (line, (name, nb, *_)) in enumerate(zip(out, probe.CEILING_CASES)):
        assert line.startswith(name) and f"k{k}" in line
        us = (100_000 + 1000 * k) / 1e3
        assert f"{us:9.2f} us" in line


def test_store_policy_summary_table(tmp_path, capsys):
    log = tmp_path / "sp.log"
    log.write_text(
        '{"check": "every policy\'s output equals the library\'s bit for bit"}\n'
        "round 0 done\n"
        '{"kernel": "library", "stores": "nt (compiler)", "median_us": 164.7, "pct": 81.49, "rounds_us": [165.1, 164.4]}\n'
        '{"kernel": "policy 1", "stores": "nt sc1", "median_us": 165.2, "pct": 81.26, "rounds_us": [164.9, 165.3]}\n')
    probe.store_policy_summary(str(log))
    out = capsys.readouterr().out
    assert "library      nt (compiler)         164.70        81.49  165.1 164.4" in out
    assert "policy 1     nt sc1                165.20        81.26  164.9 165.3" in out
    assert "bit for bit" in out


def test_counter_summary_counts_both_row_kernels(tmp_path):
    """The row-norm kernels of either kind (staged rows, rows in VGPRs) count as
    the measured kernel; torch's copy as the calibration."""
    d = tmp_path / "fetch"
    _write(str(d), "FETCH_SIZE", [("void mbn::(anonymous namespace)::rownorm_regs_kernel<(mbn::Norm)0, mbn::Bf16, 16, 1, 4, true>(mbn::RowNormArgs)", 10.0),
                                  ("void mbn::(anonymous namespace)::rownorm_kernel<(mbn::Norm)0, mbn::Bf16, 2, 2, 1, 16, true, true>(mbn::RowNormArgs)", 12.0),
                                  ("__amd_rocclr_copyBuffer", 20.0)])
    res = probe._per_kernel(str(d), "FETCH_SIZE")
    assert res == {"rmsnorm": [10.0, 12.0], "copy": [20.0]}


def test_ab_summary_table(tmp_path, capsys):
    import json

    log = tmp_path / "ab.log"
    lines = []
    for k, us in (("late weight (library)", 44.0), ("early weight (before)", 46.0)):
        for m in ("events", "sustained"):
            lines.append(json.dumps({"M": 8192, "N": 8192, "kernel": k, "timing": m, "buffer_sets": 4,
                                     "median_us": us, "pct": 1.0, "rounds_us": [us]}))
    lines.append(json.dumps({"check": "8192x8192: outputs within one bf16 ulp, 99.0000% bit-identical"}))
    log.write_text("\n".join(lines) + "\n")
    probe.ab_summary(str(log))
    out = capsys.readouterr().out
    assert "late weight (library) against early weight (before)" in out
    assert "8192x8192      events          44.00   1.00     46.00   1.00  0.957" in out
    assert "99.0000% bit-identical" in out


def test_qk_pattern_summary_table(tmp_path, capsys):
    log = tmp_path / "qkpat.log"
    log.write_text(
        "noise line\n"
        '{"T": 65536, "kernel": "qk_norm_rope_fwd", "median_us": 215.0, "pct": 78.07, "rounds_us": [215.3, 214.9]}\n'
        '{"T": 65536, "kernel": "access pattern only", "median_us": 214.5, "pct": 78.25, "rounds_us": [214.5]}\n')
    probe.qk_pattern_summary(str(log))
    out = capsys.readouterr().out
    assert "T=65536  qk_norm_rope_fwd         215.00 us  78.07%  rounds 215.3 214.9" in out
    assert "T=65536  access pattern only      214.50 us  78.25%  rounds 214.5" in out


def test_qk_counter_summary_matches_every_kmax_instance(tmp_path):
    """The QK kernel is a template over the rows a wave keeps in flight; each
    instance counts as the measured kernel."""
    d = tmp_path / "fetch"
    _write(str(d), "FETCH_SIZE", [("void mbn::(anonymous namespace)::qk_norm_rope_kernel<mbn::Bf16, 3>(unsigned short*)", 7.0),
                                  ("void mbn::(anonymous namespace)::qk_norm_rope_kernel<mbn::Bf16, 1>(unsigned short*)", 5.0),
                                  ("__amd_rocclr_copyBuffer", 20.0)])
    res = probe._per_kernel(str(d), "FETCH_SIZE", "qk_norm_rope", "copyBuffer")
    assert res == {"rmsnorm": [7.0, 5.0], "copy": [20.0]}


def test_any_width_summary_table(tmp_path, capsys):
    import json

    log = tmp_path / "any.log"
    lines = [json.dumps({"N": 16383, "M": 8192, "offset": 0, "op": "rms", "kernel": k, "median_us": us, "pct": p,
                         "rounds_us": [us]}) for k, us, p in (("library", 98.0, 68.5), ("before", 104.0, 64.5))]
    log.write_text("noise\n" + "\n".join(lines) + "\n")
    probe.any_width_summary(str(log))
    out = capsys.readouterr().out
    assert "   16383   0   8192 rms         98.00   68.5    104.00   64.5   1.061" in out


def test_qk_ab_summary_table(tmp_path, capsys):
    import json

    log = tmp_path / "qkab.log"
    lines = [json.dumps({"T": 65536, "n_q": 32, "n_kv": 8, "kernel": k, "median_us": us, "pct": p, "rounds_us": [us]})
             for k, us, p in (("library", 215.0, 78.1), ("before", 255.0, 65.8))]
    log.write_text("\n".join(lines) + "\n")
    probe.qk_ab_summary(str(log))
    out = capsys.readouterr().out
    assert "   65536  32   8     215.00   78.1    255.00   65.8   1.186" in out


def test_wide_rows_summary(tmp_path, capsys):
    """The wide-row table: one line per variant with its geometry, speed relative to
    the library and the share of bit-identical outputs."""
    import json

    log = tmp_path / "wide.log"
    lines = [{"check": v, "M": 4096, "N": 32768, "bit_identical": 1.0 if v < 5 else 0.99999, "max_bits": 0 if v < 5 else 1}
             for v in probe.WIDE_ROW_VARIANTS]
    lines.append({"kernel": "library", "M": 4096, "N": 32768, "median_us": 86.0, "pct": 78.0, "rounds": [86.0]})
    lines += [{"kernel": v, "M": 4096, "N": 32768, "median_us": 86.0 + v, "pct": 70.0, "rounds": [86.0 + v]}
              for v in probe.WIDE_ROW_VARIANTS]
    log.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    probe.wide_rows_summary(str(log))
    out = capsys.readouterr().out
    assert "1: 1024 lanes, cap 4, XCD run 4, weight with the row" in out
    assert f"{86.0 / 88.0:.3f}" in out  # variant 2 against the library
    assert "99.9990%" in out


def test_load_policy_summary(tmp_path, capsys):
    import json

    log = tmp_path / "lp.log"
    lines = [{"policy": k, "M": 16384, "N": 16384, "median_us": t, "pct": 80.0, "rounds": [t]}
             for k, t in (("nt (library)", 166.0), ("none", 174.3), ("nt sc1", 166.5))]
    log.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    probe.load_policy_summary(str(log))
    out = capsys.readouterr().out
    assert "x[16384, 16384]" in out and f"{166.0 / 174.3:.3f}" in out and "nt sc1" in out


def test_qk_angles_summary(tmp_path, capsys):
    """The angle-path table reads the library's and each mode's durations by kernel name."""
    import csv

    d = tmp_path / "t"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for name, dur in [("void mbn::(anonymous namespace)::qk_norm_rope_kernel<mbn::Bf16, 1>(x)", 3760)] * 5 + [
                (f"void mbn::(anonymous namespace)::qkx_kernel<mbn::Bf16, {m}>(x)", 3400 + 100 * m)
                for m in (0, 1, 3) for _ in range(5)]:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += 10000
    probe.qk_angles_summary(str(d))
    out = capsys.readouterr().out
    assert "library qk_norm_rope_fwd" in out and "3.76" in out
    assert "1: every wave forms the angles" in out and "3.50" in out and "3.70" in out


def test_small_regs_summary(tmp_path, capsys):
    """Blocks of launches announced in the log are matched to the traced row-norm
    kernels in order; output checks (single launches) are skipped."""
    import csv
    import json

    d = tmp_path / "t"
    d.mkdir()
    blocks = [["layer", 4096, 512, "library", 1], ["layer", 4096, 512, 10, 1],
              ["layer", 4096, 512, "library", 3], ["layer", 4096, 512, 10, 3]]
    names = {"library": "void mbn::(anonymous namespace)::rownorm_kernel<(mbn::Norm)2, mbn::Bf16, 4, 1, 1, 2, true, "
                        "false>(mbn::RowNormArgs)",
             10: "void mbn::(anonymous namespace)::rownorm_regs_kernel<(mbn::Norm)2, mbn::Bf16, 4, 1, 2, true>"
                 "(mbn::RowNormArgs)"}
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for op, N, M, case, n in blocks:
            for _ in range(n):
                w.writerow({"Kernel_Name": names[case], "Start_Timestamp": t,
                            "End_Timestamp": t + (4000 if case == "library" else 3600)})
                t += 10000
    log = tmp_path / "small.log"
    log.write_text("\n".join(json.dumps({"block": b}) for b in blocks) + "\n")
    probe.small_regs_summary(str(d), str(log))
    out = capsys.readouterr().out
    assert "small-regs layer" in out and "LayerNorm x[512, 4096]" in out
    assert "4.00 us" in out and "1.111 x library" in out


def test_small_regs_compare(tmp_path, capsys):
    text = ("  LayerNorm x[512, 4096]: library rownorm_kernel<2, 4, 1, 1, 2, true, false>: 4.66 us\n"
            "    rownorm_regs_kernel<2, 1, 1, 8, true>                   4.36 us   1.069 x library\n")
    after = ("  LayerNorm x[512, 4096]: library rownorm_regs_kernel<2, 1, 1, 8, true>: 4.36 us\n"
             "    rownorm_regs_kernel<2, 1, 1, 8, true>                   4.30 us   1.014 x library\n")
    (tmp_path / "b.txt").write_text(text)
    (tmp_path / "a.txt").write_text(after)
    probe.small_regs_compare(str(tmp_path / "b.txt"), str(tmp_path / "a.txt"))
    out = capsys.readouterr().out
    assert "4.66" in out and "4.36" in out and f"{4.66 / 4.36:.3f}" in out and "4.30" in out


def test_small_regs_summary_names_width_and_rows(tmp_path, capsys):
    """A log that starts with the run's arguments gives the command back with its
    width, row counts, rounds and launches."""
    import csv
    import json

    d = tmp_path / "t"
    d.mkdir()
    blocks = [["rms", 4096, 2560, "library", 2], ["rms", 4096, 2560, 3, 2]]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i in range(4):
            w.writerow({"Kernel_Name": "rownorm_regs_kernel<(mbn::Norm)0, mbn::Bf16, 1, 2, 8, true>",
                        "Start_Timestamp": 10000 * i, "End_Timestamp": 10000 * i + 8000})
    log = tmp_path / "small.log"
    head = {"small_regs": {"ops": "rms", "width": "4096", "rows": "2560", "rounds": 6, "launches": 40}}
    log.write_text(json.dumps(head) + "\n" + "\n".join(json.dumps({"block": b}) for b in blocks) + "\n")
    probe.small_regs_summary(str(d), str(log))
    out = capsys.readouterr().out
    assert "probe.py small-regs rms 4096 2560 >" in out
    assert "6 rounds x 40 launches" in out and "RMSNorm x[2560, 4096]" in out and "8.00 us" in out


def test_launch_modes_summary(tmp_path, capsys):
    """Traced kernels are attributed to the announced groups in order; the gap is
    the idle time between consecutive kernels of a group."""
    import csv
    import json

    d = tmp_path / "t"
    d.mkdir()
    blocks = [[4096, 4096, "plain", 3], [4096, 4096, "ev_nofence", 3], [4096, 4096, "ev_default", 2]]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for M, N, mode, n in blocks:
            for _ in range(n):
                w.writerow({"Kernel_Name": "rownorm_regs_kernel<0, 1, 2, 8, true>", "Start_Timestamp": t,
                            "End_Timestamp": t + 11000})
                t += 11000 + (1000 if mode == "plain" else 12000)
    log = tmp_path / "lm.log"
    reg = {"region": [4096, 4096, {"plain": 12.5, "ev_nofence": 25.0, "ev_default": 26.0}]}
    log.write_text("\n".join(json.dumps({"block": b}) for b in blocks) + "\n" + json.dumps(reg) + "\n")
    plain = tmp_path / "lm_plain.log"
    plain.write_text(json.dumps({"region": [4096, 4096, {"plain": 11.5, "ev_nofence": 18.0,
                                                          "ev_default": 18.5}]}) + "\n")
    probe.launch_modes_summary(str(d), str(log), str(plain))
    out = capsys.readouterr().out
    rows = [line.split() for line in out.splitlines() if line.strip().startswith("x[4096, 4096]")]
    assert [r[2] for r in rows] == ["plain", "ev_nofence", "ev_default"]
    assert rows[0][3:] == ["11.00", "1.00", "12.50", "11.50"]
    assert rows[1][3:] == ["11.00", "12.00", "25.00", "18.00"]
