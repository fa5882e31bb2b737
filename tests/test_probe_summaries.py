"""CPU tests of the hardware-counter summarizers of memory_bound_normalization_amd.probe.

The summarizers turn rocprofv3 counter CSV files into bytes per launch, with a
device copy of known size as the calibration. These tests feed them small
synthetic CSV files (no GPU) and check which dispatches count as the measured
kernel and which as the calibration copy.
"""

import csv
import os

import pytest

from memory_bound_normalization_amd import probe

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
