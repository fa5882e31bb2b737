"""The library is stateless: calls from several host threads at once, each on
a stream of its own, must give the results of the same calls made one by one.
Four threads run RMSNorm (staged-row, persistent and any-width paths), the
residual add, LayerNorm, L2Norm and the QK-norm + rotary on their own inputs
and streams, concurrently, several times over; every output is compared bit
for bit with a sequential run on the default stream, and one input set with
the fp64 oracle."""

import threading

import numpy as np
import pytest

from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import random_bf16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import memory_bound_normalization_amd as mbn  # noqa: E402
from oracle import rmsnorm_fwd as o_rms  # noqa: E402

SHAPES = [(3000, 4096), (2049, 16384), (37, 1001), (513, 2048)]


def _inputs(seed):
    rng = np.random.default_rng(seed)
    M, N = SHAPES[seed % len(SHAPES)]
    host = {
        "x": random_bf16_bits(rng, (M, N)),
        "r": random_bf16_bits(rng, (M, N)),
        "w": random_bf16_bits(rng, (N,), lo=0.5, hi=1.5),
        "b": random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5),
        "qkv": random_bf16_bits(rng, (64, 12 * 128)),
        "qw": random_bf16_bits(rng, (128,), lo=0.5, hi=1.5),
        "kw": random_bf16_bits(rng, (128,), lo=0.5, hi=1.5),
    }
    dev = {k: to_gpu_bf16(v) for k, v in host.items()}
    dev["pos"] = torch.arange(64, device="cuda", dtype=torch.int64) * 7
    return host, dev


def _run(dev, stream=None):
    """All entry points on one input set; returns the output tensors."""
    out = {}
    out["y"] = mbn.rmsnorm_fwd(dev["x"], dev["w"], eps=1e-6, stream=stream)
    out["h"], out["ya"] = mbn.add_rmsnorm_fwd(dev["x"], dev["r"], dev["w"], eps=1e-6, stream=stream)
    out["yl"] = mbn.layernorm_fwd(dev["x"], dev["w"], dev["b"], eps=1e-5, stream=stream)
    out["y2"] = mbn.l2norm_fwd(dev["x"], eps=1e-12, stream=stream)
    q = dev["qkv"].clone()
    out["qkv"] = mbn.qk_norm_rope_fwd(q, dev["qw"], dev["kw"], dev["pos"], 8, 2, 128, eps=1e-6, theta=1e6,
                                      stream=stream)
    return out


def test_concurrent_threads_and_streams():
    print("[threads] 4 threads x 4 rounds", flush=True)
    sets = [_inputs(s) for s in range(4)]
    ref = []
    for _, dev in sets:
        ref.append({k: from_gpu_bf16(v) for k, v in _run(dev).items()})
        torch.cuda.synchronize()
    assert_parity(ref[0]["y"], o_rms(sets[0][0]["x"], sets[0][0]["w"], 1e-6), "sequential rmsnorm")

    streams = [torch.cuda.Stream() for _ in sets]
    results = [[] for _ in sets]
    errors = []
    start = threading.Barrier(len(sets))

    def worker(i):
        try:
            torch.cuda.set_device(0)
            start.wait()
            for _ in range(4):
                with torch.cuda.stream(streams[i]):
                    out = _run(sets[i][1], stream=streams[i])
                streams[i].synchronize()
                results[i].append({k: from_gpu_bf16(v) for k, v in out.items()})
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(sets))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    for i, runs in enumerate(results):
        assert len(runs) == 4
        for k, got in ((k, r[k]) for r in runs for k in r):
            assert np.array_equal(got, ref[i][k]), f"thread {i}: {k} differs from the sequential run"
