"""GPU tests of the timed entry points (rmsnorm_fwd_timed, qk_norm_rope_fwd_timed):
the same outputs, bit for bit, as the plain entry points, and events that
bracket the kernels' own execution (positive, and no longer than events
recorded around the call on the same stream)."""

import ctypes

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import rmsnorm_fwd as oracle_rmsnorm
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import QK_WORKLOADS, make_qk_inputs, random_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


class Events:
    """hipEvent_t handles created through the HIP runtime torch has loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        self.made.append(e)
        return e

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream)) == 0

    def ms(self, a, b):
        v = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(v), a, b) == 0
        return v.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)


@pytest.fixture
def events():
    ev = Events()
    yield ev
    torch.cuda.synchronize()
    ev.close()


@pytest.mark.parametrize("M, N", [(37, 4096), (1000, 16384), (9, 32768), (5, 65536), (64, 1000)])
def test_rmsnorm_timed_matches_plain(events, M, N):
    print(f"[timed rmsnorm] M={M} N={N}", flush=True)
    rng = np.random.default_rng(M * 7 + N)
    x_bits = random_bf16_bits(rng, (M, N))
    w_bits = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    x, w = to_gpu_bf16(x_bits), to_gpu_bf16(w_bits)
    plain = mbn.rmsnorm_fwd(x, w, eps=1e-6)
    a, b = events.new(), events.new()
    timed = mbn.rmsnorm_fwd_timed(x, w, a, b, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    assert_parity(from_gpu_bf16(timed), oracle_rmsnorm(x_bits, w_bits, 1e-6), f"timed M={M} N={N}")
    assert events.ms(a, b) > 0.0


def test_rmsnorm_timed_interval_is_inside_the_call(events):
    """The kernels' own interval is positive and no longer than one taken by
    events recorded before and after the call on the same stream."""
    M, N = 4096, 16384
    print(f"[timed rmsnorm interval] M={M} N={N}", flush=True)
    x = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    w = torch.ones(N, device="cuda", dtype=torch.bfloat16)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        mbn.rmsnorm_fwd(x, w, y)
    pairs = []
    for _ in range(10):
        o0, k0, k1, o1 = events.new(), events.new(), events.new(), events.new()
        events.record(o0, stream)
        mbn.rmsnorm_fwd_timed(x, w, k0, k1, y=y)
        events.record(o1, stream)
        pairs.append((o0, k0, k1, o1))
    torch.cuda.synchronize()
    for o0, k0, k1, o1 in pairs:
        inner, outer = events.ms(k0, k1), events.ms(o0, o1)
        assert 0.0 < inner <= outer + 1e-3, (inner, outer)
        assert events.ms(o0, k0) >= -1e-3 and events.ms(k1, o1) >= -1e-3


def test_qk_timed_matches_plain(events):
    wl = QK_WORKLOADS["qk_256"]
    print(f"[timed qk] T={wl.T}", flush=True)
    qkv_bits, qw_bits, kw_bits, pos, eps, theta = make_qk_inputs(wl)
    q_w, k_w = to_gpu_bf16(qw_bits), to_gpu_bf16(kw_bits)
    positions = torch.from_numpy(pos).cuda()
    plain = to_gpu_bf16(qkv_bits)
    timed = to_gpu_bf16(qkv_bits)
    mbn.qk_norm_rope_fwd(plain, q_w, k_w, positions, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                         eps=eps, theta=theta)
    a, b = events.new(), events.new()
    mbn.qk_norm_rope_fwd_timed(timed, q_w, k_w, positions, wl.n_q_heads, wl.n_kv_heads, a, b,
                               head_dim=wl.head_dim, eps=eps, theta=theta)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    assert events.ms(a, b) > 0.0


def test_timed_empty_input_records_nothing(events):
    """An empty input launches nothing and leaves the events unrecorded."""
    x = torch.empty(0, 4096, device="cuda", dtype=torch.bfloat16)
    w = torch.ones(4096, device="cuda", dtype=torch.bfloat16)
    a, b = events.new(), events.new()
    y = mbn.rmsnorm_fwd_timed(x, w, a, b)
    torch.cuda.synchronize()
    assert y.shape == (0, 4096)
