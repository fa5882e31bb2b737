"""GPU parity of qk_norm_rope_fwd (HIP, through the C ABI) against the fp64 oracle.

Every output of every case is compared; the v heads must keep their bits.
"""

import numpy as np
import pytest

import memory_bound_normalization_amd as mbn
from oracle import qk_norm_rope_fwd as oracle_qk
from parity import assert_parity, assert_parity_rows, from_gpu_bf16, to_gpu_bf16
from workloads import QK_WORKLOADS, make_qk_inputs, random_bf16_bits, random_f16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
D = 128


def _run(qkv_bits, q_w_bits, k_w_bits, pos, hq, hk, eps, theta, rotary_dim=None):
    qkv = to_gpu_bf16(qkv_bits)
    q_w = to_gpu_bf16(q_w_bits)
    k_w = to_gpu_bf16(k_w_bits)
    p = torch.from_numpy(np.asarray(pos, dtype=np.int64)).cuda()
    mbn.qk_norm_rope_fwd(qkv, q_w, k_w, p, hq, hk, D, eps=eps, theta=theta, rotary_dim=rotary_dim)
    torch.cuda.synchronize()
    return from_gpu_bf16(qkv)


def _check(T, hq, hk, pos=None, eps=1e-6, theta=1e6, seed=0, scale=1.0):
    print(f"[qk] T={T} hq={hq} hk={hk} eps={eps} theta={theta} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    qkv = random_bf16_bits(rng, (T, (hq + 2 * hk) * D), scale=scale)
    q_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    if pos is None:
        pos = np.arange(T, dtype=np.int64)
    got = _run(qkv, q_w, k_w, pos, hq, hk, eps, theta)
    ref = oracle_qk(qkv, q_w, k_w, pos, hq, hk, D, eps, theta)
    nk = (hq + hk) * D
    assert np.array_equal(got[:, nk:], qkv[:, nk:]), "v heads changed"
    assert_parity(got, ref, f"T={T} hq={hq} hk={hk}")


def test_workload():
    wl = QK_WORKLOADS["qk_256"]
    print("[qk] workload qk_256", flush=True)
    qkv, q_w, k_w, pos, eps, theta = make_qk_inputs(wl)
    got = _run(qkv, q_w, k_w, pos, wl.n_q_heads, wl.n_kv_heads, eps, theta)
    ref = oracle_qk(qkv, q_w, k_w, pos, wl.n_q_heads, wl.n_kv_heads, D, eps, theta)
    assert np.array_equal(got[:, 5120:], qkv[:, 5120:])
    assert_parity(got, ref, "qk_256")
    again = _run(qkv, q_w, k_w, pos, wl.n_q_heads, wl.n_kv_heads, eps, theta)
    assert np.array_equal(got, again), "not deterministic"


@pytest.mark.parametrize("hq,hk", [(1, 0), (0, 1), (3, 1), (5, 2), (4, 4), (32, 8), (64, 8), (2, 1), (60, 9)])
def test_head_counts(hq, hk):
    _check(19, hq, hk, seed=hq * 100 + hk)


@pytest.mark.parametrize("T", [1, 2, 255, 257, 1000, 1024, 1025, 3000])
def test_token_counts(T):
    _check(T, 8, 2, seed=T)


def test_many_tokens_few_and_many_heads():
    _check(2048, 2, 1, seed=16, pos=np.arange(2048) * 3)
    _check(1500, 64, 8, seed=17)


def test_positions():
    rng = np.random.default_rng(9)
    pos = np.array([0, 1, 7, 255, 4096, 65535, 1 << 20, 1 << 24, -1, -300, 123456789, 3], dtype=np.int64)
    _check(len(pos), 4, 2, pos=pos, seed=10)
    _check(64, 4, 2, pos=rng.integers(0, 1 << 17, 64), seed=11)


@pytest.mark.parametrize("theta", [10000.0, 1e6, 5e5, 2.0])
def test_theta(theta):
    _check(33, 4, 2, theta=theta, seed=12, pos=np.arange(33) * 97)


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.25])
def test_eps(eps):
    _check(17, 4, 2, eps=eps, seed=13)


@pytest.mark.parametrize("scale", [1e-3, 50.0])
def test_scales(scale):
    _check(17, 4, 2, scale=scale, seed=14)


def test_special_values():
    rng = np.random.default_rng(15)
    T, hq, hk = 4, 2, 1
    qkv = random_bf16_bits(rng, (T, (hq + 2 * hk) * D))
    q_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    qkv[0, :D] = 0  # zero head
    qkv[1, D + 5] = 0x7FC0  # NaN in a head
    qkv[2, 2 * D + 3] = 0x7F80  # inf in the k head
    pos = np.arange(T)
    got = _run(qkv, q_w, k_w, pos, hq, hk, 1e-6, 1e6)
    ref = oracle_qk(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6)
    assert np.array_equal(got[:, 3 * D :], qkv[:, 3 * D :])
    assert_parity(got, ref, "special values")


def test_empty_and_errors():
    qkv = torch.zeros(0, 3 * D * 2, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(0, dtype=torch.int64, device="cuda")
    mbn.qk_norm_rope_fwd(qkv, w, w, p, 4, 1, D)
    qkv = torch.zeros(2, 6 * 64, dtype=torch.bfloat16, device="cuda")
    w64 = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(mbn.MbnError) as e:
        mbn.qk_norm_rope_fwd(qkv, w64, w64, p, 4, 1, 64)
    assert e.value.status == mbn.MBN_EUNSUPPORTED


@pytest.mark.parametrize("rot", [16, 32, 48, 64, 96, 112, 128])
@pytest.mark.parametrize("T", [7, 1500])
def test_partial_rotary(rot, T):
    print(f"[qk] partial rotary_dim={rot} T={T}", flush=True)
    rng = np.random.default_rng(rot * 10 + T)
    hq, hk = 5, 2
    qkv = random_bf16_bits(rng, (T, (hq + 2 * hk) * D))
    q_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    pos = rng.integers(0, 100000, size=T)
    got = _run(qkv, q_w, k_w, pos, hq, hk, 1e-6, 1e6, rotary_dim=rot)
    ref = oracle_qk(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6, rotary_dim=rot)
    nk = (hq + hk) * D
    assert np.array_equal(got[:, nk:], qkv[:, nk:]), "v heads changed"
    assert_parity(got, ref, f"partial rot={rot} T={T}")
    if rot == 128:
        full = _run(qkv, q_w, k_w, pos, hq, hk, 1e-6, 1e6)
        assert np.array_equal(full, got), "rotary_dim = head_dim differs from the full-rotary entry point"


def test_many_tokens():
    """65536 tokens (the 4-wave looping schedule): every output against the oracle."""
    T, hq, hk = 65536, 32, 8
    print(f"[qk] large T={T}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(9)
    qkv = torch.randn(T, (hq + 2 * hk) * D, device="cuda", generator=g).to(torch.bfloat16)
    q_w = (torch.rand(D, device="cuda", generator=g) + 0.5).to(torch.bfloat16)
    k_w = (torch.rand(D, device="cuda", generator=g) + 0.5).to(torch.bfloat16)
    pos = torch.arange(T, device="cuda", dtype=torch.int64)
    before = from_gpu_bf16(qkv)
    mbn.qk_norm_rope_fwd(qkv, q_w, k_w, pos, hq, hk, D, eps=1e-6, theta=1e6)
    torch.cuda.synchronize()
    after = from_gpu_bf16(qkv)
    qwb, kwb = from_gpu_bf16(q_w), from_gpu_bf16(k_w)
    toks = np.arange(T)
    n = assert_parity_rows(after, lambda lo, hi: oracle_qk(before[lo:hi], qwb, kwb, toks[lo:hi], hq, hk, D,
                                                          1e-6, 1e6), "large T", block=1024)
    assert n == after.size
    assert np.array_equal(after[:, (hq + hk) * D:], before[:, (hq + hk) * D:])


# Launch shapes that keep several head rows of a wave in flight: 5 waves of two
# steps (513 ... 1024 tokens), 4 waves of three (more tokens), and more heads
# than 48, where a wave loads a second group of rows after the first three.
@pytest.mark.parametrize("T,hq,hk,rot,dtype", [
    (700, 32, 8, 128, "bf16"),  # 5 waves x 2 steps
    (700, 30, 3, 64, "f16"),  # 33 heads: the last step of one wave holds 1 live head
    (1500, 32, 8, 48, "bf16"),  # 4 waves x 3 steps, partial rotary
    (1500, 70, 9, 128, "bf16"),  # 79 heads: 5 steps per wave, two load groups, ragged
    (2500, 61, 2, 112, "f16"),  # 63 heads, partial rotary
    (9000, 32, 8, 128, "bf16"),
])
def test_rows_in_flight(T, hq, hk, rot, dtype):
    label = f"T={T} hq={hq} hk={hk} rot={rot} {dtype}"
    print(f"[qk rows in flight] {label}", flush=True)
    rng = np.random.default_rng(T + 7 * hq + hk)
    gen = random_f16_bits if dtype == "f16" else random_bf16_bits
    qkv = gen(rng, (T, (hq + 2 * hk) * D))
    q_w = gen(rng, (D,), lo=0.5, hi=1.5)
    k_w = gen(rng, (D,), lo=0.5, hi=1.5)
    pos = rng.integers(0, 1 << 20, T).astype(np.int64)
    g = to_gpu_bf16(qkv, dtype=dtype)
    mbn.qk_norm_rope_fwd(g, to_gpu_bf16(q_w, dtype=dtype), to_gpu_bf16(k_w, dtype=dtype),
                         torch.from_numpy(pos).cuda(), hq, hk, D, eps=1e-6, theta=1e6,
                         rotary_dim=None if rot == D else rot)
    torch.cuda.synchronize()
    got = from_gpu_bf16(g)
    nk = (hq + hk) * D
    assert np.array_equal(got[:, nk:], qkv[:, nk:]), "v heads changed"
    ref = oracle_qk(qkv, q_w, k_w, pos, hq, hk, D, 1e-6, 1e6, rotary_dim=rot, dtype=dtype)
    assert_parity(got, ref, label, dtype=dtype)


@pytest.mark.parametrize("T", [7, 700, 1500])
@pytest.mark.parametrize("hq,hk", [(0, 5), (9, 0)])
def test_null_weight_of_absent_heads(T, hq, hk):
    """The C ABI takes a null q_w when there are no q heads (null k_w when
    there are no kv heads); the kernel must not read it."""
    print(f"[qk null weight] T={T} hq={hq} hk={hk}", flush=True)
    rng = np.random.default_rng(31 * T + hq)
    qkv = random_bf16_bits(rng, (T, (hq + 2 * hk) * D))
    w = random_bf16_bits(rng, (D,), lo=0.5, hi=1.5)
    pos = rng.integers(0, 1 << 20, T).astype(np.int64)
    g = to_gpu_bf16(qkv)
    wg = to_gpu_bf16(w)
    p = torch.from_numpy(pos).cuda()
    q_ptr = wg.data_ptr() if hq else None
    k_ptr = wg.data_ptr() if hk else None
    stream = torch.cuda.current_stream().cuda_stream
    rc = mbn.lib().qk_norm_rope_fwd(g.data_ptr(), q_ptr, k_ptr, p.data_ptr(), T, hq, hk, D, 1e-6, 1e6, stream)
    assert rc == mbn.MBN_OK
    torch.cuda.synchronize()
    ref = oracle_qk(qkv, w, w, pos, hq, hk, D, 1e-6, 1e6)
    assert_parity(from_gpu_bf16(g), ref, f"null weight T={T} hq={hq} hk={hk}")
