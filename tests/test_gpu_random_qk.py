"""Randomized GPU parity of the fused QK-norm + rotary kernel: a fixed-seed
draw of token count (across the one-step, two-step and looping launch shapes),
q and kv head counts, rotary dimension (16 ... 128), theta, positions and
storage type; every output (v heads untouched) against the fp64 oracle."""

import numpy as np
import pytest

from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import random_bf16_bits, random_f16_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import memory_bound_normalization_amd as mbn  # noqa: E402
from oracle import qk_norm_rope_fwd as o_qk  # noqa: E402


def _cases(n=40, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([1, 2, 5, 63, 256, 511, 512, 513, 1000, 1024, 1025, 2049, 3000]))
        n_q = int(rng.integers(0, 65))
        n_kv = int(rng.integers(0 if n_q else 1, 17))
        rot = int(rng.choice([16, 32, 48, 64, 96, 112, 128]))
        theta = float(rng.choice([1e4, 5e5, 1e6]))
        dtype = "f16" if rng.random() < 0.3 else "bf16"
        out.append((i, T, n_q, n_kv, rot, theta, dtype))
    return out


CASES = _cases()


@pytest.mark.parametrize("i,T,n_q,n_kv,rot,theta,dtype", CASES)
def test_random_qk(i, T, n_q, n_kv, rot, theta, dtype):
    label = f"case {i}: T={T} q={n_q} kv={n_kv} rot={rot} theta={theta:g} {dtype}"
    print(f"[random qk] {label}", flush=True)
    rng = np.random.default_rng(5000 + i)
    gen = random_f16_bits if dtype == "f16" else random_bf16_bits
    qkv = gen(rng, (T, (n_q + 2 * n_kv) * 128), scale=float(rng.choice([0.1, 1.0, 8.0])))
    q_w = gen(rng, (128,), lo=0.5, hi=1.5)
    k_w = gen(rng, (128,), lo=0.5, hi=1.5)
    pos = rng.integers(0, 1 << 20, T).astype(np.int64)
    g = to_gpu_bf16(qkv, dtype=dtype)
    mbn.qk_norm_rope_fwd(g, to_gpu_bf16(q_w, dtype=dtype), to_gpu_bf16(k_w, dtype=dtype),
                         torch.from_numpy(pos).cuda(), n_q, n_kv, 128, eps=1e-6, theta=theta,
                         rotary_dim=None if rot == 128 else rot)
    torch.cuda.synchronize()
    ref = o_qk(qkv, q_w, k_w, pos, n_q, n_kv, 128, 1e-6, theta, rotary_dim=rot, dtype=dtype)
    assert_parity(from_gpu_bf16(g), ref, label, dtype=dtype)
