"""One row-norm launch through the C ABI checked against the fp64 oracle, for
the GPU tests that reach launch-table entries ("rms", "add", "layer", "l2")."""

import numpy as np
import torch

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import random_bf16_bits, random_f16_bits

TABLE_OPS = {"kRmsTable": "rms", "kAddRmsTable": "add", "kLayerTable": "layer", "kL2Table": "l2"}


def check_norm(op, M, N, seed, label, dtype="bf16"):
    """Run `op` on seeded inputs of M x N (bf16 or f16 storage) and compare
    every output."""
    rng = np.random.default_rng(seed)
    gen = random_f16_bits if dtype == "f16" else random_bf16_bits

    def up(bits):
        return to_gpu_bf16(bits, dtype=dtype)

    x = gen(rng, (M, N))
    w = gen(rng, (N,), lo=0.5, hi=1.5)
    if op == "rms":
        y = mbn.rmsnorm_fwd(up(x), up(w), eps=1e-6)
        ref = o_rms(x, w, 1e-6, dtype=dtype)
    elif op == "layer":
        b = gen(rng, (N,), lo=-0.5, hi=0.5)
        y = mbn.layernorm_fwd(up(x), up(w), up(b), eps=1e-5)
        ref = o_ln(x, w, b, 1e-5, dtype=dtype)
    elif op == "l2":
        y = mbn.l2norm_fwd(up(x), eps=1e-12)
        ref = o_l2(x, 1e-12, dtype=dtype)
    else:
        r = gen(rng, (M, N))
        h, y = mbn.add_rmsnorm_fwd(up(x), up(r), up(w), eps=1e-6)
        rh, ref = o_add(x, r, w, 1e-6, dtype=dtype)
        torch.cuda.synchronize()
        assert np.array_equal(from_gpu_bf16(h), rh), f"{label}: h = round(x + r) not bit-exact"
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, label, dtype=dtype)
