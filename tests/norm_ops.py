"""One row-norm launch through the C ABI checked against the fp64 oracle, for
the GPU tests that reach launch-table entries ("rms", "add", "layer", "l2")."""

import numpy as np
import torch

import memory_bound_normalization_amd as mbn
from oracle import add_rmsnorm_fwd as o_add, l2norm_fwd as o_l2, layernorm_fwd as o_ln, rmsnorm_fwd as o_rms
from parity import assert_parity, from_gpu_bf16, to_gpu_bf16
from workloads import random_bf16_bits

TABLE_OPS = {"kRmsTable": "rms", "kAddRmsTable": "add", "kLayerTable": "layer", "kL2Table": "l2"}


def check_norm(op, M, N, seed, label):
    """Run `op` on seeded bf16 inputs of M x N and compare every output."""
    rng = np.random.default_rng(seed)
    x = random_bf16_bits(rng, (M, N))
    w = random_bf16_bits(rng, (N,), lo=0.5, hi=1.5)
    if op == "rms":
        y = mbn.rmsnorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), eps=1e-6)
        ref = o_rms(x, w, 1e-6)
    elif op == "layer":
        b = random_bf16_bits(rng, (N,), lo=-0.5, hi=0.5)
        y = mbn.layernorm_fwd(to_gpu_bf16(x), to_gpu_bf16(w), to_gpu_bf16(b), eps=1e-5)
        ref = o_ln(x, w, b, 1e-5)
    elif op == "l2":
        y = mbn.l2norm_fwd(to_gpu_bf16(x), eps=1e-12)
        ref = o_l2(x, 1e-12)
    else:
        r = random_bf16_bits(rng, (M, N))
        h, y = mbn.add_rmsnorm_fwd(to_gpu_bf16(x), to_gpu_bf16(r), to_gpu_bf16(w), eps=1e-6)
        rh, ref = o_add(x, r, w, 1e-6)
        torch.cuda.synchronize()
        assert np.array_equal(from_gpu_bf16(h), rh), f"{label}: h = bf16(x + r) not bit-exact"
    torch.cuda.synchronize()
    assert_parity(from_gpu_bf16(y), ref, label)
