"""Oracle drift guard: the oracle must keep reproducing its frozen tiny outputs.

The fixtures in tests/golden/ were written by tests/golden/make_golden.py,
which calls only the oracle. They are regression locks, not pins (the pages
print no worked example); a change here must name the reading that justifies it.
"""

import os

import numpy as np

from oracle import qk_norm_rope_fwd, rmsnorm_fwd

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            out[key] = np.array([int(v, 16) for v in vals], dtype=np.uint16)
    return out


def test_rmsnorm_golden():
    g = _load("rmsnorm_4x8.txt")
    y = rmsnorm_fwd(g["x"].reshape(4, 8), g["w"], 1e-6)
    assert np.array_equal(y.reshape(-1), g["y"])


def test_qk_golden():
    g = _load("qk_norm_rope_t2_h2_1_d8.txt")
    qkv = g["qkv"].reshape(2, 32)
    out = qk_norm_rope_fwd(qkv, g["q_w"], g["k_w"], np.array([0, 7]), 2, 1, 8, 1e-6, 1e6)
    assert np.array_equal(out.reshape(-1), g["out"])
