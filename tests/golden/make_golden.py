"""Write the oracle regression fixtures in this folder.

Calls only the oracle and the seeded input generators. The pages print no
worked numeric example of either operator, so these files are not pins: they
freeze the oracle's bits for a few tiny cases so that any later change to the
oracle's arithmetic shows up as a diff that has to be justified.

Run from the repository root:  python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import qk_norm_rope_fwd, rmsnorm_fwd  # noqa: E402
from workloads import random_bf16_bits  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def _hex(a):
    return " ".join(f"{int(v):04x}" for v in np.asarray(a).reshape(-1))


def rms_case():
    rng = np.random.default_rng(100)
    x = random_bf16_bits(rng, (4, 8))
    w = random_bf16_bits(rng, (8,), lo=0.5, hi=1.5)
    return x, w, 1e-6


def qk_case():
    rng = np.random.default_rng(101)
    t, hq, hk, d = 2, 2, 1, 8
    qkv = random_bf16_bits(rng, (t, (hq + 2 * hk) * d))
    q_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    k_w = random_bf16_bits(rng, (d,), lo=0.5, hi=1.5)
    pos = np.array([0, 7], dtype=np.int64)
    return qkv, q_w, k_w, pos, hq, hk, d, 1e-6, 1e6


def main():
    x, w, eps = rms_case()
    with open(os.path.join(HERE, "rmsnorm_4x8.txt"), "w") as f:
        f.write("# oracle RMSNorm, x[4,8] ~ N(0,1) seed 100, w ~ U(0.5,1.5), eps 1e-6; bf16 hex\n")
        f.write("x " + _hex(x) + "\n")
        f.write("w " + _hex(w) + "\n")
        f.write("y " + _hex(rmsnorm_fwd(x, w, eps)) + "\n")
    qkv, q_w, k_w, pos, hq, hk, d, eps, theta = qk_case()
    out = qk_norm_rope_fwd(qkv, q_w, k_w, pos, hq, hk, d, eps, theta)
    with open(os.path.join(HERE, "qk_norm_rope_t2_h2_1_d8.txt"), "w") as f:
        f.write("# oracle QK-norm+RoPE, T=2, 2 q + 1 k + 1 v heads, D=8, pos (0, 7), eps 1e-6, theta 1e6; bf16 hex\n")
        f.write("qkv " + _hex(qkv) + "\n")
        f.write("q_w " + _hex(q_w) + "\n")
        f.write("k_w " + _hex(k_w) + "\n")
        f.write("out " + _hex(out) + "\n")


if __name__ == "__main__":
    main()
