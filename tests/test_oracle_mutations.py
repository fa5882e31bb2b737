"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pins catch each one: a pin suite that a wrong oracle passes proves
nothing. Each mutation is one textual change in a temporary copy; the pin tests
then run in a subprocess and must fail on an assertion (not on an error)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_bf16.py", "test_oracle_rmsnorm.py", "test_oracle_qk.py", "test_oracle_norms.py",
        "test_oracle_f16.py"]
# the pin file that covers each oracle module (its dependents' pins are not needed to catch it)
PIN_FOR = {"bf16.py": "test_oracle_bf16.py", "rmsnorm.py": "test_oracle_rmsnorm.py",
           "qk_norm_rope.py": "test_oracle_qk.py", "norms.py": "test_oracle_norms.py"}

MUTATIONS = [
    ("rmsnorm.py", "ms = np.sum(x * x, axis=1) / n", "ms = np.sum(x * x, axis=1) / (n - 1 if n > 1 else 1)"),
    ("rmsnorm.py", "rstd = 1.0 / np.sqrt(ms + eps64)", "rstd = 1.0 / (np.sqrt(ms) + eps64)"),
    ("rmsnorm.py", "return (x * rstd[:, None]) * w[None, :]", "return (x * rstd[:, None])"),
    ("rmsnorm.py", "eps64 = float(np.float32(eps))", "eps64 = 0.0"),
    ("bf16.py", "qexp = np.maximum(e - 8, -133)", "qexp = np.maximum(e - 9, -133)"),
    ("bf16.py", "np.rint(", "np.floor("),
    ("bf16.py", "qexp = np.maximum(e - 8, -133)", "qexp = e - 8"),
    ("qk_norm_rope.py", "a * c - b * s, b * c + a * s", "a * c + b * s, b * c - a * s"),
    ("qk_norm_rope.py", "(-(2.0 * i) / head_dim)", "(-(1.0 * i) / head_dim)"),
    ("qk_norm_rope.py", "a = u[..., :half]", "a = u[..., 0::2]"),
    ("qk_norm_rope.py", "b = u[..., half:]", "b = u[..., 1::2]"),
    ("qk_norm_rope.py", "np.tile(q_w, (n_q_heads, 1)), np.tile(k_w, (n_kv_heads, 1))",
     "np.tile(k_w, (n_q_heads, 1)), np.tile(q_w, (n_kv_heads, 1))"),
    ("qk_norm_rope.py", "ms = np.mean(x * x, axis=-1)", "ms = np.mean(x * x)"),
    ("qk_norm_rope.py", "rstd = 1.0 / np.sqrt(ms + eps64)", "rstd = 1.0 / np.sqrt(ms)"),
    ("qk_norm_rope.py", "rotated = rope_rotate_neox(u[..., :rot], pos[:, None], theta64)",
     "rotated = rope_rotate_neox(u, pos[:, None], theta64)[..., :rot]"),
    ("norms.py", "return h_bits, rmsnorm_fwd(h_bits, w_bits, eps, dtype)",
     "return h_bits, rmsnorm_fwd(x_bits, w_bits, eps, dtype)"),
    ("norms.py", "h_bits = narrow(x + r, dtype)", "h_bits = narrow(x + r * 0.5, dtype)"),
    ("norms.py", "var = np.sum(d * d, axis=1) / n", "var = np.sum(d * d, axis=1) / max(n - 1, 1)"),
    ("norms.py", "return d * rstd[:, None] * w[None, :] + b[None, :]", "return d * rstd[:, None] * w[None, :]"),
    ("norms.py", "d = x - mu[:, None]", "d = x"),
    ("norms.py", "rstd = 1.0 / np.sqrt(var + eps64)", "rstd = 1.0 / (np.sqrt(var) + eps64)"),
    ("norms.py", "return x / np.maximum(nrm, eps64)[:, None]", "return x / (nrm + eps64)[:, None]"),
    ("norms.py", "nrm = np.sqrt(np.sum(x * x, axis=1))", "nrm = np.sum(np.abs(x), axis=1)"),
    ("bf16.py", "qexp = np.maximum(e - 11, -24)", "qexp = np.maximum(e - 12, -24)", "test_oracle_f16.py"),
    ("bf16.py", "qexp = np.maximum(e - 11, -24)", "qexp = np.maximum(e - 11, -25)", "test_oracle_f16.py"),
    ("bf16.py", "_F16_NAN = np.uint16(0x7E00)", "_F16_NAN = np.uint16(0x7C00)", "test_oracle_f16.py"),
    ("bf16.py", "return b.view(np.float16).astype(np.float64)", "return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)", "test_oracle_f16.py"),
]


@pytest.mark.parametrize("mut", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_pins_catch_mutation(tmp_path, mut):
    fname, old, new = mut[:3]
    pin = mut[3] if len(mut) > 3 else PIN_FOR[fname]
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d, ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in PINS + ["exact.py", "conftest.py"]:
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    target = tmp_path / "oracle" / fname
    src = target.read_text()
    assert old in src, f"mutation site vanished from oracle/{fname}: {old!r}"
    target.write_text(src.replace(old, new))
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", f"tests/{pin}"],
        cwd=tmp_path, capture_output=True, text=True, timeout=600,
    )
    assert res.returncode == 1 and "FAILED" in res.stdout, res.stdout[-2000:]
