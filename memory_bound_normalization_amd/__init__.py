"""Python binding of libmbn.so: RMSNorm family and fused QK-norm + rotary on MI355X.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels. PyTorch supplies device memory and streams. There is no CPU
fallback; importing works without a GPU, but any call raises if the library is
not built or the tensors are not on the GPU.

Functions with the C names take torch tensors, all bfloat16 or all float16
(float16 tensors are routed to the ``*_f16`` entry points):

* ``rmsnorm_fwd(x, w, y=None, eps=1e-6, stream=None)`` -- x [..., N] bf16,
  w [N] bf16; returns y (allocated like x when not given; ``y is x`` runs in
  place).
* ``add_rmsnorm_fwd(x, r, w, h=None, y=None, eps=1e-6, stream=None)`` --
  h = x + r (bf16), y = RMSNorm(h) * w; returns (h, y).
* ``layernorm_fwd(x, w, b, y=None, eps=1e-5, stream=None)``.
* ``l2norm_fwd(x, y=None, eps=1e-12, stream=None)``.
* ``qk_norm_rope_fwd(qkv, q_w, k_w, positions, n_q_heads, n_kv_heads,
  head_dim=128, eps=1e-6, theta=1e6, stream=None)`` -- modifies qkv in place
  and returns it.
* ``rmsnorm_fwd_timed(x, w, start_event, stop_event, y=None, eps=1e-6,
  stream=None)`` and ``qk_norm_rope_fwd_timed(qkv, q_w, k_w, positions,
  n_q_heads, n_kv_heads, start_event, stop_event, ...)`` -- bf16 only; the
  same calls, with the kernels' own start and end recorded into two
  caller-created hipEvent_t handles (ints or ctypes.c_void_p).
* ``mbn_strerror(status)``.

``lib()`` returns the raw ctypes handle (C signatures of include/mbn.h).
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "MBN_OK",
    "MBN_EINVAL",
    "MBN_EUNSUPPORTED",
    "MBN_EHIP",
    "MBN_RMSNORM_MAX_N",
    "MBN_QK_HEAD_DIM",
    "MbnError",
    "add_rmsnorm_fwd",
    "l2norm_fwd",
    "layernorm_fwd",
    "lib",
    "lib_path",
    "mbn_strerror",
    "qk_norm_rope_fwd",
    "qk_norm_rope_fwd_timed",
    "rmsnorm_fwd",
    "rmsnorm_fwd_timed",
]

MBN_OK = 0
MBN_EINVAL = 1
MBN_EUNSUPPORTED = 2
MBN_EHIP = 3
MBN_RMSNORM_MAX_N = 65536
MBN_QK_HEAD_DIM = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libmbn.so")


class MbnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({mbn_strerror(status)})")


def lib() -> ctypes.CDLL:
    """Load libmbn.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m memory_bound_normalization_amd.build`"
            )
        h = ctypes.CDLL(path)
        vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        h.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, f32, vp]
        h.rmsnorm_fwd.restype = ctypes.c_int
        h.add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, vp]
        h.add_rmsnorm_fwd.restype = ctypes.c_int
        h.layernorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, vp]
        h.layernorm_fwd.restype = ctypes.c_int
        h.l2norm_fwd.argtypes = [vp, vp, i64, i64, f32, vp]
        h.l2norm_fwd.restype = ctypes.c_int
        h.qk_norm_rope_fwd.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, f32, f32, vp]
        h.qk_norm_rope_fwd.restype = ctypes.c_int
        h.qk_norm_rope_partial_fwd.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, i32, f32, f32, vp]
        h.qk_norm_rope_partial_fwd.restype = ctypes.c_int
        for name in ("rmsnorm_fwd", "add_rmsnorm_fwd", "layernorm_fwd", "l2norm_fwd",
                     "qk_norm_rope_partial_fwd"):
            f16 = getattr(h, name + "_f16")
            f16.argtypes = getattr(h, name).argtypes
            f16.restype = ctypes.c_int
        h.rmsnorm_fwd_timed.argtypes = h.rmsnorm_fwd.argtypes + [vp, vp]
        h.rmsnorm_fwd_timed.restype = ctypes.c_int
        h.qk_norm_rope_fwd_timed.argtypes = h.qk_norm_rope_fwd.argtypes + [vp, vp]
        h.qk_norm_rope_fwd_timed.restype = ctypes.c_int
        h.mbn_strerror.argtypes = [ctypes.c_int]
        h.mbn_strerror.restype = ctypes.c_char_p
        _LIB = h
    return _LIB


def mbn_strerror(status: int) -> str:
    try:
        return lib().mbn_strerror(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def _stream_handle(stream, device):
    import torch

    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check_bf16_cuda(name, t, dtype=None):
    """Check a 16-bit GPU tensor; ``dtype`` (if given) is the call's storage type."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    want = (torch.bfloat16, torch.float16) if dtype is None else (dtype,)
    if t.dtype not in want:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in want)}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fn(name, dtype):
    """The C entry point for the storage type of the call."""
    import torch

    return getattr(lib(), name + "_f16" if dtype == torch.float16 else name)


def rmsnorm_fwd(x, w, y=None, eps: float = 1e-6, stream=None):
    """y = x * rsqrt(mean(x^2, -1) + eps) * w over the last dim of bf16 x."""
    import torch

    _check_bf16_cuda("x", x)
    _check_bf16_cuda("w", w, x.dtype)
    n = x.shape[-1] if x.dim() > 0 else 0
    if w.dim() != 1 or w.shape[0] != n:
        raise ValueError(f"w must have shape [{n}], got {tuple(w.shape)}")
    if y is None:
        y = torch.empty_like(x)
    else:
        _check_bf16_cuda("y", y, x.dtype)
        if y.shape != x.shape:
            raise ValueError("y must have the shape of x")
    m = x.numel() // n if n else 0
    rc = _fn("rmsnorm_fwd", x.dtype)(
        x.data_ptr(), w.data_ptr(), y.data_ptr(), m, n, float(eps), _stream_handle(stream, x.device)
    )
    if rc != MBN_OK:
        raise MbnError(rc, "rmsnorm_fwd")
    return y


def _event_handle(e):
    return e.value if isinstance(e, ctypes.c_void_p) else int(e)


def rmsnorm_fwd_timed(x, w, start_event, stop_event, y=None, eps: float = 1e-6, stream=None):
    """rmsnorm_fwd (bf16) with the kernels' own start / end recorded in two hipEvent_t."""
    import torch

    _check_bf16_cuda("x", x, torch.bfloat16)
    m, n = _rows_of(x)
    _check_vec("w", w, n, x.dtype)
    y = _out_like(x, y, "y")
    rc = lib().rmsnorm_fwd_timed(
        x.data_ptr(), w.data_ptr(), y.data_ptr(), m, n, float(eps), _stream_handle(stream, x.device),
        _event_handle(start_event), _event_handle(stop_event),
    )
    if rc != MBN_OK:
        raise MbnError(rc, "rmsnorm_fwd_timed")
    return y


def _rows_of(x, what="x"):
    n = x.shape[-1] if x.dim() > 0 else 0
    return (x.numel() // n if n else 0), n


def _out_like(x, y, name):
    import torch

    if y is None:
        return torch.empty_like(x)
    _check_bf16_cuda(name, y, x.dtype)
    if y.shape != x.shape:
        raise ValueError(f"{name} must have the shape of x")
    return y


def _check_vec(name, v, n, dtype):
    _check_bf16_cuda(name, v, dtype)
    if v.dim() != 1 or v.shape[0] != n:
        raise ValueError(f"{name} must have shape [{n}], got {tuple(v.shape)}")


def add_rmsnorm_fwd(x, r, w, h=None, y=None, eps: float = 1e-6, stream=None):
    """h = bf16(x + r); y = h * rsqrt(mean(h^2, -1) + eps) * w. Returns (h, y)."""
    _check_bf16_cuda("x", x)
    _check_bf16_cuda("r", r, x.dtype)
    if r.shape != x.shape:
        raise ValueError("r must have the shape of x")
    m, n = _rows_of(x)
    _check_vec("w", w, n, x.dtype)
    h = _out_like(x, h, "h")
    y = _out_like(x, y, "y")
    rc = _fn("add_rmsnorm_fwd", x.dtype)(x.data_ptr(), r.data_ptr(), w.data_ptr(), h.data_ptr(), y.data_ptr(),
                               m, n, float(eps), _stream_handle(stream, x.device))
    if rc != MBN_OK:
        raise MbnError(rc, "add_rmsnorm_fwd")
    return h, y


def layernorm_fwd(x, w, b, y=None, eps: float = 1e-5, stream=None):
    """y = (x - mean) * rsqrt(var + eps) * w + b over the last dim of bf16 x."""
    _check_bf16_cuda("x", x)
    m, n = _rows_of(x)
    _check_vec("w", w, n, x.dtype)
    _check_vec("b", b, n, x.dtype)
    y = _out_like(x, y, "y")
    rc = _fn("layernorm_fwd", x.dtype)(x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr(), m, n,
                             float(eps), _stream_handle(stream, x.device))
    if rc != MBN_OK:
        raise MbnError(rc, "layernorm_fwd")
    return y


def l2norm_fwd(x, y=None, eps: float = 1e-12, stream=None):
    """y = x / max(||x||_2, eps) over the last dim of bf16 x."""
    _check_bf16_cuda("x", x)
    m, n = _rows_of(x)
    y = _out_like(x, y, "y")
    rc = _fn("l2norm_fwd", x.dtype)(x.data_ptr(), y.data_ptr(), m, n, float(eps), _stream_handle(stream, x.device))
    if rc != MBN_OK:
        raise MbnError(rc, "l2norm_fwd")
    return y


def qk_norm_rope_fwd(
    qkv, q_w, k_w, positions, n_q_heads: int, n_kv_heads: int, head_dim: int = MBN_QK_HEAD_DIM,
    eps: float = 1e-6, theta: float = 1e6, stream=None, rotary_dim: int | None = None,
):
    """In-place per-head RMSNorm (q_w / k_w) + rotate-half RoPE on qkv [T, (Hq+2Hkv)*D].

    ``rotary_dim`` (default: head_dim) rotates only the first rotary_dim values
    of each head (qk_norm_rope_partial_fwd); the rest are normalized only.
    """
    import torch

    _check_bf16_cuda("qkv", qkv)
    _check_bf16_cuda("q_w", q_w, qkv.dtype)
    _check_bf16_cuda("k_w", k_w, qkv.dtype)
    if positions.dtype != torch.int64 or not positions.is_cuda or not positions.is_contiguous():
        raise TypeError("positions must be a contiguous int64 GPU tensor")
    t = qkv.shape[0] if qkv.dim() else 0
    if qkv.dim() != 2 or qkv.shape[1] != (n_q_heads + 2 * n_kv_heads) * head_dim:
        raise ValueError("qkv must have shape [T, (n_q_heads + 2 * n_kv_heads) * head_dim]")
    if positions.numel() != t:
        raise ValueError("positions must have T entries")
    if rotary_dim is None and qkv.dtype == torch.bfloat16:
        rc = lib().qk_norm_rope_fwd(
            qkv.data_ptr(), q_w.data_ptr(), k_w.data_ptr(), positions.data_ptr(), t,
            int(n_q_heads), int(n_kv_heads), int(head_dim), float(eps), float(theta),
            _stream_handle(stream, qkv.device),
        )
        where = "qk_norm_rope_fwd"
    else:
        rot = head_dim if rotary_dim is None else rotary_dim
        rc = _fn("qk_norm_rope_partial_fwd", qkv.dtype)(
            qkv.data_ptr(), q_w.data_ptr(), k_w.data_ptr(), positions.data_ptr(), t,
            int(n_q_heads), int(n_kv_heads), int(head_dim), int(rot), float(eps),
            float(theta), _stream_handle(stream, qkv.device),
        )
        where = "qk_norm_rope_partial_fwd" + ("_f16" if qkv.dtype == torch.float16 else "")
    if rc != MBN_OK:
        raise MbnError(rc, where)
    return qkv


def qk_norm_rope_fwd_timed(
    qkv, q_w, k_w, positions, n_q_heads: int, n_kv_heads: int, start_event, stop_event,
    head_dim: int = MBN_QK_HEAD_DIM, eps: float = 1e-6, theta: float = 1e6, stream=None,
):
    """qk_norm_rope_fwd (bf16, full rotary) with the kernels' own start / end in two hipEvent_t."""
    import torch

    _check_bf16_cuda("qkv", qkv, torch.bfloat16)
    _check_bf16_cuda("q_w", q_w, qkv.dtype)
    _check_bf16_cuda("k_w", k_w, qkv.dtype)
    if positions.dtype != torch.int64 or not positions.is_cuda or not positions.is_contiguous():
        raise TypeError("positions must be a contiguous int64 GPU tensor")
    t = qkv.shape[0] if qkv.dim() else 0
    if qkv.dim() != 2 or qkv.shape[1] != (n_q_heads + 2 * n_kv_heads) * head_dim:
        raise ValueError("qkv must have shape [T, (n_q_heads + 2 * n_kv_heads) * head_dim]")
    if positions.numel() != t:
        raise ValueError("positions must have T entries")
    rc = lib().qk_norm_rope_fwd_timed(
        qkv.data_ptr(), q_w.data_ptr(), k_w.data_ptr(), positions.data_ptr(), t,
        int(n_q_heads), int(n_kv_heads), int(head_dim), float(eps), float(theta),
        _stream_handle(stream, qkv.device), _event_handle(start_event), _event_handle(stop_event),
    )
    if rc != MBN_OK:
        raise MbnError(rc, "qk_norm_rope_fwd_timed")
    return qkv
