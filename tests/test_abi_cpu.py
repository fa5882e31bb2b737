"""C-ABI checks that need no GPU: the library builds, loads, exports every
symbol include/mbn.h declares, and rejects invalid arguments on the host before
any HIP call (every case below is invalid by construction, so no kernel is ever
launched and no pointer is dereferenced)."""

import ctypes
import os
import re

import pytest

import memory_bound_normalization_amd as mbn
from memory_bound_normalization_amd import build as mbn_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbn.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mbn.lib_path()):
        mbn_build.build()
    return mbn.lib()


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MBN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def _header_constants():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(MBN_\w+)\s+(\d+)", text)}


def test_header_declares_the_entry_points():
    assert set(_declared_functions()) == {
        "rmsnorm_fwd", "add_rmsnorm_fwd", "layernorm_fwd", "l2norm_fwd", "qk_norm_rope_fwd",
        "qk_norm_rope_partial_fwd", "rmsnorm_fwd_f16", "add_rmsnorm_fwd_f16", "layernorm_fwd_f16",
        "l2norm_fwd_f16", "qk_norm_rope_partial_fwd_f16", "rmsnorm_fwd_timed",
        "qk_norm_rope_fwd_timed", "mbn_strerror"}


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_python_constants_match_header():
    c = _header_constants()
    for name in ("MBN_OK", "MBN_EINVAL", "MBN_EUNSUPPORTED", "MBN_EHIP", "MBN_RMSNORM_MAX_N", "MBN_QK_HEAD_DIM"):
        assert getattr(mbn, name) == c[name], name


def test_strerror(lib):
    for s in range(5):
        assert isinstance(mbn.mbn_strerror(s), str) and mbn.mbn_strerror(s)
    assert mbn.mbn_strerror(0) == "success"


def test_build_command_targets_gfx950_without_fast_math():
    cmd = mbn_build.compile_command("/tmp/x.so")
    assert "--offload-arch=gfx950" in cmd
    assert "-packed-fp32-ops" in cmd
    assert not any("fast-math" in a or a == "-ffast-math" for a in cmd)


def rms(lib, x=FAKE, w=FAKE + 0x10000000, y=FAKE + 0x20000000, M=4, N=64, eps=1e-6):
    return lib.rmsnorm_fwd(x, w, y, M, N, eps, None)


@pytest.mark.parametrize(
    "kw, status",
    [
        (dict(M=-1), mbn.MBN_EINVAL),
        (dict(N=0), mbn.MBN_EINVAL),
        (dict(N=-8), mbn.MBN_EINVAL),
        (dict(eps=-1e-6), mbn.MBN_EINVAL),
        (dict(eps=float("nan")), mbn.MBN_EINVAL),
        (dict(eps=float("inf")), mbn.MBN_EINVAL),
        (dict(x=None), mbn.MBN_EINVAL),
        (dict(w=None), mbn.MBN_EINVAL),
        (dict(y=None), mbn.MBN_EINVAL),
        (dict(N=65544), mbn.MBN_EUNSUPPORTED),
        (dict(N=65537), mbn.MBN_EUNSUPPORTED),
        (dict(M=1 << 31), mbn.MBN_EUNSUPPORTED),
        (dict(x=FAKE + 1), mbn.MBN_EUNSUPPORTED),  # odd address: not an element boundary
        (dict(w=FAKE + 0x10000001), mbn.MBN_EUNSUPPORTED),
        (dict(y=FAKE + 0x20000003), mbn.MBN_EUNSUPPORTED),
        (dict(N=12, x=FAKE + 3), mbn.MBN_EUNSUPPORTED),  # any-width path, odd x
        (dict(y=FAKE + 16), mbn.MBN_EINVAL),  # partial overlap of y with x
        (dict(w=FAKE + 0x20000000 + 64), mbn.MBN_EINVAL),  # w inside y
    ],
)
def test_rmsnorm_rejects(lib, kw, status):
    assert rms(lib, **kw) == status


def test_rmsnorm_empty_is_a_noop(lib):
    assert lib.rmsnorm_fwd(None, None, None, 0, 64, 1e-6, None) == mbn.MBN_OK


def qk(lib, qkv=FAKE, q_w=FAKE + 0x10000000, k_w=FAKE + 0x10001000, pos=FAKE + 0x10002000,
       T=4, hq=4, hk=2, d=128, eps=1e-6, theta=1e6):
    return lib.qk_norm_rope_fwd(qkv, q_w, k_w, pos, T, hq, hk, d, eps, theta, None)


@pytest.mark.parametrize(
    "kw, status",
    [
        (dict(T=-1), mbn.MBN_EINVAL),
        (dict(hq=-1), mbn.MBN_EINVAL),
        (dict(hk=-2), mbn.MBN_EINVAL),
        (dict(d=0), mbn.MBN_EINVAL),
        (dict(d=127), mbn.MBN_EINVAL),
        (dict(eps=-1.0), mbn.MBN_EINVAL),
        (dict(eps=float("nan")), mbn.MBN_EINVAL),
        (dict(theta=0.0), mbn.MBN_EINVAL),
        (dict(theta=-10.0), mbn.MBN_EINVAL),
        (dict(theta=float("inf")), mbn.MBN_EINVAL),
        (dict(qkv=None), mbn.MBN_EINVAL),
        (dict(pos=None), mbn.MBN_EINVAL),
        (dict(q_w=None), mbn.MBN_EINVAL),
        (dict(k_w=None), mbn.MBN_EINVAL),
        (dict(d=64), mbn.MBN_EUNSUPPORTED),
        (dict(d=256), mbn.MBN_EUNSUPPORTED),
        (dict(qkv=FAKE + 8), mbn.MBN_EUNSUPPORTED),
        (dict(q_w=FAKE + 0x10000002), mbn.MBN_EUNSUPPORTED),
        (dict(pos=FAKE + 0x10002004), mbn.MBN_EUNSUPPORTED),
        (dict(q_w=FAKE + 256), mbn.MBN_EINVAL),  # weight inside the q/k span
        (dict(pos=FAKE + 1024), mbn.MBN_EINVAL),
    ],
)
def test_qk_rejects(lib, kw, status):
    assert qk(lib, **kw) == status


def test_qk_empty_is_a_noop(lib):
    assert qk(lib, qkv=None, q_w=None, k_w=None, pos=None, T=0) == mbn.MBN_OK
    assert qk(lib, hq=0, hk=0) == mbn.MBN_OK


def test_python_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.ones(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        mbn.rmsnorm_fwd(x, w)
    with pytest.raises(TypeError):
        mbn.rmsnorm_fwd(x.float(), w)


B = 0x10000000  # spacing of the fake buffers below


@pytest.mark.parametrize(
    "kw, status",
    [
        (dict(M=-1), mbn.MBN_EINVAL),
        (dict(eps=float("nan")), mbn.MBN_EINVAL),
        (dict(r=None), mbn.MBN_EINVAL),
        (dict(h=None), mbn.MBN_EINVAL),
        (dict(N=65544), mbn.MBN_EUNSUPPORTED),
        (dict(r=FAKE + 1 * B + 1), mbn.MBN_EUNSUPPORTED),
        (dict(h=FAKE + 3 * B + 5), mbn.MBN_EUNSUPPORTED),
        (dict(h=FAKE + 4 * B), mbn.MBN_EINVAL),  # h == y
        (dict(h=FAKE + 4 * B + 64), mbn.MBN_EINVAL),  # h overlaps y
        (dict(y=FAKE + 16), mbn.MBN_EINVAL),  # y overlaps x partially
        (dict(h=FAKE + 1 * B + 32), mbn.MBN_EINVAL),  # h overlaps r partially
        (dict(w=FAKE + 3 * B + 16), mbn.MBN_EINVAL),  # w inside h
    ],
)
def test_add_rmsnorm_rejects(lib, kw, status):
    a = dict(x=FAKE, r=FAKE + 1 * B, w=FAKE + 2 * B, h=FAKE + 3 * B, y=FAKE + 4 * B, M=4, N=64, eps=1e-6)
    a.update(kw)
    assert lib.add_rmsnorm_fwd(a["x"], a["r"], a["w"], a["h"], a["y"], a["M"], a["N"], a["eps"], None) == status


@pytest.mark.parametrize(
    "kw, status",
    [
        (dict(N=0), mbn.MBN_EINVAL),
        (dict(eps=-1.0), mbn.MBN_EINVAL),
        (dict(b=None), mbn.MBN_EINVAL),
        (dict(w=None), mbn.MBN_EINVAL),
        (dict(N=65544), mbn.MBN_EUNSUPPORTED),
        (dict(b=FAKE + 2 * B + 1), mbn.MBN_EUNSUPPORTED),
        (dict(b=FAKE + 3 * B + 32), mbn.MBN_EINVAL),  # b inside y
        (dict(y=FAKE + 496), mbn.MBN_EINVAL),  # y overlaps the tail of x
    ],
)
def test_layernorm_rejects(lib, kw, status):
    a = dict(x=FAKE, w=FAKE + 1 * B, b=FAKE + 2 * B, y=FAKE + 3 * B, M=4, N=64, eps=1e-5)
    a.update(kw)
    assert lib.layernorm_fwd(a["x"], a["w"], a["b"], a["y"], a["M"], a["N"], a["eps"], None) == status


@pytest.mark.parametrize(
    "kw, status",
    [
        (dict(M=-3), mbn.MBN_EINVAL),
        (dict(x=None), mbn.MBN_EINVAL),
        (dict(eps=float("inf")), mbn.MBN_EINVAL),
        (dict(N=70000), mbn.MBN_EUNSUPPORTED),
        (dict(y=FAKE + 1 * B + 7), mbn.MBN_EUNSUPPORTED),
        (dict(y=FAKE + 256), mbn.MBN_EINVAL),
    ],
)
def test_l2norm_rejects(lib, kw, status):
    a = dict(x=FAKE, y=FAKE + 1 * B, M=4, N=64, eps=1e-12)
    a.update(kw)
    assert lib.l2norm_fwd(a["x"], a["y"], a["M"], a["N"], a["eps"], None) == status


def test_new_entry_points_empty_is_a_noop(lib):
    assert lib.add_rmsnorm_fwd(None, None, None, None, None, 0, 64, 1e-6, None) == mbn.MBN_OK
    assert lib.layernorm_fwd(None, None, None, None, 0, 64, 1e-5, None) == mbn.MBN_OK
    assert lib.l2norm_fwd(None, None, 0, 64, 1e-12, None) == mbn.MBN_OK


@pytest.mark.parametrize(
    "rot, status",
    [(0, mbn.MBN_EINVAL), (-16, mbn.MBN_EINVAL), (33, mbn.MBN_EINVAL), (144, mbn.MBN_EINVAL),
     (24, mbn.MBN_EUNSUPPORTED), (8, mbn.MBN_EUNSUPPORTED), (100, mbn.MBN_EUNSUPPORTED)],
)
def test_qk_partial_rejects(lib, rot, status):
    args = (FAKE, FAKE + 0x10000000, FAKE + 0x10001000, FAKE + 0x10002000, 4, 4, 2, 128, rot, 1e-6, 1e6, None)
    assert lib.qk_norm_rope_partial_fwd(*args) == status


def test_qk_partial_other_checks_still_apply(lib):
    # a valid rotary_dim with an invalid head_dim / null pointer is still rejected before any HIP call
    assert lib.qk_norm_rope_partial_fwd(FAKE, FAKE, FAKE, FAKE, 4, 4, 2, 64, 32, 1e-6, 1e6, None) == mbn.MBN_EUNSUPPORTED
    assert lib.qk_norm_rope_partial_fwd(None, FAKE, FAKE, FAKE, 4, 4, 2, 128, 64, 1e-6, 1e6, None) == mbn.MBN_EINVAL


def test_f16_entry_points_validate_like_bf16(lib):
    """Every invalid-by-construction call gets the same status from both storage types."""
    cases = [
        ("rmsnorm_fwd", (FAKE, FAKE + B, FAKE + 16, 4, 64, 1e-6, None)),
        ("rmsnorm_fwd", (FAKE, FAKE + B, FAKE + 2 * B, 4, 12, 1e-6, None)),
        ("rmsnorm_fwd", (None, FAKE + B, FAKE + 2 * B, 4, 64, 1e-6, None)),
        ("add_rmsnorm_fwd", (FAKE, FAKE + B, FAKE + 2 * B, FAKE + 3 * B, FAKE + 3 * B, 4, 64, 1e-6, None)),
        ("layernorm_fwd", (FAKE, FAKE + B, FAKE + 2 * B, FAKE + 3 * B + 2, 4, 64, 1e-5, None)),
        ("l2norm_fwd", (FAKE, FAKE + B, -1, 64, 1e-12, None)),
        ("qk_norm_rope_partial_fwd", (FAKE, FAKE + B, FAKE + B + 4096, FAKE + B + 8192, 4, 4, 2, 128, 24, 1e-6, 1e6, None)),
        ("qk_norm_rope_partial_fwd", (FAKE, FAKE + B, FAKE + B + 4096, FAKE + B + 8192, 4, 4, 2, 128, 256, 1e-6, 1e6, None)),
    ]
    for name, args in cases:
        a = getattr(lib, name)(*args)
        b = getattr(lib, name + "_f16")(*args)
        assert a == b and a != mbn.MBN_OK, (name, args, a, b)


def test_timed_entry_points_validate_like_the_plain_ones(lib):
    """The timed variants run the plain entry point's checks (same status, no
    HIP call for a rejected or empty input) and reject null events first."""
    ev = FAKE + 0x30000000  # never dereferenced: every call below fails or is empty on the host
    rms_cases = [
        (FAKE, FAKE + B, FAKE + 16, 4, 64, 1e-6, None),      # y overlaps x
        (FAKE, FAKE + B, FAKE + 2 * B, 4, 64, -1.0, None),   # eps < 0
        (FAKE + 1, FAKE + B, FAKE + 2 * B, 4, 64, 1e-6, None),  # odd address
        (None, None, None, 0, 64, 1e-6, None),               # empty: MBN_OK, nothing launched
    ]
    for args in rms_cases:
        assert lib.rmsnorm_fwd_timed(*args, ev, ev + 8) == lib.rmsnorm_fwd(*args), args
    qk_cases = [
        (FAKE, FAKE + B, FAKE + B + 4096, FAKE + B + 8192, 4, 4, 2, 64, 1e-6, 1e6, None),   # head_dim
        (None, FAKE + B, FAKE + B + 4096, FAKE + B + 8192, 4, 4, 2, 128, 1e-6, 1e6, None),  # null qkv
        (FAKE, FAKE + B, FAKE + B + 4096, FAKE + B + 8192, 0, 4, 2, 128, 1e-6, 1e6, None),  # empty
    ]
    for args in qk_cases:
        assert lib.qk_norm_rope_fwd_timed(*args, ev, ev + 8) == lib.qk_norm_rope_fwd(*args), args
    assert lib.rmsnorm_fwd_timed(*rms_cases[0][:7], None, ev) == mbn.MBN_EINVAL
    assert lib.rmsnorm_fwd_timed(*rms_cases[0][:7], ev, None) == mbn.MBN_EINVAL
    assert lib.qk_norm_rope_fwd_timed(*qk_cases[0], None, None) == mbn.MBN_EINVAL


def test_stream_reference_library_loads_and_validates():
    """libmbn_stream.so (the streaming kernels the ceiling measurement times)
    exports its three entry points and rejects, before any launch, sizes that
    are not whole workgroups, unknown workgroup shapes and misaligned or null
    pointers."""
    from probe import stream_lib

    h = stream_lib()  # compiled on first use
    assert h.mbn_stream_copy(FAKE, FAKE + (1 << 30), 4096 + 16, 256, 1, None) == 1  # ragged
    assert h.mbn_stream_copy(FAKE, FAKE + (1 << 30), 4096, 256, 3, None) == 1  # no such shape
    assert h.mbn_stream_copy(FAKE + 8, FAKE + (1 << 30), 4096, 256, 1, None) == 1  # misaligned
    assert h.mbn_stream_copy(FAKE, 0, 4096, 256, 1, None) == 1  # null
    assert h.mbn_stream_read(FAKE, 0, 4096, 256, 1, None) == 1  # null sink
    assert h.mbn_stream_write(FAKE, 0, 256, 1, 0, None) == 1  # empty
    assert h.mbn_stream_copy_policy(FAKE, FAKE + (1 << 30), 4096, 1, 4, None) == 1  # no such policy
    assert h.mbn_stream_copy_policy(FAKE, FAKE + (1 << 30), 4096, 2, 1, None) == 1  # no such shape
    assert h.mbn_stream_copy_policy(FAKE, FAKE + (1 << 30), 4096 + 16, 1, 1, None) == 1  # ragged
    assert h.mbn_stream_qk_pattern(FAKE, 16, 768, 1025, None) == 1  # more q/k chunks than the kernel holds
    assert h.mbn_stream_qk_pattern(FAKE, 16, 600, 640, None) == 1  # row shorter than its q/k part
    assert h.mbn_stream_qk_pattern(FAKE + 8, 16, 768, 640, None) == 1  # misaligned


def test_c_client_builds_and_sees_host_validation():
    """The plain C client links against libmbn.so and the HIP runtime only;
    a call the library rejects on the host returns MBN_EINVAL without a GPU."""
    if not os.path.exists(mbn_build.C_CLIENT_LIB):
        mbn_build.build_c_client()
    lib = ctypes.CDLL(mbn_build.C_CLIENT_LIB)
    assert lib.mbn_c_client_reject() == mbn.MBN_EINVAL
