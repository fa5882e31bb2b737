"""The C ABI from a plain C client (tests/c_abi/mbn_c_client.c): device memory
from hipMalloc, the operators through the entry points of include/mbn.h, no
PyTorch on the path. Its outputs are compared with the fp64 oracle, every
output (an aligned width, an odd width, and the fused QK-norm + RoPE)."""

import ctypes
import os

import numpy as np
import pytest

from memory_bound_normalization_amd import build as mbn_build
from oracle import qk_norm_rope_fwd as o_qk, rmsnorm_fwd as o_rms
from parity import assert_parity
from workloads import random_bf16_bits

pytestmark = pytest.mark.gpu

U16P = ctypes.POINTER(ctypes.c_uint16)
I64P = ctypes.POINTER(ctypes.c_int64)


@pytest.fixture(scope="module")
def client():
    if not os.path.exists(mbn_build.C_CLIENT_LIB):
        pytest.fail(f"{mbn_build.C_CLIENT_LIB} is not built (python -m memory_bound_normalization_amd.build)")
    lib = ctypes.CDLL(mbn_build.C_CLIENT_LIB)
    lib.mbn_c_client_rmsnorm.argtypes = [U16P, U16P, U16P, ctypes.c_int64, ctypes.c_int64, ctypes.c_float]
    lib.mbn_c_client_rmsnorm.restype = ctypes.c_int
    lib.mbn_c_client_qk_norm_rope.argtypes = [U16P, U16P, U16P, I64P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_float, ctypes.c_float]
    lib.mbn_c_client_qk_norm_rope.restype = ctypes.c_int
    return lib


def _p(a, t=U16P):
    return a.ctypes.data_as(t)


@pytest.mark.parametrize("M,N", [(37, 4104), (5, 1001), (3, 16384)])
def test_rmsnorm_from_c(client, M, N):
    print(f"[c client rmsnorm] M={M} N={N}", flush=True)
    rng = np.random.default_rng(M * N)
    x = np.ascontiguousarray(random_bf16_bits(rng, (M, N)))
    w = np.ascontiguousarray(random_bf16_bits(rng, (N,), lo=0.5, hi=1.5))
    y = np.zeros((M, N), dtype=np.uint16)
    assert client.mbn_c_client_rmsnorm(_p(x), _p(w), _p(y), M, N, 1e-6) == 0
    assert_parity(y, o_rms(x, w, 1e-6), f"C client rmsnorm M={M} N={N}")


def test_qk_norm_rope_from_c(client):
    T, hq, hkv = 9, 4, 2
    print(f"[c client qk] T={T}", flush=True)
    rng = np.random.default_rng(5)
    qkv = np.ascontiguousarray(random_bf16_bits(rng, (T, (hq + 2 * hkv) * 128)))
    q_w = np.ascontiguousarray(random_bf16_bits(rng, (128,), lo=0.5, hi=1.5))
    k_w = np.ascontiguousarray(random_bf16_bits(rng, (128,), lo=0.5, hi=1.5))
    pos = np.arange(T, dtype=np.int64) * 37
    ref = o_qk(qkv, q_w, k_w, pos, hq, hkv, 128, 1e-6, 1e6)
    got = qkv.copy()
    assert client.mbn_c_client_qk_norm_rope(_p(got), _p(q_w), _p(k_w), _p(pos, I64P), T, hq, hkv, 1e-6, 1e6) == 0
    assert_parity(got, ref, "C client qk_norm_rope")
