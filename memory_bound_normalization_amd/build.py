"""Build libmbn.so (the HIP kernels and the C entry points) for gfx950, in tree.

    python -m memory_bound_normalization_amd.build

Compiles every ``csrc/*.hip`` file with hipcc into one shared library next to
this file. No fast-math: the kernels rely on IEEE fp32/fp64 behaviour.
``build_c_client()`` compiles the plain C client of the C ABI the tests use
(``tests/c_abi``) with gcc, and ``build_rope_host()`` a host build of the
kernels' rotary-angle functions (``csrc/rope_math.h``) for the CPU tests. (The measurement tools next to bench.py build
their own streaming reference kernels with ``build(out=..., sources_=...)``.)
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmbn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmbn.so)")


def sources(src_dir: str = CSRC) -> list[str]:
    return sorted(glob.glob(os.path.join(src_dir, "*.hip")))


def compile_command(out: str, extra: list[str] | None = None, srcs: list[str] | None = None) -> list[str]:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-fvisibility=hidden",
        "-Wall",
        # packed fp32 VALU ops stay off (device pass; the host pass ignores it)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        *(extra or []),
        "-o", out,
        *(srcs if srcs is not None else sources()),
    ]


def build(verbose: bool = False, out: str = LIB_PATH, extra: list[str] | None = None,
          sources_: list[str] | None = None) -> str:
    """Compile the library (or, with ``sources_``, those HIP files with the
    same flags); always rebuilds. Returns the path of the .so."""
    tmp = out + ".tmp"
    cmd = compile_command(tmp, extra, sources_)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "mbn_c_client.c")
C_CLIENT_LIB = os.path.join(ROOT, "tests", "c_abi", "libmbn_c_client.so")


def build_c_client(verbose: bool = False) -> str:
    """Compile tests/c_abi/libmbn_c_client.so (C, against libmbn.so and the
    HIP runtime only); always rebuilds. Needs libmbn.so built first."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-shared", "-fPIC", "-std=c11", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CLIENT_SRC,
           "-L", PKG, "-lmbn", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../memory_bound_normalization_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_CLIENT_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"gcc failed with status {res.returncode}")
    os.replace(C_CLIENT_LIB + ".tmp", C_CLIENT_LIB)
    return C_CLIENT_LIB


ROPE_HOST_SRC = os.path.join(ROOT, "tests", "c_abi", "rope_math_host.hip")
ROPE_HOST_LIB = os.path.join(ROOT, "tests", "c_abi", "librope_math_host.so")


def build_rope_host(verbose: bool = False) -> str:
    """Compile tests/c_abi/librope_math_host.so: the QK kernel's sincos and
    inverse-frequency functions built for the host; always rebuilds."""
    return build(verbose=verbose, out=ROPE_HOST_LIB, sources_=[ROPE_HOST_SRC])


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client(verbose=True))
    print(build_rope_host(verbose=True))
