"""Build libmbn.so (the HIP kernels and the C entry points) for gfx950, in tree.

    python -m memory_bound_normalization_amd.build

Compiles every ``csrc/*.hip`` file with hipcc into one shared library next to
this file. No fast-math: the kernels rely on IEEE fp32/fp64 behaviour.
``build_stream()`` compiles ``probe_csrc/*.hip`` into libmbn_stream.so, the
plain streaming kernels the measurement tools time beside the norms (not part
of the normalization path). ``build_c_client()`` compiles the plain C client
of the C ABI the tests use (``tests/c_abi``) with gcc.
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
PROBE_CSRC = os.path.join(PKG, "probe_csrc")
STREAM_LIB_PATH = os.path.join(PKG, "libmbn_stream.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmbn.so)")


def sources(src_dir: str = CSRC) -> list[str]:
    return sorted(glob.glob(os.path.join(src_dir, "*.hip")))


def compile_command(out: str, extra: list[str] | None = None, src_dir: str = CSRC) -> list[str]:
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
        *sources(src_dir),
    ]


def build(verbose: bool = False, out: str = LIB_PATH, extra: list[str] | None = None,
          src_dir: str = CSRC) -> str:
    """Compile the library; always rebuilds. Returns the path of the .so."""
    tmp = out + ".tmp"
    cmd = compile_command(tmp, extra, src_dir)
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


def build_stream(verbose: bool = False) -> str:
    """Compile libmbn_stream.so (the streaming reference kernels); always rebuilds."""
    return build(verbose=verbose, out=STREAM_LIB_PATH, src_dir=PROBE_CSRC)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_stream(verbose=True))
    print(build_c_client(verbose=True))
