"""CPU check of the built library's per-chunk-wait kernels (their gfx950 ISA,
disassembled from libmbn.so with the ROCm LLVM tools).

In those kernels pass 1 reads chunk q of the staged row set as soon as
`s_waitcnt vmcnt(RPL * MAXC - 1 - q)` returns: vector-memory operations
complete in issue order, so that wait means "chunk q's copy has landed" only if
the RPL * MAXC row copies (global_load_lds_dwordx4) are the last vector-memory
operations issued before the waits. This test holds every such kernel in
libmbn.so to that: the weight (and bias) loads come before the first copy, no
other vector-memory operation sits among the copies, there are exactly
RPL * MAXC of them, and the waits of the fast path count down from
RPL * MAXC - 1 to 0. A compiler that sank a weight load among the copies, or
moved another memory operation there, would fail it. No GPU is needed.
"""

import os
import re
import shutil
import subprocess

import pytest

from memory_bound_normalization_amd import build as mbn_build

ROCM_LLVM = "/opt/rocm/llvm/bin"
TOOLS = {t: os.path.join(ROCM_LLVM, t) for t in ("clang-offload-bundler", "llvm-objdump")}
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# rownorm_kernel<Norm MODE, DT, WPR, ROWS, RPL, MAXC, FULL = true, CHUNK_WAIT = true>
CW_KERNEL = re.compile(
    r"^[0-9a-f]+ <(_ZN3mbn12_GLOBAL__N_114rownorm_kernelILNS_4NormE(\d)ENS_\d(?:Bf16|F16)ELi(\d+)ELi(\d+)ELi(\d+)"
    r"ELi(\d+)ELb1ELb1EEEvNS_11RowNormArgsE)>:$")
VMEM = re.compile(r"^\s*(global_|buffer_|flat_)")


def _disassemble(tmp_path):
    for t in TOOLS.values():
        if not os.path.exists(t):
            pytest.skip(f"{t} not available")
    if not shutil.which("objcopy"):
        pytest.skip("objcopy not available")
    if not os.path.exists(mbn_build.LIB_PATH):
        mbn_build.build()
    fat = tmp_path / "fatbin.bin"
    # objcopy rewrites the file it reads when given no output file: work on a
    # copy, and write the copy's result to another scratch file
    lib = tmp_path / "libmbn_copy.so"
    shutil.copyfile(mbn_build.LIB_PATH, lib)
    subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", str(lib), str(tmp_path / "stripped.so")],
                   check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    text = []
    for k, s in enumerate(starts):
        part = tmp_path / f"b{k}.bin"
        part.write_bytes(data[s:starts[k + 1] if k + 1 < len(starts) else len(data)])
        obj = tmp_path / f"b{k}.o"
        subprocess.run([TOOLS["clang-offload-bundler"], "--unbundle", "--type=o", f"--input={part}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={obj}"], check=True)
        out = subprocess.run([TOOLS["llvm-objdump"], "-d", "--no-show-raw-insn", str(obj)], check=True,
                             capture_output=True, text=True).stdout
        text.append(out)
    return "\n".join(text)


def _kernels(asm):
    """{name: (mode, wpr, rows, rpl, maxc, [instruction lines])} for the
    per-chunk-wait instantiations."""
    out, cur = {}, None
    for line in asm.split("\n"):
        m = CW_KERNEL.match(line)
        if m:
            cur = m.group(1)
            out[cur] = (*(int(v) for v in m.groups()[1:]), [])
            continue
        if cur is None:
            continue
        if re.match(r"^[0-9a-f]+ <", line):
            cur = None
            continue
        ins = line.split("//")[0].strip()
        if ins:
            out[cur][-1].append(ins)
    return out


def test_per_chunk_wait_kernels_issue_the_copies_last(tmp_path):
    ks = _kernels(_disassemble(tmp_path))
    assert len(ks) >= 20, f"only {len(ks)} per-chunk-wait kernels found"
    for name, (mode, wpr, rows, rpl, maxc, ins) in ks.items():
        copies = [i for i, s in enumerate(ins) if s.startswith("global_load_lds_dwordx4")]
        assert copies, name
        first, last = copies[0], copies[-1]
        # exactly RPL * MAXC copies, contiguous among the vector-memory operations
        assert len(copies) == rpl * maxc, (name, len(copies))
        between = [s for s in ins[first:last + 1] if VMEM.match(s) and not s.startswith("global_load_lds")]
        assert not between, (name, between[:3])
        # the weight and bias loads come first: none after the first copy
        # until the waits of pass 1 have begun
        waits = [i for i, s in enumerate(ins) if i > last and s.startswith("s_waitcnt") and "vmcnt(" in s]
        assert waits, name
        after = [s for s in ins[last + 1:waits[0]] if VMEM.match(s)]
        assert not after, (name, after[:3])
        loads_before = [s for s in ins[:first] if s.startswith("global_load_dwordx4")]
        n_affine = (maxc if mode != 3 else 0) + (maxc if mode == 2 else 0)  # weight, bias (L2Norm: none)
        assert len(loads_before) == n_affine, (name, len(loads_before), n_affine)
        # the fast path counts down: vmcnt(RPL*MAXC-1), ..., vmcnt(0) in this order
        counts = [int(re.search(r"vmcnt\((\d+)\)", ins[i]).group(1)) for i in waits]
        want = list(range(rpl * maxc - 1, -1, -1))
        it = iter(counts)
        assert all(any(c == w for c in it) for w in want), (name, counts[:40])
