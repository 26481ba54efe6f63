"""Code-generation guard for the decode kernels (host only: hipcc cross-compiles for gfx950).

The decode kernel's QK loop issues a batch of LDS reads and lets each MFMA wait only for its own
operand (``s_waitcnt lgkmcnt(N)`` with N > 0). A register-pressure change elsewhere in the kernel
can make the compiler read every operand into one register quad instead, so that each MFMA
waits for all outstanding LDS reads (``lgkmcnt(0)``): the results stay bit-identical and nothing
spills, but the kernel runs tens of percent slower (it happened to the shared-rows
instantiation, 34 such waits instead of 3). This test compiles decode.hip to assembly with the
library's own flags and bounds those waits in every decode instantiation.
"""

import os
import re
import shutil
import subprocess

import pytest

from nvfp4_compressed_mla_amd import build as B

MAX_SERIALIZED_WAITS = 4      # every instantiation has 1-3 (prologue and epilogue reads)


def _kernel_bodies(asm):
    """(name, instructions, next_free_vgpr) of every decode_kernel instantiation."""
    lines = asm.split("\n")
    out = []
    for i, line in enumerate(lines):
        if not (line.startswith("_ZN3mla13decode_kernel") and ":" in line):
            continue
        name = line.split(":")[0]
        j = i
        while not lines[j].startswith(".Lfunc_end"):
            j += 1
        ins = [l.split(";")[0].strip() for l in lines[i + 1:j]
               if l.startswith("\t") and not l.strip().startswith((".", ";"))]
        meta = asm[asm.index("\t.amdhsa_kernel " + name):]
        vgpr = int(re.search(r"\.amdhsa_next_free_vgpr\s+(\d+)", meta).group(1))
        out.append((name, ins, vgpr))
    return out


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "decode.s"
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [B.HIPCC, *flags, "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC, "-S",
           "--cuda-device-only", os.path.join(B.CSRC, "decode.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_decode_kernels_keep_lds_reads_in_flight(decode_asm):
    kernels = _kernel_bodies(decode_asm)
    # 4 fused-append + 8 NVFP4 (sparse and dense) + 8 FP8 + 1 shared-rows instantiations
    assert len(kernels) == 21, [k[0] for k in kernels]
    bad = []
    for name, ins, vgpr in kernels:
        serialized = sum(1 for a, b in zip(ins, ins[1:])
                         if a == "s_waitcnt lgkmcnt(0)" and b.startswith("v_mfma"))
        scratch = sum(1 for x in ins if x.startswith("scratch_") or x.startswith("buffer_store"))
        if serialized > MAX_SERIALIZED_WAITS or scratch or vgpr > 168:
            bad.append((name, serialized, scratch, vgpr))
    assert not bad, f"(kernel, lgkmcnt(0)->mfma waits, scratch ops, vgprs): {bad}"


def _compile(tmp_path_factory, name):
    out = tmp_path_factory.mktemp("asm_" + name) / (name + ".s")
    flags = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [B.HIPCC, *flags, "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC, "-S",
           "--cuda-device-only", os.path.join(B.CSRC, name + ".hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


@pytest.mark.parametrize("name", ["codec", "decode", "fp8", "indexer", "layout", "topk", "union"])
def test_no_waterfall_loops_and_no_scratch(tmp_path_factory, name):
    """A buffer resource or scalar operand the compiler cannot prove wave-uniform is rebuilt around
    every access in a loop of readfirstlane + 64-bit compare + exec mask (the indexer's score
    stores and the top-k filter's list stores once spent most of their time there). Every kernel
    keeps such values in scalar registers, and none spills to scratch."""
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    asm = _compile(tmp_path_factory, name)
    lines = [l.split(";")[0].strip() for l in asm.split("\n")]
    waterfalls = sum(1 for i in range(len(lines) - 6)
                     if lines[i].startswith("v_readfirstlane_b32")
                     and any(x.startswith("v_cmp_eq_u64") for x in lines[i:i + 8])
                     and any(x.startswith("s_and_saveexec_b64") for x in lines[i:i + 10]))
    scratch = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", asm)
    assert waterfalls == 0, f"{name}.hip: {waterfalls} waterfall loops"
    assert scratch and all(int(s) == 0 for s in scratch), f"{name}.hip: scratch {scratch}"
