"""Checks on the gfx950 assembly of the product kernels (compiled here with hipcc, no GPU).

The INT4 product kernels end every slab with `s_waitcnt lgkmcnt(N); s_barrier` (N > 0): the
barrier publishes the trits this wave wrote to LDS, and may leave the wave's last N LDS
operations in flight.  That is correct only if at least N LDS reads follow the last LDS write
before each such barrier (LDS operations complete in order), which the source arranges with
scheduling barriers; this test reads the compiled code of every instantiation to confirm it."""
import os
import re
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "ternary_weight_bit_bitlinear_amd", "csrc")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return shutil.which("hipcc")


@pytest.mark.skipif(hipcc() is None, reason="hipcc needed")
def test_relaxed_barriers_follow_enough_lds_reads(tmp_path):
    out = tmp_path / "gemm.s"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, "gemm.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    kernels = re.split(r"\n(?=_ZN\S*gemm_tern4\w*_kernel\S*:)", text)[1:]
    assert len(kernels) >= 4
    seen = 0
    for k in kernels:
        body = k.split(".Lfunc_end", 1)[0]
        name = body.split(":", 1)[0]
        reads, after_write, pending = 0, False, None
        for line in body.splitlines():
            op = line.strip().split(" ", 1)[0]
            if pending is not None:
                # the relaxed wait of a barrier: s_waitcnt lgkmcnt(N) right before s_barrier
                if op == "s_barrier":
                    after, nreads, n = pending
                    assert after and nreads >= n, f"{name}: {nreads} reads after the last write, lgkmcnt({n})"
                    seen += 1
                pending = None
            if op.startswith("ds_write"):
                reads, after_write = 0, True
            elif op.startswith("ds_read"):
                reads += 1
            elif op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", line)
                if m and int(m.group(1)) > 0:
                    pending = (after_write, reads, int(m.group(1)))
    assert seen >= 4 * 5


def _vregs(tok):
    """VGPR numbers named by an operand such as v7 or v[12:15] (AGPRs and SGPRs give none)."""
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return range(int(m.group(1)), int(m.group(2)) + 1)
    m = re.fullmatch(r"v(\d+)", tok)
    return range(int(m.group(1)), int(m.group(1)) + 1) if m else range(0)


@pytest.mark.skipif(hipcc() is None, reason="hipcc needed")
def test_mfma_operands_settle_before_use(tmp_path):
    """The MFMAs are inline asm, so the compiler inserts no wait states between a vector
    instruction that writes an A or B operand register and the MFMA that reads it; the source
    places them (or an s_nop that takes the operand as input).  Every MFMA must find its operand
    registers last written by a vector instruction at least five wait states earlier (one per
    instruction, N + 1 per s_nop N), counted in layout order through block labels: conservative
    where a branch skips code, and it also sees a write that the compiler sank past a branch
    into the block of its MFMA."""
    out = tmp_path / "gemm.s"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, "gemm.hip")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = out.read_text()
    kernels = re.split(r"\n(?=_ZN\S*gemm_tern\w*_kernel\S*:)", text)[1:]
    assert len(kernels) >= 6
    need, checked = 5, 0
    for k in kernels:
        body = k.split(".Lfunc_end", 1)[0]
        name = body.split(":", 1)[0]
        clock, written = 0, {}
        for line in body.splitlines()[1:]:
            s = line.split(";", 1)[0].strip()
            if not s or s.startswith("."):
                continue
            op, _, rest = s.partition(" ")
            ops = [t.strip() for t in rest.split(",")]
            if op.startswith("v_mfma"):
                for src in ops[1:3]:
                    for r in _vregs(src):
                        if r in written:
                            assert clock - written[r] >= need, f"{name}: v{r} written {clock - written[r]} wait states before {s}"
                checked += 1
            elif op.startswith("v_") and ops:
                for r in _vregs(ops[0]):
                    written[r] = clock
            clock += int(ops[0], 0) + 1 if op == "s_nop" else 1
    assert checked >= 4 * 640
