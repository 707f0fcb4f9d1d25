"""Host-side check of the prefill GEMMs' machine code (no GPU needed).

Their LDS operand reads are written in inline assembly, so the compiler does
not know when their destination registers are written: any instruction it
places between such a read and the s_waitcnt lgkmcnt that covers it may read
or overwrite a register whose load is still in flight (a copy made there
reads stale data; a register reused for an address can be overwritten by the
arriving load).  The kernels therefore wait for every such read inside the
same assembly block.  This test compiles gemm_fp8.hip for gfx950 and walks
each prefill kernel's instructions in order: between a ds_read and the
lgkmcnt wait that retires it (LDS returns in order), no other instruction
may name its destination registers.
"""

import os
import re
import shutil
import subprocess

import pytest

from mxfp4_block_scaled_top_amd import build

SRC = os.path.join(build.CSRC, "gemm_fp8.hip")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return []
    return [t.strip() for t in re.split(r",\s*", parts[1].split(" offset:")[0].split(";")[0])]


def lds_read_hazards(asm):
    """(kernel, line) pairs where an instruction names a register of an LDS
    read still in flight; also the number of kernels and ds_reads seen."""
    bad, kernels, reads = [], 0, 0
    for name in re.findall(r"^(_ZN2mx\d+prefill_gemm\w*kernel\S*):", asm, re.M):
        kernels += 1
        body = asm[asm.index(name + ":"):asm.index(".Lfunc_end", asm.index(name + ":"))]
        pending = []
        for line in (l.strip() for l in body.split("\n")):
            if not line or line.startswith((".", ";", "//")) or line.endswith(":"):
                continue
            op = line.split()[0]
            ops = _operands(line)
            if op == "s_waitcnt" and "lgkmcnt" in line:
                n = int(re.search(r"lgkmcnt\((\d+)\)", line).group(1))
                pending = pending[len(pending) - n:] if len(pending) > n else pending
                continue
            live = set().union(*pending) if pending else set()
            named = set()
            for t in ops:
                named |= _regs(t)
            if named & live:
                bad.append((name, line))
            if op.startswith("ds_read"):
                reads += 1
                pending.append(_regs(ops[0]))
            elif op.startswith(("s_load", "s_buffer_load")):
                pending.append(set())   # also counted by lgkmcnt
    return bad, kernels, reads


def test_prefill_lds_reads_are_waited_before_use(tmp_path):
    hipcc = build._hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    out = tmp_path / "gemm_fp8.s"
    cmd = [hipcc] + build.FLAGS + ["--cuda-device-only", "-S", SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    bad, kernels, reads = lds_read_hazards(out.read_text())
    assert kernels >= 9 and reads > 100
    assert not bad, "registers of LDS reads in flight used: %s" % bad[:5]


def test_the_check_finds_a_planted_hazard():
    # a copy of a read's destination before its wait is flagged; after it, not
    asm = ("_ZN2mx19prefill_gemm_kernelX:\n"
           "\tds_read_b128 v[4:7], v1\n\tv_mov_b32_e32 v9, v5\n\ts_waitcnt lgkmcnt(0)\n"
           "\tds_read_b128 v[4:7], v1\n\ts_waitcnt lgkmcnt(0)\n\tv_mov_b32_e32 v9, v5\n.Lfunc_end0:\n")
    bad, kernels, reads = lds_read_hazards(asm)
    assert kernels == 1 and reads == 2
    assert [l for _, l in bad] == ["v_mov_b32_e32 v9, v5"]
