"""CPU check of the gfx950 code hipcc makes from kernels.hip: every LDS DMA
load (buffer_load ... lds, issued from inline asm, where the compiler's own
hazard checks do not reach) has at least 5 wait states after any VALU
instruction that wrote an SGPR the load reads (its buffer descriptor or scalar
offset), and at least 1 after the write of m0.

A build without them faulted the GPU: a spilled descriptor, reloaded by
v_readlane one to three instructions before such a load, was read stale.
This test compiles the kernels to assembly (about half a minute) and scans
every function."""
import os
import re
import subprocess

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "bounded_kv_block_amd", "csrc", "kernels.hip")
VMEM_SGPR_WAITS = 5       # VALU writes an SGPR -> VMEM reads it
M0_WAITS = 1              # scalar write of m0 -> LDS DMA reads it


def _sgprs(tok):
    out = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", tok):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", tok):
        out.add(int(m.group(1)))
    if re.search(r"\bm0\b", tok):
        out.add("m0")
    return out


def _instructions(asm):
    """(line, text) of each instruction, labels, directives and comments dropped"""
    out = []
    for i, ln in enumerate(asm.splitlines()):
        t = ln.split(";")[0].strip()
        if t and not t.endswith(":") and not t.startswith("."):
            out.append((i + 1, t))
    return out


def scan(asm):
    """Violations: (load line, writer line, wait states between) for LDS DMA
    loads that read an SGPR (or m0) written too recently."""
    ins = _instructions(asm)
    bad = []
    for k, (ln, t) in enumerate(ins):
        if not (t.startswith("buffer_load") and t.endswith(" lds")):
            continue
        ops = [p.strip() for p in t.split(None, 1)[1].split(",")]
        reads = _sgprs(ops[1]) | _sgprs(ops[2]) | {"m0"}
        ws = 0
        for j in range(k - 1, max(-1, k - 16), -1):
            lj, tj = ins[j]
            op = tj.split()[0]
            if op == "s_nop":
                ws += int(tj.split()[1], 0) + 1
                continue
            if ws >= VMEM_SGPR_WAITS:
                break
            if op.startswith("s_endpgm") or op.startswith("s_branch") or op.startswith("s_cbranch"):
                break
            ops_j = [x.strip() for x in tj.split(None, 1)[1].split(",")] if " " in tj else []
            dst = _sgprs(ops_j[0]) if ops_j else set()
            # VOP3 forms that also write an SGPR pair (carry out, or the scale flag)
            if len(ops_j) > 1 and re.match(r"v_(add|sub|subrev|addc|subb|subbrev)_co|v_mad_[iu]64_[iu]32|v_div_scale", op):
                dst |= _sgprs(ops_j[1])
            hit = dst & reads
            if hit:
                if op.startswith("v_") and not op.startswith("v_mfma") and ws < VMEM_SGPR_WAITS:
                    bad.append((ln, lj, ws, tj))
                elif "m0" in hit and ws < M0_WAITS:
                    bad.append((ln, lj, ws, tj))
            ws += 1
    return bad


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-function",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.dirname(SRC)}",
           "--cuda-device-only", "-S", SRC, "-o", str(out)]
    if not os.path.exists(cmd[0]):
        pytest.skip("hipcc not installed")
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def test_scan_finds_the_hazard_it_looks_for():
    """The scan itself: a descriptor reloaded by v_readlane two instructions
    before the load is reported; with s_nop 4 between them it is not."""
    bad = ("v_readlane_b32 s7, v253, 5\n\ts_mov_b32 m0, s2\n\ts_nop 0\n"
           "\tbuffer_load_dwordx4 v172, s[4:7], s2 offen lds\n")
    good = ("v_readlane_b32 s7, v253, 5\n\ts_mov_b32 m0, s2\n\ts_nop 4\n"
            "\tbuffer_load_dwordx4 v172, s[4:7], s2 offen lds\n")
    assert len(scan(bad)) == 1 and scan(good) == []
    assert len(scan("\ts_mov_b32 m0, s2\n\tbuffer_load_dwordx4 v1, s[4:7], s3 offen lds\n")) == 1
    carry = "\tv_add_co_u32_e64 v1, s[6:7], v2, v3\n\ts_nop 1\n\tbuffer_load_dwordx4 v1, s[4:7], s3 offen lds\n"
    assert len(scan(carry)) == 1


def test_lds_dma_loads_have_their_wait_states(device_asm):
    loads = sum(1 for _, t in _instructions(device_asm) if t.startswith("buffer_load") and t.endswith(" lds"))
    assert loads > 0
    bad = scan(device_asm)
    assert bad == [], bad[:5]
