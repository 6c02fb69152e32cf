"""The product kernels' LDS fragment reads are inline asm, so the compiler
does not know they are in flight: it takes their registers as written when
the read issues.  The last contraction stage reads the next stage's fragments
(never used), so unless the kernel waits for those reads and keeps their
registers live through the wait, the code after the loop may be given those
registers while a read is still landing in them.  This compiles gemm.hip for
gfx950 (device code only, the library's own flags) and checks, in every
product kernel, that no instruction between the loop's exit and the first
lgkmcnt(0) wait writes a register that an LDS fragment read in the loop's
last stage targets, and more generally that no instruction touches any
fragment read's registers before a wait that covers that read.  It also
checks the quantizers' hand-written DPP instructions for the two wait states
a DPP source needs after a VALU write.  CPU only (hipcc cross-compiles).
"""
import os
import re
import shutil
import subprocess

import pytest

from w8a8_integer_linear_amd import build as hip_build

_READ = re.compile(r"^(ds_read_b128|ds_read_b64_tr_b8)\s+v\[(\d+):(\d+)\]")
_LOAD = ("ds_read", "ds_load", "global_load", "buffer_load", "flat_load", "scratch_load")
_NOT_VGPR_DEST = ("v_cmp", "v_readlane", "v_readfirstlane")


def _dest_vgprs(line):
    """VGPRs an instruction writes (its first operand, for VALU ops and loads)."""
    op = line.split()[0]
    if not (op.startswith("v_") or op.startswith(_LOAD)) or op.startswith(_NOT_VGPR_DEST):
        return set()
    rest = line[len(op):].strip()
    m = re.match(r"v\[(\d+):(\d+)\]", rest)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)\b", rest)
    return {int(m.group(1))} if m else set()


def loop_exit_hazards(body):
    """Instructions (after the main loop, before the first lgkmcnt(0) wait)
    that write a register targeted by an LDS fragment read of the final
    stage.  body: the kernel's assembly lines."""
    lines = [l.split(";")[0].strip() for l in body]
    mfma = [k for k, l in enumerate(lines) if l.startswith("v_mfma")]
    assert mfma, "no MFMA in the kernel"
    k = mfma[-1]
    while not lines[k].startswith(("s_cbranch", "s_branch")):
        k += 1
    targets = set()
    for l in lines[max(0, k - 200):k]:
        m = _READ.match(l)
        if m:
            targets.update(range(int(m.group(2)), int(m.group(3)) + 1))
    assert targets, "no fragment reads before the loop's back edge"
    bad = []
    for l in lines[k + 1:]:
        if not l or l.startswith(".") or l.endswith(":"):
            continue
        if l.startswith("s_waitcnt") and "lgkmcnt(0)" in l:
            return bad
        if _dest_vgprs(l) & targets:
            bad.append(l)
    raise AssertionError("no lgkmcnt(0) wait after the main loop")


def _kernels(asm):
    out = {}
    for m in re.finditer(r"^(_Z\w*gemm_kernel\w*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        out[m.group(1)] = asm[m.end():end].split("\n")
    return out


def test_destination_parser():
    assert _dest_vgprs("v_lshl_or_b32 v128, v171, 6, s30") == {128}
    assert _dest_vgprs("ds_read_b64_tr_b8 v[130:131], v2 offset:64") == {130, 131}
    assert _dest_vgprs("v_cmp_gt_i32_e32 vcc, v1, v0") == set()
    assert _dest_vgprs("global_store_dwordx4 v[2:3], v[4:7], off") == set()
    assert _dest_vgprs("s_mov_b32 s3, 0") == set()


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    """The product kernels' gfx950 assembly: {kernel symbol: lines}."""
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [cc, *hip_build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(hip_build.CSRC, "gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = _kernels(out.read_text())
    assert len(kernels) >= 10
    return kernels


def test_no_register_reuse_before_fragment_reads_land(gemm_asm):
    found = {name: loop_exit_hazards(body) for name, body in gemm_asm.items()}
    assert not any(found.values()), {k: v[:3] for k, v in found.items() if v}


_VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _regs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def fragment_read_hazards(body):
    """Instructions that read or write the registers of an inline-asm LDS
    fragment read before a wait that covers it.  LDS operations complete in
    order, so s_waitcnt lgkmcnt(n) covers a read once n or more LDS
    operations were issued after it.  The scan follows the text order (a
    loop's last reads continue into the code after the loop)."""
    lines = [l.split(";")[0].strip() for l in body]
    bad = []
    for i, l in enumerate(lines):
        m = _READ.match(l)
        if not m:
            continue
        dst = set(range(int(m.group(2)), int(m.group(3)) + 1))
        after = 0
        for l2 in lines[i + 1:]:
            if not l2 or l2.startswith(".") or l2.endswith(":"):
                continue
            w = re.search(r"lgkmcnt\((\d+)\)", l2)
            if l2.startswith("s_waitcnt") and w and after >= int(w.group(1)):
                break
            op = l2.split()[0]
            operands = l2[len(op):]
            if op.startswith("ds_read") or op.startswith("ds_load"):
                # Another LDS read: in-order returns make a shared
                # destination harmless; its address must not be one of ours.
                touched = _regs(operands.split(",", 1)[1]) if "," in operands else set()
            else:
                touched = _regs(operands)
            if touched & dst:
                bad.append((l, l2))
                break
            if op.startswith("ds_"):
                after += 1
    return bad


def test_fragment_reads_are_waited_for_before_use(gemm_asm):
    found = {name: fragment_read_hazards(body) for name, body in gemm_asm.items()}
    assert not any(found.values()), {k: v[:3] for k, v in found.items() if v}


# ------------------------------------------------------- DPP wait states

_DPP = re.compile(r"^(v_\w+_dpp)\s+(v\d+|v\[\d+:\d+\]),\s*(v\d+|v\[\d+:\d+\])")


def dpp_hazards(body):
    """DPP instructions whose DPP source (src0) a VALU instruction wrote less
    than two wait states before (s_nop n counts n + 1, any other instruction
    one).  The scan stops at a label: the quantizers' DPP asm sits in
    straight-line blocks that start with their own s_nop."""
    lines = [l.split(";")[0].strip() for l in body]
    bad = []
    for i, l in enumerate(lines):
        m = _DPP.match(l)
        if not m:
            continue
        src = _regs(m.group(3))
        waits = 0
        for l2 in reversed(lines[:i]):
            if not l2 or l2.startswith("."):
                if l2.endswith(":"):
                    break
                continue
            if l2.endswith(":"):
                break
            op = l2.split()[0]
            if op == "s_nop":
                waits += int(l2.split()[1], 0) + 1
            else:
                if op.startswith("v_") and _dest_vgprs(l2) & src:
                    bad.append((l2, l))
                    break
                waits += 1
            if waits >= 2:
                break
    return bad


def test_dpp_sources_have_their_wait_states(tmp_path):
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path / "quant.s"
    cmd = [cc, *hip_build.FLAGS, "--cuda-device-only", "-S",
           os.path.join(hip_build.CSRC, "quant.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    kernels = {}
    for m in re.finditer(r"^(_Z\w*kernel\w*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        kernels[m.group(1)] = asm[m.end():end].split("\n")
    n_dpp = sum(1 for body in kernels.values() for l in body if "_dpp " in l)
    assert n_dpp > 100, "the quantizers' DPP butterflies are missing from the assembly"
    found = {name: dpp_hazards(body) for name, body in kernels.items()}
    assert not any(found.values()), {k: v[:3] for k, v in found.items() if v}


def test_dpp_checker_flags_a_missing_wait():
    write = "v_add_f32_e32 v41, v1, v2"
    dpp = "v_fmac_f32_dpp v41, v41, v53 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
    assert dpp_hazards([write, dpp])
    assert dpp_hazards([write, "v_mov_b32_e32 v7, v8", dpp])
    assert not dpp_hazards([write, "s_nop 1", dpp])
    assert not dpp_hazards([write, "v_mov_b32_e32 v7, v8", "v_mov_b32_e32 v9, v8", dpp])
