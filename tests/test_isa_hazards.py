"""Hazards around the inline-asm MFMAs, checked in the generated assembly.

The output MFMAs that keep O in AGPRs are inline asm, so the compiler's
hazard recognizer inserts no wait states on either side of them.  The
kernels keep the distances by construction; tests/isa_check.py finds
violations over every path of each kernel's control-flow graph:

* a VALU write of a VGPR that an inline-asm MFMA reads as A or B within 4
  wait states before it (the compiler once moved the last P pack right in
  front of the first output MFMA of a tile, which then read a stale value on
  some runs);
* a compiler-issued read of an AGPR that an inline-asm MFMA writes (VALU,
  v_accvgpr_read/mov, a compiler-issued MFMA reading it as C, a store) within
  19 wait states after it (the explicit `s_nop` groups, with the accumulators
  pinned behind them, keep these at 20 or more);
* a compiler write of an accumulator that an inline-asm MFMA reads as C
  within 4 wait states before it (the zeroing of O, once sunk next to the
  first output MFMA of the d = 256 general-mask kernel).

The device code is compiled with the library's own flags.  The checker itself
is tested on small hand-written listings, including the cases it must flag.
"""
import os
import shutil
import subprocess

import pytest

from exact_attention_21_amd import _build
from tests import isa_check as ic

HAVE_HIPCC = shutil.which("hipcc") is not None or os.path.exists("/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory) -> str:
    tmp = tmp_path_factory.mktemp("isa")
    cmd = [c for c in _build.build_command(str(tmp / "unused.so")) if c not in ("-shared", "-fPIC")]
    i = cmd.index("-o")
    cmd[i + 1] = str(tmp / "fa2.s")
    cmd[1:1] = ["--cuda-device-only", "-S"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return (tmp / "fa2.s").read_text()


@pytest.mark.skipif(not HAVE_HIPCC, reason="hipcc not available")
def test_no_hazard_around_inline_asm_mfmas(device_asm):
    results = ic.check_text(device_asm)
    assert len(results) >= 50, "expected every kernel instantiation in the assembly"
    offenders = [f"{name[:60]}: {kind}: {msg}" for name, found in results.items() for kind, msg in found]
    assert not offenders, "\n".join(offenders[:10])
    # Not vacuous: the kernels with O in AGPRs (d >= 128) hold inline-asm
    # MFMAs whose accumulators the compiler reads afterwards.
    bodies = ic.kernel_bodies(device_asm)
    with_asm = [n for n, items in bodies.items()
                if any(not isinstance(x, str) and x.asm and ic.MFMA_RE.match(x.text) for x in items)]
    assert len(with_asm) >= 24, len(with_asm)


# ---- the checker on hand-written listings ---------------------------------

def _listing(body: str) -> str:
    return "_ZN3fa214fa2_fwd_kernelTEST:\n" + body + "\n.Lfunc_end0:\n"


ASM_MFMA = "\t;;#ASMSTART\n\tv_mfma_f32_32x32x16_f16 a[0:15], v[2:5], v[6:9], a[0:15]\n\t;;#ASMEND\n"
NOPS = "\t;;#ASMSTART\n\ts_nop 7\n s_nop 7\n s_nop 3\n\t;;#ASMEND\n"


def _kinds(body):
    return sorted(k for k, _ in ic.check_text(_listing(body))["_ZN3fa214fa2_fwd_kernelTEST"])


def test_checker_flags_read_right_after_asm_mfma():
    assert _kinds(ASM_MFMA + "\tv_add_u32_e32 v1, 1, v1\n\tv_accvgpr_read_b32 v10, a3\n") == \
        ["agpr_read_after_asm_mfma"]


def test_checker_accepts_read_after_the_wait():
    assert _kinds(ASM_MFMA + NOPS + "\tv_accvgpr_read_b32 v10, a3\n") == []


def test_checker_ignores_other_registers():
    assert _kinds(ASM_MFMA + "\tv_accvgpr_read_b32 v10, a16\n") == []


def test_checker_follows_branches():
    # The read sits in a block reached only by a branch taken right after the
    # MFMA; the wait on the fall-through path does not help it.
    body = (ASM_MFMA + "\ts_cbranch_scc1 .LBB0_2\n" + NOPS + "\ts_endpgm\n"
            ".LBB0_2:\n\tv_accvgpr_read_b32 v10, a0\n\ts_endpgm\n")
    assert _kinds(body) == ["agpr_read_after_asm_mfma"]
    body_ok = (ASM_MFMA + NOPS + "\ts_cbranch_scc1 .LBB0_2\n\ts_endpgm\n"
               ".LBB0_2:\n\tv_accvgpr_read_b32 v10, a0\n\ts_endpgm\n")
    assert _kinds(body_ok) == []


def test_checker_follows_loop_back_edges():
    # The read at the top of a loop body follows the asm MFMA at its bottom.
    body = (".LBB0_1:\n\tv_accvgpr_read_b32 v10, a5\n\ts_nop 3\n" + ASM_MFMA +
            "\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    assert _kinds(body) == ["agpr_read_after_asm_mfma"]


def test_checker_flags_compiler_mfma_reading_the_accumulator():
    body = ASM_MFMA + "\tv_mfma_f32_32x32x16_f16 a[0:15], v[2:5], v[6:9], a[0:15]\n"
    assert _kinds(body) == ["agpr_read_after_asm_mfma"]


def test_checker_flags_operand_writes_before_asm_mfma():
    assert _kinds("\tv_cvt_pk_f16_f32 v7, v1, v2\n" + ASM_MFMA) == ["valu_write_before_asm_mfma"]
    assert _kinds("\tv_accvgpr_write_b32 a4, v1\n\ts_nop 0\n" + ASM_MFMA) == ["agpr_write_before_asm_mfma"]
    assert _kinds("\tv_cvt_pk_f16_f32 v7, v1, v2\n\ts_nop 4\n" + ASM_MFMA) == []


def test_checker_operand_write_superseded_by_a_load():
    # A VALU write of an operand register that a load then overwrites: the
    # MFMA reads the load's result (awaited by s_waitcnt), not the VALU's.
    load = "\tds_read_b64 v[2:3], v2\n\ts_waitcnt lgkmcnt(0)\n"
    assert _kinds("\tv_add_u32_e32 v2, 0, v2\n" + load + ASM_MFMA) == []
    # The load covers v2 and v3 only: a write of v4 still counts.
    assert _kinds("\tv_add_u32_e32 v4, 0, v4\n" + load + ASM_MFMA) == ["valu_write_before_asm_mfma"]
    # A load straight into LDS writes no VGPR (its first operand is an address).
    assert _kinds("\tv_add_u32_e32 v2, 0, v2\n\tbuffer_load_dword v2, s[0:3], 0 offen lds\n" + ASM_MFMA) == \
        ["valu_write_before_asm_mfma"]


def test_checker_flags_inline_asm_valu_writes():
    asm_xor = "\t;;#ASMSTART\n\tv_xor_b32 v6, s1, v6\n\t;;#ASMEND\n"
    assert _kinds(asm_xor + ASM_MFMA) == ["valu_write_before_asm_mfma"]
    assert _kinds(asm_xor + "\tds_read_b128 v[6:9], v6\n\ts_waitcnt lgkmcnt(0)\n" + ASM_MFMA) == []
