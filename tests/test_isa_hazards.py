"""The output MFMAs that keep O in AGPRs are inline asm, so the compiler
inserts no wait states between a VALU write of one of their VGPR operands and
the MFMA that reads it.  The kernels keep such writes (the packing of P) away
from those MFMAs; this test compiles the device code with the library's own
flags and checks the generated gfx950 assembly: no inline-asm MFMA may read a
VGPR that one of the four instructions before it writes with a VALU
instruction.  (The compiler once moved the last P pack right in front of the
first output MFMA of a tile, which then read a stale value on some runs.)"""
import os
import re
import shutil
import subprocess

import pytest

from exact_attention_21_amd import _build

ASM_MFMA = re.compile(r"v_mfma_f32_32x32x16_\w+ a\[\d+:\d+\], v\[(\d+):(\d+)\], v\[(\d+):(\d+)\]")
VALU_DST = re.compile(r"(v_\w+)\s+v\[?(\d+)(?::(\d+))?")


def device_asm(tmp_path) -> str:
    cmd = [c for c in _build.build_command(str(tmp_path / "unused.so")) if c not in ("-shared", "-fPIC")]
    i = cmd.index("-o")
    cmd[i + 1] = str(tmp_path / "fa2.s")
    cmd[1:1] = ["--cuda-device-only", "-S"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return (tmp_path / "fa2.s").read_text()


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_valu_write_right_before_asm_output_mfma(tmp_path):
    text = device_asm(tmp_path)
    names = re.findall(r"^(_ZN3fa2\S*_kernel\S*):", text, re.M)
    assert len(names) >= 40, "expected every kernel instantiation in the assembly"
    offenders = []
    for name in names:
        start = text.index(name + ":")
        body = [l.strip() for l in text[start:text.index(".Lfunc_end", start)].splitlines()]
        code = [l for l in body if l and not l.startswith((";", ".", "//")) and not l.endswith(":")]
        for i, line in enumerate(code):
            m = ASM_MFMA.search(line)
            if not m:
                continue
            a0, a1, b0, b1 = map(int, m.groups())
            srcs = set(range(a0, a1 + 1)) | set(range(b0, b1 + 1))
            for prev in code[max(0, i - 4):i]:
                w = VALU_DST.match(prev)
                if not w or prev.startswith(("v_mfma", "v_accvgpr_read", "v_smfmac")):
                    continue
                lo = int(w.group(2))
                hi = int(w.group(3)) if w.group(3) else lo
                if srcs & set(range(lo, hi + 1)):
                    offenders.append(f"{name[:60]}: '{prev}' before '{line}'")
    assert not offenders, "\n".join(offenders[:10])
