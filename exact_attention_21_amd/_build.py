"""Build step for the HIP library: one hipcc invocation for gfx950.

``build_library()`` compiles ``csrc/fa2_api.hip`` (which includes the kernel
header) into ``libfa2.so`` next to this file.  It always recompiles.
``build_variant()`` builds the same sources with design switches flipped
(``-D`` defines, see the top of ``csrc/fa2_kernel.hpp``) into
``_build/variants/``, for measuring what each choice is worth.
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libfa2.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "fa2_api.hip")]
ARCH = "gfx950"
VARIANT_DIR = os.path.join(PKG_DIR, "_build", "variants")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked at $HIPCC, /opt/rocm/bin/hipcc and PATH)")


def build_command(out: str = LIB_PATH, defines: dict | None = None) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        # Packed fp32 VALU forms are kept out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results in arch VGPRs unless a kernel asks for AGPRs: the
        # softmax reads the score accumulators with VALU instructions.
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(REPO_DIR, "include"),
        "-I", os.path.join(PKG_DIR, "csrc"),
        *(f"-D{k}={int(v)}" for k, v in sorted((defines or {}).items())),
        *SOURCES, "-o", out,
    ]


def _compile(out: str, defines: dict | None, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = build_command(tmp, defines)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    return _compile(LIB_PATH, None, verbose)


def variant_path(name: str) -> str:
    return os.path.join(VARIANT_DIR, f"libfa2_{name}.so")


def build_variant(name: str, defines: dict, verbose: bool = False) -> str:
    """The library with the given design switches, as _build/variants/libfa2_<name>.so."""
    os.makedirs(VARIANT_DIR, exist_ok=True)
    return _compile(variant_path(name), defines, verbose)


if __name__ == "__main__":
    print(build_library(verbose=True))
