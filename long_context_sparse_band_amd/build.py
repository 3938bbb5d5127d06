"""Build liblfattn.so (the HIP library) in-tree with hipcc for gfx950."""

from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblfattn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def command(out: str):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            # Packed fp32 VALU forms are kept out of the generated code.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # The leading scalar kernel arguments (the work-table pointer of
            # the band and backward kernels, the record base, list extents and
            # geometry of the merge kernels) arrive preloaded in SGPRs.
            "-mllvm", "-amdgpu-kernarg-preload-count=11",
            "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
            *sources(), "-o", out]


def build() -> str:
    """Compile every HIP source into liblfattn.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    proc = subprocess.run(command(tmp), capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
