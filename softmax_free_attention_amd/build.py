"""Build liblssar.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m softmax_free_attention_amd.build`` or through
``__graft_entry__.build()``.  The library is written next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "lssar.hip")
OUT = os.path.join(HERE, "liblssar.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are turned off for all device code.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               # MFMA results stay in ordinary VGPRs (no AGPR round trips)
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(out: str = OUT, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
