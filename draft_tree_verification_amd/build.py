"""Build step for libtev.so: hipcc for gfx950, in-tree.

The library is built from the HIP sources in ``csrc/`` into
``draft_tree_verification_amd/_build/libtev.so``.  Packed fp32 vector ops are
disabled for device code (``-packed-fp32-ops``); hipcc's host pass warns that it
does not know the feature, which is harmless.  MFMA accumulators are kept in
ordinary VGPRs (``-amdgpu-mfma-vgpr-form``): the attention kernel fits its 256
registers per wave that way, with no copies between register files.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libtev.so")
SOURCES = ["tev_api.hip", "exit_law.hip", "tree_attn.hip", "round.hip", "commit.hip",
           "exit_loss.hip", "tree_build.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return ([HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-o", out] + [os.path.join(CSRC, s) for s in SOURCES] + (extra or []))


def build(verbose: bool = False) -> str:
    """Compile libtev.so (always recompiles)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
