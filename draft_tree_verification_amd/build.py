"""Build step for libtev.so: hipcc for gfx950, in-tree.

Each HIP source in ``csrc/`` is compiled to an object of its own (in
parallel), then the objects are linked into
``draft_tree_verification_amd/_build/libtev.so``.  No device function crosses
a translation unit, so no relocatable device code is involved.  Packed fp32
vector ops are disabled for device code (``-packed-fp32-ops``); hipcc's host
pass warns that it does not know the feature, which is harmless.  MFMA
accumulators are kept in ordinary VGPRs (``-amdgpu-mfma-vgpr-form``): the
attention kernels fit their 256 registers per wave that way, with no copies
between register files.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libtev.so")
SOURCES = ["tev_api.hip", "exit_law.hip", "tree_attn.hip", "round.hip", "commit.hip",
           "exit_loss.hip", "tree_build.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
NOISE = "is not a recognized feature for this target"


def compile_flags(src: str) -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc_command(out: str = LIB, extra: list[str] | None = None) -> list[list[str]]:
    """The compile commands (one per source) followed by the link command."""
    objs = [os.path.join(OUT_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC] + compile_flags(s) + ["-c", os.path.join(CSRC, s), "-o", o] + (extra or [])
            for s, o in zip(SOURCES, objs)]
    cmds.append([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out] + objs)
    return cmds


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{errs}")
    return errs


def build(verbose: bool = False) -> str:
    """Compile libtev.so (always recompiles every source)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmds = hipcc_command(tmp)
    with ThreadPoolExecutor(max_workers=min(len(cmds) - 1, os.cpu_count() or 1)) as ex:
        logs = list(ex.map(_run, cmds[:-1]))
    logs.append(_run(cmds[-1]))
    if verbose:
        for l in logs:
            if l.strip():
                print(l, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
