"""Build the gfx950 shared libraries in-tree with hipcc.

libmoeverify.so          -- the MoE verify-block library (C ABI in include/moe_verify.h)
workloads/libworkload_fill.so -- device twin of the seeded weight generator (inputs only)
"""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]

TARGETS = {
    os.path.join(PKG, "libmoeverify.so"): [os.path.join(PKG, "csrc", "moe_verify.hip")],
    os.path.join(PKG, "workloads", "libworkload_fill.so"): [os.path.join(PKG, "workloads", "fill.hip")],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 libraries)")


def build(verbose: bool = False) -> list[str]:
    """Compile every library (always; a stale library is never reused)."""
    built = []
    for out, srcs in TARGETS.items():
        tmp = out + ".tmp"
        cmd = [hipcc(), *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", *srcs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {out}:\n" + "\n".join(msgs))
        os.replace(tmp, out)
        built.append(out)
    return built


if __name__ == "__main__":
    for p in build(verbose=True):
        print("built", p)
