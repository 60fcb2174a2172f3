"""Compile the gfx950 HIP library in-tree: ``libfa_mi355x.so`` beside this file."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["fa_api.hip", "fa_fwd_mfma.hip", "fa_fwd_mfma16.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip",
           "fa_rope.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str = LIB_PATH) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Always recompiles; writes to a temporary name first so a failed build
    never leaves a half-written library behind."""
    tmp = LIB_PATH + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
