"""Compiles the HIP library (libmimopre.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmimopre.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["plan.cpp", "runtime.hip", "preprocess.hip", "vit_tables.hip", "patch_embed.hip", "hf_resize.hip",
           "pixel_embed.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MiMo pixel-path library needs ROCm's hipcc")


def compile_command(out_path: str) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 VALU instructions (v_pk_*_f32) anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the only fused multiply-adds are the explicit ones
        "-ffp-contract=off",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out_path,
    ]


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the path of the built library."""
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if msg.strip():
            print(msg)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
