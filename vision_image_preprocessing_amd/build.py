"""Compiles the HIP library (libmimopre.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmimopre.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["plan.cpp", "runtime.hip", "preprocess.hip", "vit_tables.hip", "patch_embed.hip", "hf_resize.hip",
           "pixel_embed.hip"]
# Code-generation options of one source only.  The contrast kernel's
# matrix-core products chain through VALU shifts, so their accumulators
# belong in ordinary VGPRs; the GEMM kernels keep theirs in AGPRs.
SOURCE_FLAGS = {"hf_resize.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the only fused multiply-adds are the explicit ones
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MiMo pixel-path library needs ROCm's hipcc")


def compile_command(source: str, obj_path: str) -> list:
    """One source to one object (its device code for gfx950 included)."""
    return [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(source, []), "-I", INCLUDE, "-I", CSRC, "-c",
            os.path.join(CSRC, source), "-o", obj_path]


def link_command(objects: list, out_path: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objects, "-o", out_path]


def _run(cmd: list) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stdout + res.stderr


def build(verbose: bool = False) -> str:
    """Always recompiles (the sources in parallel); returns the path of the built library."""
    with tempfile.TemporaryDirectory(prefix="mimopre_build_") as tmpdir:
        objects = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        jobs = max(1, min(len(SOURCES), 16, os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            logs = list(pool.map(_run, [compile_command(s, o) for s, o in zip(SOURCES, objects)]))
        tmp = LIB_PATH + f".tmp{os.getpid()}"
        logs.append(_run(link_command(objects, tmp)))
    if verbose:
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in "".join(logs).splitlines() if noise not in l)
        if msg.strip():
            print(msg)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
