"""Builds libsap.so (host planner, C ABI and gfx950 HIP kernels) in-tree.

    python long_context_sequence_doc_amd/build.py [--verbose] [--resource-usage]

Each source is compiled by hipcc for gfx950 into ``_build/`` and linked into
``long_context_sequence_doc_amd/libsap.so``. Packed-FP32 instructions are
disabled for device code (``-packed-fp32-ops``) and matrix-core results are
kept in VGPRs (``-amdgpu-mfma-vgpr-form``).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsap.so")

SOURCES = ["planner.cpp", "sap_api.cpp", "attn_fwd.hip", "lse_merge.hip", "attn_bwd.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"-I{os.path.join(ROOT, 'include')}"]
# Matrix-core results go straight to VGPRs (no AGPR staging copies in the
# softmax loops), and packed-FP32 instructions are disabled.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsap.so)")


def _compile(src: str, resource_usage: bool, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", "-o", obj] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    cmd += [os.path.join(CSRC, src)]
    if src.endswith(".hip"):
        if resource_usage:
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    # run in the build folder, so any temporaries hipcc leaves land there
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if verbose or resource_usage:
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.resource_usage))


if __name__ == "__main__":
    main()
