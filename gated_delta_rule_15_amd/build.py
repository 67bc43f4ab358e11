"""Build the HIP library ``libkda.so`` in-tree with hipcc for gfx950.

Usage: ``python -m gated_delta_rule_15_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles all sources (objects go to ``gated_delta_rule_15_amd/_build``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libkda.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["kda_step.hip", "kda_compose.hip", "kda_prefill.hip", "kda_contract.hip", "kda_probe.hip", "kda_api.hip"]
# No contraction of separate multiplies and adds into fused operations where
# results must be bit-reproducible across code paths: the step kernels between
# decode, verify and commit; the prefill between its two workgroup shapes (the
# compiler's fusion choices could differ between the instantiations); the row
# contract between its one-row and sixteen-row instantiations.
PER_FILE_FLAGS = {"kda_step.hip": ["-ffp-contract=off"], "kda_prefill.hip": ["-ffp-contract=off"],
                  "kda_contract.hip": ["-ffp-contract=off"],
                  # the MFMA probe's accumulators in VGPRs: with AGPR accumulators the allocator
                  # rotated them between loop trips (48 accumulator moves per 32 MFMAs)
                  "kda_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU ops are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON_FLAGS, *PER_FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip() and verbose:
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
