"""Build libkda.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(_HERE, "csrc")
SOURCES = ["kda_api.cpp", "kda_gate.hip", "kda_decode.hip", "kda_chunk.hip", "kda_fused.hip",
           "kda_validate.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code; hipcc's host pass warns that it does
# not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # keep MFMA accumulators in VGPRs (no AGPR round trips when VALU touches them)
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def lib_path() -> str:
    return os.path.join(_HERE, "libkda.so")


def build_library(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object (in parallel) and link libkda.so."""
    bdir = os.path.join(_HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Wno-unused-function", *DEVICE_FLAGS, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs.pop(0))
    while procs:
        _drain(procs.pop(0))
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _drain(item):
    src, proc = item
    out, _ = proc.communicate()
    text = out.decode(errors="replace")
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        sys.stderr.write(text + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if text.strip():
        sys.stderr.write(text + "\n")


if __name__ == "__main__":
    print(build_library(verbose=True))
