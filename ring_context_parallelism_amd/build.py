"""Builds libra.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

Usage: python -m ring_context_parallelism_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libra.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["ra_api.cpp", "ra_fwd.hip", "ra_bwd.hip", "ra_misc.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    # Packed-fp32 VALU forms stay off: the kernels are written for scalar fp32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _objects(build_dir):
    return [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link libra.so next to this file."""
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = []
    for src, obj in zip(SOURCES, _objects(build_dir)):
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS + inc + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + _objects(build_dir)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode != 0:
        sys.stderr.write(text)
        raise RuntimeError(f"hipcc failed on {src}")
    # hipcc's host pass does not know the packed-fp32 target feature; that note is noise.
    text = "\n".join(ln for ln in text.splitlines() if "is not a recognized feature" not in ln)
    if text.strip():
        sys.stderr.write(text + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
