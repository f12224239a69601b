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

SOURCES = ["ra_api.cpp", "ra_fwd.hip", "ra_fwd_f32.hip", "ra_bwd.hip", "ra_misc.hip",
           "ra_noalloc.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    # Packed-fp32 VALU forms stay off: the kernels are written for scalar fp32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source code-generation flags (LLVM's AMDGPU backend).  The bf16 forward runs 2-3%
# faster under the iterative ILP instruction scheduler and the backward kernels 1.4%
# faster under the max-ILP one; the fp32 forward is 5-18% slower under either, so it
# sits in a file of its own with the default scheduler.  There, MFMA accumulators in
# VGPRs instead of AGPRs remove ~110 accumulator copies per key tile (the S init, S to
# the softmax, the O rescale), which cannot overlap the fp32 MFMAs: 2.9% faster on the
# d = 24 tabular forward.
SOURCE_FLAGS = {
    "ra_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "ra_fwd_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ra_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


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
        cmd = ([HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + inc + lang +
               ["-c", os.path.join(CSRC, src), "-o", obj])
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


HOST_SOURCES = ["ra_api.cpp"]  # the C ABI's host code: validation, drivers, host helpers


def build_host_sanitized(out_path: str, sanitizer: str = "address", cxx: str = "g++") -> str:
    """Links a copy of the library whose host code (HOST_SOURCES) is compiled with a
    sanitizer ("address" or "undefined"), reusing build()'s kernel objects (GPU code stays
    uninstrumented).  Undefined-behaviour reports abort the process.  An AddressSanitizer
    copy must be loaded in a process that preloads the sanitizer runtime."""
    build_dir = os.path.join(HERE, "_build")
    kernel_objs = [o for src, o in zip(SOURCES, _objects(build_dir)) if src not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in kernel_objs):
        build()
    san = [f"-fsanitize={sanitizer}"]
    if sanitizer == "undefined":
        san.append("-fno-sanitize-recover=undefined")
    out_dir = os.path.dirname(os.path.abspath(out_path))
    host_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + f".{sanitizer}.o")
        subprocess.run([cxx, "-fPIC"] + san + ["-fno-omit-frame-pointer", "-g", "-O1",
                        "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                        os.path.join(CSRC, src), "-o", obj], check=True)
        host_objs.append(obj)
    subprocess.run([cxx, "-shared"] + san + ["-o", out_path] + host_objs + kernel_objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return out_path


def build_host_asan(out_path: str, cxx: str = "g++") -> str:
    """build_host_sanitized with AddressSanitizer."""
    return build_host_sanitized(out_path, "address", cxx)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
