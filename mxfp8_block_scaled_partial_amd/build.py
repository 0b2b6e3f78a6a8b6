"""Build libmxfp8partial.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package dir.

Run ``python -m mxfp8_block_scaled_partial_amd.build``; ``__graft_entry__.build()`` calls it.
``--ablation`` also builds libmxfp8partial_guards.so from the same sources with
MXFP8_RUNTIME_GUARDS=1: the amax and the plain cast of rows of whole 16-byte chunks run one
kernel per dtype for row-only and bidirectional calls, their column-wise work selected at run
time by the column-wise pointer (the kernels the pages measured before the compile-time
specialization).  It exists for the benchmark's ``--ablation`` timing and its parity test
only; the product is libmxfp8partial.so.
"""
from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmxfp8partial.so")
GUARDS_LIB = os.path.join(HERE, "libmxfp8partial_guards.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "abi.cpp"),
           os.path.join(CSRC, "paths.cpp")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxfp8partial.so)")


def kernel_source_hash(path: str = os.path.join(CSRC, "kernels.hip")) -> str:
    """16 hex digits of SHA-256 over the kernel source with its comments and blank space
    removed (no string literal in it holds a comment marker): the identity of the kernels a
    build holds, unchanged by comment edits.  The library reports the hash it was built from
    (mxfp8_build_id), so measurements can be tied to the source they ran."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


def flags(runtime_guards: bool = False) -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed FP32 instructions are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-DMXFP8_RUNTIME_GUARDS={int(runtime_guards)}",
            f'-DMXFP8_KERNEL_SOURCE_HASH="{kernel_source_hash()}"',
            "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def _build(out: str, runtime_guards: bool, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc()] + flags(runtime_guards) + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, ablation: bool = False) -> str:
    """Builds the library (and with ``ablation`` the runtime-guard library); returns the
    library's path."""
    _build(LIB, False, verbose)
    if ablation:
        _build(GUARDS_LIB, True, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, ablation="--ablation" in sys.argv))
