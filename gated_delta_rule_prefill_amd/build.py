"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m gated_delta_rule_prefill_amd.build`` or ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
KERNEL_SOURCES = ["chunk_table.hip", "prefill_intra.hip", "prefill_state.hip", "prefill_chain.hip",
                  "decode.hip", "recurrent.hip", "backward.hip", "backward_chunk.hip",
                  "kda_noalloc.hip"]
HOST_SOURCES = ["kda_api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", CSRC, "-I", INCLUDE]
# Packed fp32 ALU forms are left to no one: the feature is switched off for
# device code (the host pass warns that it does not know it; harmless).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-ffp-contract=fast", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libkda needs the ROCm toolchain")


# Per-source extra flags.  backward.hip: with packed fp32 switched off, the
# SLP vectoriser's v2f32 conversions trip instruction selection (a compiler
# crash); that file's kernels gain nothing from it anyway.
EXTRA = {"backward.hip": ["-fno-slp-vectorize"]}


def _compile(src: str, device: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + (DEVICE + ["-x", "hip"] if device else []) + \
        EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libkda.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(8, len(os.sched_getaffinity(0)))
    work = [(s, True) for s in KERNEL_SOURCES] + [(s, False) for s in HOST_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda a: _compile(*a), work))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
