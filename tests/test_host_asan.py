"""Host AddressSanitizer run of the library's C entry points (no GPU needed).

The host-code sources (the C ABI in kda_api.cpp and the allocation-free entry
point in kda_noalloc.hip) are rebuilt with AddressSanitizer on their host
pass only (device code is built as usual), linked with the regular device
objects, and the CPU boundary tests run against that library in a child
process with the sanitizer runtime preloaded.  Every validation path, the
workspace-size arithmetic, the status strings and the thread-local error text
run under it; any heap or stack overflow, use after free or double free in
the host code fails the test.
"""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_CODE = ["kda_api.cpp", "kda_noalloc.hip"]


def _asan_runtime(hipcc: str) -> str:
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(cand):
            out = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True).stdout.strip()
            if out and os.path.isabs(out) and os.path.exists(out):
                return out
    return ""


def _build_asan_library(out_dir: str) -> str:
    from gated_delta_rule_prefill_amd import build as kb
    hipcc = kb.hipcc()
    device_objs = [os.path.join(kb.BUILD_DIR, s + ".o") for s in kb.KERNEL_SOURCES if s not in HOST_CODE]
    if not all(os.path.exists(o) for o in device_objs):
        kb.build()
    objs = []
    for src in HOST_CODE:
        obj = os.path.join(out_dir, src + ".o")
        device = src.endswith(".hip")
        cmd = [hipcc] + kb.COMMON + ["-g", "-O1"] + (kb.DEVICE + ["-x", "hip"] if device else []) + \
            ASAN_HOST + ["-c", os.path.join(kb.CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        objs.append(obj)
    lib = os.path.join(out_dir, "libkda_asan.so")
    cmd = [hipcc, f"--offload-arch={kb.ARCH}", "-shared", "-fPIC", "-o", lib] + objs + device_objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return lib


CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
ctypes.CDLL(None)["__asan_init"]            # the sanitizer runtime is in the process
import gated_delta_rule_prefill_amd.kda as kda
kda.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {target!r}]))
"""


def test_boundary_under_host_asan(tmp_path):
    try:
        from gated_delta_rule_prefill_amd import build as kb
        hipcc = kb.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    runtime = _asan_runtime(hipcc)
    if not runtime:
        pytest.skip("no AddressSanitizer runtime next to the ROCm clang")
    lib = _build_asan_library(str(tmp_path))
    # the host code really is instrumented
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm and "__asan_report_store" in nm
    child = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                         target=os.path.join(ROOT, "tests", "test_boundary_cpu.py"))
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                         timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
