"""The C ABI without a GPU: the library loads, exports every function that
include/kda.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_prefill_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

A = 1 << 20  # a 16-byte-aligned fake device address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert "kda_prefill" in names and "kda_decode_step" in names
    assert set(names) == set(kda.SIGNATURES), (names, sorted(kda.SIGNATURES))


def test_library_exports_every_declared_symbol():
    lib = kda.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.kda_version() >= 100


def test_status_strings():
    for s in range(5):
        assert kda.status_string(s).startswith("KDA_")
    assert kda.status_string(99) == "unknown kda_status"


def test_workspace_bytes():
    w = kda.workspace_bytes(4096, 1, 32, 128, 128, True)
    chunks = 4096 // 64 + 1
    per_chunk_head = 2 * (64 * 128 * 3 + 64 * 64 + 128 * 64) + 128 * 4
    assert w >= chunks * 32 * per_chunk_head
    assert w % 256 == 0
    assert kda.workspace_bytes(0, 1, 1, 64, 64, False) > 0
    assert kda.workspace_bytes(10, 0, 1, 64, 64, False) == 0
    assert kda.workspace_bytes(-1, 1, 1, 64, 64, False) == 0


def _prefill(**kw):
    args = dict(q=A, k=A, v=A, la=A, beta=A, s0=None, cu=None, T=128, N=1, H=2, dk=64, dv=64,
                dtype=kda.KDA_DTYPE_BF16, o=A, fin=None, ws=A, wsb=1 << 40, stream=None)
    args.update(kw)
    lib = kda.lib()
    return lib.kda_prefill(args["q"], args["k"], args["v"], args["la"], args["beta"], args["s0"],
                           args["cu"], args["T"], args["N"], args["H"], args["dk"], args["dv"],
                           args["dtype"], args["o"], args["fin"], args["ws"], args["wsb"],
                           args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=-5), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=1 << 31), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dv=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=7), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=129, N=2), kda.KDA_ERR_INVALID_ARGUMENT),    # unequal rows need cu_seqlens
    (dict(q=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(o=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(k=A + 4), kda.KDA_ERR_INVALID_ARGUMENT),       # misaligned
    (dict(ws=None, wsb=10), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(wsb=100), kda.KDA_ERR_WORKSPACE),
])
def test_prefill_rejects_before_any_hip_call(kw, status):
    assert _prefill(**kw) == status
    assert kda.last_error()  # a message explains it


def _decode(**kw):
    args = dict(state=A, q=A, k=A, v=A, la=A, beta=A, N=4, H=2, dk=128, dv=128,
                dtype=kda.KDA_DTYPE_BF16, o=A, stream=None)
    args.update(kw)
    return kda.lib().kda_decode_step(args["state"], args["q"], args["k"], args["v"], args["la"],
                                     args["beta"], args["N"], args["H"], args["dk"], args["dv"],
                                     args["dtype"], args["o"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=2), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(state=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(beta=A + 8), kda.KDA_ERR_INVALID_ARGUMENT),
])
def test_decode_rejects_before_any_hip_call(kw, status):
    assert _decode(**kw) == status
    assert kda.last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kda, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(ImportError):
        kda.lib()


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "gated_delta_rule_prefill_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "kda_oracle" not in text and "liboracle" not in text, f


def _prefill_ex(flags=0, cs=None, **kw):
    args = dict(q=A, k=A, v=A, la=A, beta=A, s0=None, cu=None, T=128, N=1, H=2, dk=64, dv=64,
                dtype=kda.KDA_DTYPE_BF16, o=A, fin=None, ws=A, wsb=1 << 40, stream=None)
    args.update(kw)
    return kda.lib().kda_prefill_ex(args["q"], args["k"], args["v"], args["la"], args["beta"],
                                    args["s0"], args["cu"], args["T"], args["N"], args["H"],
                                    args["dk"], args["dv"], args["dtype"], flags, args["o"],
                                    args["fin"], cs, args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(flags=4), kda.KDA_ERR_INVALID_ARGUMENT),        # unknown option bit
    (dict(flags=1 << 31), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(cs=A + 8), kda.KDA_ERR_INVALID_ARGUMENT),       # misaligned chunk states
    (dict(flags=3, dk=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(flags=3, wsb=100), kda.KDA_ERR_WORKSPACE),
])
def test_prefill_ex_rejects_before_any_hip_call(kw, status):
    assert _prefill_ex(**kw) == status


def _decode_tokens(**kw):
    args = dict(pool=A, slots=A, q=A, k=A, v=A, la=A, beta=A, cu=None, T=8, N=2, H=2, dk=64,
                dv=64, P=4, dtype=kda.KDA_DTYPE_BF16, flags=0, o=A, stream=None)
    args.update(kw)
    return kda.lib().kda_decode_tokens(args["pool"], args["P"], args["slots"], args["q"], args["k"],
                                       args["v"], args["la"], args["beta"], args["cu"], args["T"],
                                       args["N"], args["H"], args["dk"], args["dv"],
                                       args["dtype"], args["flags"], args["o"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(N=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(H=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=7), kda.KDA_ERR_INVALID_ARGUMENT),           # unequal rows need cu_seqlens
    (dict(slots=None, P=1), kda.KDA_ERR_INVALID_ARGUMENT),   # identity slots need P >= N
    (dict(pool=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(q=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(slots=A + 4), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(flags=8), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dtype=3), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dv=32), kda.KDA_ERR_UNSUPPORTED),
])
def test_decode_tokens_rejects_before_any_hip_call(kw, status):
    assert _decode_tokens(**kw) == status


def _backward(**kw):
    args = dict(q=A, k=A, v=A, la=A, beta=A, s0=None, cu=None, T=128, N=1, H=2, dk=64, dv=64,
                dtype=kda.KDA_DTYPE_BF16, do=A, dfin=None, cs=None, dq=A, dk_=A, dv_=A, dla=A,
                db=A, ds0=None, ws=A, wsb=1 << 40, stream=None)
    args.update(kw)
    a = args
    return kda.lib().kda_backward(a["q"], a["k"], a["v"], a["la"], a["beta"], a["s0"], a["cu"],
                                  a["T"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], a["do"],
                                  a["dfin"], a["cs"], a["dq"], a["dk_"], a["dv_"], a["dla"],
                                  a["db"], a["ds0"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(T=129, N=2), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(do=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dla=None), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(cs=A + 4), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(dk=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=5), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(wsb=64), kda.KDA_ERR_WORKSPACE),
])
def test_backward_rejects_before_any_hip_call(kw, status):
    assert _backward(**kw) == status


def test_backward_workspace_bytes():
    w = kda.backward_workspace_bytes(4096, 1, 32, 128, 128, True)
    assert w >= kda.workspace_bytes(4096, 1, 32, 128, 128, True) and w % 256 == 0
    assert kda.backward_workspace_bytes(10, 0, 1, 64, 64, False) == 0


def test_noalloc_rejects_sizes_beyond_its_array_before_any_hip_call():
    lib = kda.lib()
    scratch = 64 << 20
    assert lib.kda_prefill_workspace_bytes(1280, 1, 32, 128, 128, kda.KDA_DTYPE_BF16) <= scratch
    assert lib.kda_prefill_workspace_bytes(1344, 1, 32, 128, 128, kda.KDA_DTYPE_BF16) > scratch
    st = lib.kda_prefill_noalloc(A, A, A, A, A, None, None, 1344, 1, 32, 128, 128,
                                 kda.KDA_DTYPE_BF16, A, None, None)
    assert st == kda.KDA_ERR_WORKSPACE and "fixed scratch" in kda.last_error()
    st = lib.kda_prefill_noalloc(A, A, A, A, A, None, None, 128, 0, 2, 64, 64,
                                 kda.KDA_DTYPE_BF16, A, None, None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "kda.h"

int main(void) {
    if (kda_version() <= 0) return 1;
    if (strcmp(kda_status_string(KDA_ERR_WORKSPACE), "KDA_ERR_WORKSPACE") != 0) return 2;
    size_t ws = kda_prefill_workspace_bytes(4096, 1, 32, 128, 128, KDA_DTYPE_BF16);
    if (ws == 0 || ws % 256 != 0) return 3;
    /* an unsupported head size is rejected before any HIP call */
    kda_status st = kda_prefill(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 64, 1, 1, 96, 128,
                                KDA_DTYPE_BF16, NULL, NULL, NULL, 0, NULL);
    if (st != KDA_ERR_UNSUPPORTED) return 4;
    if (strlen(kda_last_error_message()) == 0) return 5;
    printf("ok %zu\n", ws);
    return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/kda.h compiles as C11 and a C program links against libkda.so
    and calls its host-side entry points (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    lib_dir = os.path.dirname(kda.LIB_PATH)
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    src = tmp_path / "use_kda.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "use_kda"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    cmd = [gcc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(root, "include"), str(src),
           "-o", str(exe), kda.LIB_PATH, f"-Wl,-rpath,{lib_dir}",
           "-Wl,-rpath,/opt/rocm/lib"]
    # under the host sanitizer run the library is instrumented: link its runtime too
    cmd += [p for p in os.environ.get("LD_PRELOAD", "").split(":") if "asan" in p]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.startswith("ok"), (run.returncode, run.stdout, run.stderr)
