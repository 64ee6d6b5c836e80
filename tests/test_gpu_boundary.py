"""The C ABI called directly through ctypes on the GPU: kda_prefill (the
two-call boundary's own prefill, without the _ex options) against the fp64
oracle, the per-thread kernel timing, and the KDA_DEBUG_SYNC offset check."""
import os
import subprocess
import sys
import threading

import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import assert_units, device_inputs, host, oracle_prefill, unit_errors

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("packed", [True, False])
def test_kda_prefill_c_abi(dtype, packed):
    """kda_prefill through ctypes with a caller workspace, and again with
    NULL/0 (the library's stream-ordered allocation)."""
    import torch
    from gated_delta_rule_prefill_amd import kda as b
    lens = [150, 0, 64, 1, 99] if packed else [96, 96, 96]
    x = gen.make_prefill(71, lens, H=4, dk=128, dv=128, dtype=dtype, state_std=0.02,
                         packed=packed)
    d = device_inputs(x)
    T, H, dk, dv, N = x.T, x.H, x.dk, x.dv, x.num_seqs
    code = b.KDA_DTYPE_BF16 if dtype == "bf16" else b.KDA_DTYPE_F32
    lib = b.lib()
    ro, rf = oracle_prefill(x)
    need = lib.kda_prefill_workspace_bytes(T, N, H, dk, dv, code)
    assert need > 0
    stream = torch.cuda.current_stream().cuda_stream
    for ws_given in (True, False):
        o = torch.full((T, H, dv), float("nan"), dtype=d["q"].dtype, device="cuda")
        fin = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if ws_given else None
        st = lib.kda_prefill(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                             d["log_alpha"].data_ptr(), d["beta"].data_ptr(),
                             d["initial_state"].data_ptr(),
                             d["cu_seqlens"].data_ptr() if packed else None,
                             T, N, H, dk, dv, code, o.data_ptr(), fin.data_ptr(),
                             ws.data_ptr() if ws_given else None, need if ws_given else 0,
                             stream)
        assert st == b.KDA_OK, b.last_error()
        torch.cuda.synchronize()
        errs = unit_errors(host(o), ro, host(fin), rf, x.lengths())
        assert_units(errs, dtype, f"kda_prefill C ABI packed={packed} workspace={ws_given}")


def test_kernel_timing_is_per_thread():
    """Timing enabled on one thread records that thread's calls only."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x = gen.make_prefill(72, [256], H=2, dk=64, dv=64, dtype="bf16")
    d = device_inputs(x)
    res = {}

    def timed():
        torch.cuda.set_device(0)
        kda.set_kernel_timing(True)
        kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
        res["timed"] = kda.prefill_kernel_times()
        kda.set_kernel_timing(False)

    def untimed():
        torch.cuda.set_device(0)
        kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
        try:
            kda.prefill_kernel_times()
            res["untimed"] = "recorded"
        except RuntimeError:
            res["untimed"] = "none"

    for fn in (timed, untimed):
        th = threading.Thread(target=fn)
        th.start()
        th.join()
    names = [n for n, _ in res["timed"]]
    assert names == ["prefill_intra", "prefill_state"], res
    assert all(ms > 0 for _, ms in res["timed"]), res
    assert res["untimed"] == "none", res


_DEBUG_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from gated_delta_rule_prefill_amd import kda as b
from gated_delta_rule_prefill_amd import inputs as gen
sys.path.insert(0, sys.argv[1] + '/tests')
from gpu_util import device_inputs
x = gen.make_prefill(73, [100, 100], H=2, dk=64, dv=64, dtype="bf16", packed=True)
d = device_inputs(x)
lib = b.lib()
out = []
# offsets that stay inside [0, T]: a first offset of 1, then a last offset short of T
for cu in ([1, 100, 200], [0, 100, 150], [0, 100, 200]):
    c = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o = torch.empty((200, 2, 64), dtype=torch.bfloat16, device="cuda")
    st = lib.kda_prefill(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                         d["log_alpha"].data_ptr(), d["beta"].data_ptr(), None, c.data_ptr(),
                         200, 2, 2, 64, 64, b.KDA_DTYPE_BF16, o.data_ptr(), None, None, 0,
                         torch.cuda.current_stream().cuda_stream)
    out.append(f"{st}:{b.last_error()}")
torch.cuda.synchronize()
print("RESULT|" + "|".join(out), flush=True)
"""


def test_debug_sync_checks_offsets():
    """With KDA_DEBUG_SYNC=1 a first offset other than 0 and a last offset
    other than T are rejected (KDA_ERR_INVALID_ARGUMENT) before any kernel."""
    env = dict(os.environ, KDA_DEBUG_SYNC="1")
    r = subprocess.run([sys.executable, "-c", _DEBUG_CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("RESULT|")]
    assert r.returncode == 0 and line, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    res = line[0].split("|")[1:]
    print("[debug sync]", res, flush=True)
    assert res[0].startswith("1:") and "cu_seqlens[0]" in res[0]
    assert res[1].startswith("1:") and "cu_seqlens[N]" in res[1]
    assert res[2].startswith("0:")
