"""kda_prefill_noalloc (the entry point that allocates nothing; its workspace
is the library's fixed device array) through the C ABI against kda_prefill
with a caller workspace: two calls in a row, the second smaller, both equal to
the workspace path bit for bit and within tolerance of the fp64 oracle; sizes
beyond the fixed array are rejected before any HIP call."""
import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import assert_units, device_inputs, host, oracle_prefill, unit_errors

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _call(lib, fn, x, d, code, o, fin, ws=None):
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    args = [d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_alpha"].data_ptr(),
            d["beta"].data_ptr(),
            d["initial_state"].data_ptr() if d["initial_state"] is not None else None,
            d["cu_seqlens"].data_ptr() if d["cu_seqlens"] is not None else None,
            x.T, x.num_seqs, x.H, x.dk, x.dv, code, o.data_ptr(), fin.data_ptr()]
    if fn == "kda_prefill":
        args += [ws.data_ptr(), ws.numel()]
    return getattr(lib, fn)(*args, stream)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_path(dtype):
    import torch
    from gated_delta_rule_prefill_amd import kda as b
    lib = b.lib()
    code = b.KDA_DTYPE_BF16 if dtype == "bf16" else b.KDA_DTYPE_F32
    cases = [gen.make_prefill(91, [700, 0, 65, 300], H=8, dk=128, dv=128, dtype=dtype,
                              state_std=0.02, packed=True),
             gen.make_prefill(92, [130, 1], H=4, dk=64, dv=128, dtype=dtype, state_std=0.02,
                              packed=True)]
    for i, x in enumerate(cases):   # the second call is smaller than the first
        d = device_inputs(x)
        need = lib.kda_prefill_workspace_bytes(x.T, x.num_seqs, x.H, x.dk, x.dv, code)
        assert 0 < need <= SCRATCH_BYTES
        outs = []
        for fn in ("kda_prefill_noalloc", "kda_prefill"):
            o = torch.full((x.T, x.H, x.dv), float("nan"), dtype=d["q"].dtype, device="cuda")
            fin = torch.full((x.num_seqs, x.H, x.dk, x.dv), float("nan"), dtype=torch.float32,
                             device="cuda")
            ws = torch.empty(need, dtype=torch.uint8, device="cuda") if fn == "kda_prefill" else None
            st = _call(lib, fn, x, d, code, o, fin, ws)
            assert st == b.KDA_OK, (fn, b.last_error())
            torch.cuda.synchronize()
            outs.append((host(o), host(fin)))
        (o_n, f_n), (o_w, f_w) = outs
        assert np.array_equal(o_n, o_w) and np.array_equal(f_n, f_w), f"call {i}: differs"
        ro, rf = oracle_prefill(x)
        assert_units(unit_errors(o_n, ro, f_n, rf, x.lengths()), dtype, f"noalloc call {i}")


def test_noalloc_rejects_sizes_beyond_the_array():
    from gated_delta_rule_prefill_amd import kda as b
    lib = b.lib()
    T = 4096
    need = lib.kda_prefill_workspace_bytes(T, 1, 32, 128, 128, b.KDA_DTYPE_BF16)
    assert need > SCRATCH_BYTES
    A = 1 << 20   # never dereferenced: the call returns before any HIP call
    st = lib.kda_prefill_noalloc(A, A, A, A, A, None, None, T, 1, 32, 128, 128,
                                 b.KDA_DTYPE_BF16, A, None, None)
    assert st == b.KDA_ERR_WORKSPACE
    assert "fixed scratch" in b.last_error()
