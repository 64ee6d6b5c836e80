"""GPU parity of kda_decode_step against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import ROW_TOL, TOL, dev_f32, dev_qkv, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_decode(seed, N, H, dk, dv, steps, dtype):
    """Run `steps` decode tokens on the GPU and on the oracle for every
    (sequence, head).  Returns the worst whole-step o error, the worst
    (sequence, head) o error over all steps, the worst single o row, and the
    whole and worst (sequence, head) state errors after the last step."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    S0 = gen.decode_state(seed, N, H, dk, dv)
    state = dev_f32(S0)
    ref_state = S0.astype(np.float64)
    worst_step = worst_row = 0.0
    e2 = np.zeros((N, H))
    r2 = np.zeros((N, H))
    for step in range(steps):
        x = gen.decode_token(seed, step, N, H, dk, dv, dtype=dtype)
        o = kda.decode_step(state, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v),
                            dev_f32(x.log_alpha), dev_f32(x.beta))
        ro = oracle.decode_step(ref_state, x.q, x.k, x.v, x.log_alpha, x.beta)
        go = host(o)
        worst_step = max(worst_step, rel_l2(go, ro))
        de = ((go - ro) ** 2).sum(axis=2)
        dr = (ro ** 2).sum(axis=2)
        e2 += de
        r2 += dr
        worst_row = max(worst_row, float(np.max(np.sqrt(de) / np.maximum(np.sqrt(dr), 1e-300))))
    torch.cuda.synchronize()
    gs = host(state)
    es = rel_l2(gs, ref_state)
    unit_s = np.sqrt(((gs - ref_state) ** 2).sum(axis=(2, 3)) / (ref_state ** 2).sum(axis=(2, 3)))
    unit_o = np.sqrt(e2 / r2)
    return worst_step, float(unit_o.max()), worst_row, es, float(unit_s.max())


def _gate(res, dtype, label):
    eo, uo, ro, es, us = res
    print(f"[parity] decode {label} {dtype}: worst step o={eo:.3e}, worst (seq,head) o={uo:.3e}, "
          f"worst row={ro:.3e}; state={es:.3e}, worst (seq,head) state={us:.3e}", flush=True)
    assert max(eo, uo, es, us) <= TOL[dtype], res
    assert ro <= ROW_TOL[dtype], res


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, dk, dv):
    _gate(run_decode(41, N=3, H=2, dk=dk, dv=dv, steps=8, dtype=dtype), dtype, f"{dk}x{dv}")


def test_decode_config5_full():
    """256 sequences x 32 heads, 128 steps; the oracle follows every one of the
    8,192 (sequence, head) states through all 128 steps."""
    c = gen.DECODE_CONFIG
    _gate(run_decode(c["seed"], c["N"], c["H"], c["dk"], c["dv"], c["steps"], c["dtype"]),
          c["dtype"], "config 5 (all 8192 units, 128 steps)")


def test_hand_worked_example():
    """The two-token example of tests/golden/ as two decode steps."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    from golden_case import load
    x, o_ref, fin_ref = load(d=64, H=2)
    state = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    for t in range(2):
        o = kda.decode_step(state, dev_qkv(x.q[t:t + 1]), dev_qkv(x.k[t:t + 1]),
                            dev_qkv(x.v[t:t + 1]), dev_f32(x.log_alpha[t:t + 1]),
                            dev_f32(x.beta[t:t + 1]))
        assert np.abs(host(o)[0] - o_ref[t]).max() < 1e-5
    assert np.abs(host(state) - fin_ref).max() < 1e-5
