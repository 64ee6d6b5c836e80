"""GPU parity of kda_decode_step against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, dev_f32, dev_qkv, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_decode(seed, N, H, dk, dv, steps, dtype, sample=None):
    """Run `steps` decode tokens on the GPU and on the oracle (for the sampled
    (sequence, head) pairs); return the worst per-step o error and the state error."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    S0 = gen.decode_state(seed, N, H, dk, dv)
    state = dev_f32(S0)
    if sample is None:
        sample = [(s, h) for s in range(N) for h in range(H)]
    ss = np.array([p[0] for p in sample])
    hh = np.array([p[1] for p in sample])
    ref_state = S0[ss, hh][:, None].astype(np.float64).copy()   # [P,1,dk,dv]
    worst = 0.0
    for step in range(steps):
        x = gen.decode_token(seed, step, N, H, dk, dv, dtype=dtype)
        o = kda.decode_step(state, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v),
                            dev_f32(x.log_alpha), dev_f32(x.beta))
        ro = oracle.decode_step(ref_state, x.q[ss, hh][:, None], x.k[ss, hh][:, None],
                                x.v[ss, hh][:, None], x.log_alpha[ss, hh][:, None],
                                x.beta[ss, hh][:, None])
        worst = max(worst, rel_l2(host(o)[ss, hh], ro[:, 0]))
    torch.cuda.synchronize()
    es = rel_l2(host(state)[ss, hh], ref_state[:, 0])
    return worst, es


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, dk, dv):
    eo, es = run_decode(41, N=3, H=2, dk=dk, dv=dv, steps=8, dtype=dtype)
    print(f"[parity] decode {dk}x{dv} {dtype}: worst step o={eo:.3e} state={es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_config5_sampled():
    """256 sequences x 32 heads, 128 steps; the oracle follows 48 (sequence, head) pairs."""
    c = gen.DECODE_CONFIG
    g = np.random.default_rng(5)
    sample = [(int(s), int(h)) for s, h in zip(g.integers(0, c["N"], 48), g.integers(0, c["H"], 48))]
    eo, es = run_decode(c["seed"], c["N"], c["H"], c["dk"], c["dv"], c["steps"], c["dtype"], sample)
    print(f"[parity] decode config 5: worst step o={eo:.3e} state after 128={es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


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
