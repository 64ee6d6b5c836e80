"""GPU parity of kda_prefill against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, check_prefill, gpu_prefill, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_prefill_amd.kda as k
    k.lib()


# -- small shapes: several chunks plus a ragged tail, every head-size pairing --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_small_ragged(dtype, dk, dv):
    x = gen.make_prefill(31, [200], H=3, dk=dk, dv=dv, dtype=dtype, mu=3.0, state_std=0.02)
    check_prefill(x, label=f"small {dk}x{dv}")


@pytest.mark.parametrize("d", [64, 128])
def test_hand_worked_example(d):
    """The two-token example of tests/golden/, worked by hand, in d channels."""
    from golden_case import load
    x, o_ref, fin_ref = load(d=d, H=3)
    o, fin = gpu_prefill(x)
    assert np.abs(host(o) - o_ref).max() < 1e-5
    assert np.abs(host(fin) - fin_ref).max() < 1e-5


def test_config1_tiny_fp32():
    x = gen.config_prefill(1)
    check_prefill(x, label="config 1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_edges(dtype):
    """Lengths around the chunk size, a zero-length sequence, nonzero states."""
    lens = [1, 63, 64, 65, 0, 127, 4097, 2]
    x = gen.make_prefill(32, lens, H=2, dk=128, dv=128, dtype=dtype, mu=3.0, state_std=0.02,
                         packed=True)
    check_prefill(x, label="varlen edges")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64),
                                         ("f32", 64, 128)])
def test_many_chains(dtype, dk, dv):
    """More (sequence, head, 16-column) chains than the GPU has CUs, so the
    sequential kernel's workgroups (one CU each) run in several rounds: a
    packed batch of 40 sequences with an empty and a one-token one, nonzero
    initial states."""
    g = np.random.default_rng(33)
    lens = [int(n) for n in g.integers(0, 150, 40)]
    lens[3], lens[7] = 0, 1
    x = gen.make_prefill(33, lens, H=8, dk=dk, dv=dv, dtype=dtype, mu=3.0, state_std=0.02,
                         packed=True)
    check_prefill(x, label=f"many chains {dk}x{dv}")


def test_config2_single_sequence():
    x = gen.config_prefill(2)
    check_prefill(x, label="config 2")


def test_config3_packed_varlen_sampled():
    """Full packed batch on the GPU; the oracle checks 4 of the 16 sequences."""
    import torch
    x = gen.config_prefill(3)
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    o, fin = host(o), host(fin)
    lens = x.lengths()
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 3, 11})
    y = x.select_seqs(seqs)
    ro, rf = oracle.prefill(y.q, y.k, y.v, y.log_alpha, y.beta, y.initial_state, y.cu_seqlens)
    offs = np.concatenate([[0], np.cumsum(lens)])
    go = np.concatenate([o[offs[s]:offs[s + 1]] for s in seqs])
    eo, ef = rel_l2(go, ro), rel_l2(fin[seqs], rf)
    print(f"[parity] config 3 seqs {seqs} (T={x.T}): o={eo:.3e} state={ef:.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def test_config4_long_sampled_heads():
    """T = 65536 on the GPU; the oracle checks two heads over the whole sequence."""
    import torch
    x = gen.config_prefill(4)
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    heads = [0, 17]
    o_s = host(o[:, heads])
    f_s = host(fin[:, heads])
    y = x.select_heads(heads)
    ro, rf = oracle.prefill(y.q, y.k, y.v, y.log_alpha, y.beta, y.initial_state, None, num_seqs=1)
    eo, ef = rel_l2(o_s, ro), rel_l2(f_s, rf)
    print(f"[parity] config 4 heads {heads}: o={eo:.3e} state={ef:.3e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
