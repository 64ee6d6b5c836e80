"""GPU parity of kda_prefill against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import assert_units, check_prefill, gpu_prefill, host, unit_errors

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


def test_tiny_T256_fp32():
    x = gen.workload_prefill("tiny_T256")
    check_prefill(x, label="tiny T=256")


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


def test_single_sequence_T4096():
    x = gen.workload_prefill("single_T4096")
    check_prefill(x, label="single sequence T=4096")


def test_packed_16_sequences_full():
    """The packed 16-sequence batch with nonzero initial states: every
    sequence and head against the oracle, gated per (sequence, head), per
    64-token chunk and per row."""
    import torch
    x = gen.workload_prefill("packed_16")
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    errs = unit_errors(host(o), ro, host(fin), rf, x.lengths())
    assert_units(errs, "bf16", f"packed 16 sequences, T={x.T}")


def test_long_T65536_all_heads():
    """T = 65536 on the GPU in one call; the oracle checks all 32 heads over the
    whole sequence, eight heads at a time (keeps its fp64 output near 0.5 GB)."""
    import torch
    x = gen.workload_prefill("long_T65536")
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    worst = None
    for h0 in range(0, x.H, 8):
        heads = list(range(h0, h0 + 8))
        y = x.select_heads(heads)
        ro, rf = oracle.prefill(y.q, y.k, y.v, y.log_alpha, y.beta, y.initial_state, None,
                                num_seqs=1)
        errs = unit_errors(host(o[:, h0:h0 + 8]), ro, host(fin[:, h0:h0 + 8]), rf, x.lengths())
        assert_units(errs, "bf16", f"T=65536 heads {h0}..{h0 + 7}")
        worst = errs if worst is None else {k: max(worst[k], errs[k]) if k != "worst_row" else
                                            worst[k] for k in errs}
    print(f"[parity] T=65536 all heads: worst o={worst['o']:.3e} state={worst['state']:.3e} "
          f"chunk={worst['chunk_o']:.3e} row={worst['row_o']:.3e}", flush=True)


# -- strong, mixed per-channel decay -------------------------------------------
# The pages single out the per-channel forgetting rate.  These draws push the
# summed log-decay of a 16-token block far from zero: mu = 0 gives about -13
# per block, mu = -1 about -22, and a fixed log_alpha = -3 on every even key
# channel gives -48 there next to the drawn odd channels (the kernels' stated
# range is a block sum above -80).
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("mu,fixed", [(0.0, None), (-1.0, None), (3.0, -3.0)])
def test_strong_decay(dtype, dk, dv, mu, fixed):
    lens = [200, 1, 64, 0, 131, 77]
    x = gen.make_prefill(35, lens, H=3, dk=dk, dv=dv, dtype=dtype, mu=mu, state_std=0.02,
                         packed=True, fixed_even_log_alpha=fixed)
    la = x.log_alpha.astype(np.float64)
    # the draw really is strong: some 16-token block sums beyond -12
    assert la[:16].sum(axis=0).min() < -12
    check_prefill(x, label=f"strong decay mu={mu} fixed={fixed} {dk}x{dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strong_decay_single_sequence(dtype):
    """Equal rows (no chunk table), strong mixed decay, two sequences of 1000."""
    x = gen.make_prefill(36, [1000, 1000], H=4, dk=128, dv=128, dtype=dtype, mu=0.0,
                         state_std=0.02, fixed_even_log_alpha=-3.5)
    check_prefill(x, label="strong decay, equal rows")
