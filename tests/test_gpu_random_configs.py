"""Prefill parity on seeded random configurations (needs an MI355X).

Each case draws, from its own fixed seed, a batch shape across the axes the
kernels branch on: the number of sequences and their lengths (empty,
one-token, chunk-edge and ragged lengths, packed or equal rows), the head
count (including counts that are not a multiple of 8, which take another
grid mapping), the key and value sizes, the dtype and the presence of
initial states.  Every case is gated against the oracle at every
granularity (whole tensors, each (sequence, head), each chunk, each row).
"""
import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import check_prefill

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = [0, 1, 63, 64, 65, 127, 128, 129]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_case(seed: int):
    g = np.random.default_rng([20, seed])
    dtype = ["f32", "bf16"][int(g.integers(2))]
    dk, dv = [(64, 64), (128, 128), (64, 128), (128, 64)][int(g.integers(4))]
    H = int(g.choice([1, 2, 3, 5, 8, 12]))
    N = int(g.integers(1, 25))
    packed = bool(g.integers(2)) and N > 1
    if packed:
        lens = [int(x) for x in g.integers(0, 400, N)]
        for i in range(min(3, N)):   # a few edge lengths in random places
            lens[int(g.integers(N))] = int(g.choice(EDGE_LENGTHS))
    else:
        lens = [int(g.choice([64, 100, 130, 257]))] * N
    state_std = 0.02 if g.integers(2) else 0.0
    mu = float(g.choice([0.0, 3.0, 4.0]))
    return dict(dtype=dtype, dk=dk, dv=dv, H=H, lens=lens, packed=packed, state_std=state_std,
                mu=mu)


@pytest.mark.parametrize("seed", range(12))
def test_random_configuration(seed):
    c = draw_case(seed)
    x = gen.make_prefill(400 + seed, c["lens"], H=c["H"], dk=c["dk"], dv=c["dv"], dtype=c["dtype"],
                         mu=c["mu"], state_std=c["state_std"], packed=c["packed"])
    check_prefill(x, label=f"random case {seed} ({'packed' if c['packed'] else 'equal rows'}, "
                           f"N={len(c['lens'])}, mu={c['mu']}, S0 std={c['state_std']})")


def test_two_slice_kernel_odd_head_count():
    """bf16 at d = 128 with more chains than CUs (12 sequences x 3 heads x 8
    value slices), so the two-slice sequential kernel runs them in rounds,
    longest first, with a head count that is not a multiple of 8; ragged
    lengths with an empty and a one-token sequence, nonzero initial states."""
    g = np.random.default_rng(21)
    lens = [int(x) for x in g.integers(0, 900, 12)]
    lens[2], lens[9] = 0, 1
    x = gen.make_prefill(421, lens, H=3, dk=128, dv=128, dtype="bf16", state_std=0.02,
                         packed=True)
    check_prefill(x, label="two-slice kernel, H = 3")


def draw_pool_case(seed: int):
    g = np.random.default_rng([21, seed])
    dtype = ["f32", "bf16"][int(g.integers(2))]
    dk, dv = [(64, 64), (128, 128), (64, 128), (128, 64)][int(g.integers(4))]
    H = int(g.choice([1, 2, 3, 8]))
    N = int(g.integers(1, 20))
    one_token = bool(g.integers(2))
    lens = [1] * N if one_token else [int(x) for x in g.integers(0, 41, N)]
    P = int(g.integers(N, 3 * N + 2))   # dense enough for the slot walk, or not
    slots = [int(x) for x in g.permutation(P)[:N]]
    for _ in range(int(g.integers(0, 3))):   # padding: -1 or past the pool
        slots[int(g.integers(N))] = int(g.choice([-1, P, P + 5]))
    flags = bool(g.integers(2))
    return dict(dtype=dtype, dk=dk, dv=dv, H=H, lens=lens, P=P, slots=slots, flags=flags,
                one_token=one_token)


@pytest.mark.parametrize("seed", range(10))
def test_random_pooled_tokens(seed):
    """kda_decode_tokens on seeded random pools against the oracle: the pool
    after the call (slots no sequence names unchanged, bit for bit) and every
    output row (padding sequences' rows zero)."""
    import torch
    import oracle
    import gated_delta_rule_prefill_amd as kda
    from gpu_util import TOL, dev_f32, device_inputs, host, rel_l2
    c = draw_pool_case(seed)
    N = len(c["lens"])
    x = gen.make_prefill(500 + seed, c["lens"], H=c["H"], dk=c["dk"], dv=c["dv"], dtype=c["dtype"],
                         raw=c["flags"], packed=not c["one_token"] and len(set(c["lens"])) > 1)
    pool = (0.02 * np.random.default_rng([22, seed]).standard_normal(
        (c["P"], c["H"], c["dk"], c["dv"]))).astype(np.float32)
    d = device_inputs(x)
    p = dev_f32(pool)
    sl = torch.tensor(c["slots"], dtype=torch.int32, device="cuda")
    o = kda.decode_tokens(p, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state_indices=sl,
                          cu_seqlens=d["cu_seqlens"], num_seqs=N, l2norm_qk=c["flags"],
                          beta_sigmoid=c["flags"])
    torch.cuda.synchronize()
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, np.asarray(c["slots"], np.int32), x.q, x.k, x.v,
                              x.log_alpha, x.beta, x.cu_seqlens, num_seqs=N,
                              l2norm_qk=c["flags"], beta_logit=c["flags"])
    go, gp = host(o), host(p)
    eo = rel_l2(go, ro) if ro.size else 0.0
    ep = rel_l2(gp, ref_pool)
    print(f"[pooled] random case {seed}: {c['dtype']} {c['dk']}x{c['dv']} H={c['H']} N={N} "
          f"P={c['P']} one_token={c['one_token']} flags={c['flags']}: o={eo:.3e} pool={ep:.3e}",
          flush=True)
    assert eo <= TOL[c["dtype"]] and ep <= TOL[c["dtype"]]
    starts = np.concatenate([[0], np.cumsum(c["lens"])])
    for s, sl_ in enumerate(c["slots"]):
        if not 0 <= sl_ < c["P"]:
            assert not np.any(go[starts[s]:starts[s + 1]]), (seed, s)
    used = {sl_ for sl_ in c["slots"] if 0 <= sl_ < c["P"]}
    for untouched in set(range(c["P"])) - used:
        assert np.array_equal(gp[untouched], pool[untouched].astype(np.float64)), (seed, untouched)
