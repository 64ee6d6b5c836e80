"""Batches with many sequences (needs an MI355X).

Branches that only large sequence counts reach:
  * prefill with more than 1,024 sequences: the chunk table's prefix over the
    sequence counts runs in several passes of its block, and the
    longest-first order of the two-slice sequential kernel falls back to index
    order (it is ranked in LDS for at most 1,024 sequences);
  * pooled tokens with more than 4,096 sequences: the recurrent kernels and
    the one-token decode kernel walk the sequences instead of the pool's
    slots (one pass over the slot array per workgroup is only kept short up to
    that count).
Each is compared with the oracle per (sequence, head) or per slot, not only
over the whole tensors.
"""
import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, check_prefill, dev_f32, device_inputs, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _lengths(seed: int, n: int, hi: int):
    g = np.random.default_rng([30, seed])
    lens = [int(x) for x in g.integers(0, hi, n)]
    for i, e in enumerate([0, 1, 63, 64, 65, 200]):   # edge lengths among them
        lens[(i * 331 + 7) % n] = e
    return lens


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64)])
def test_prefill_more_sequences_than_the_ranked_order(dtype, dk, dv):
    """1,500 packed sequences of 0..60 tokens (and a few edge lengths), H = 2,
    nonzero initial states: bf16 at d = 128 runs the two-slice kernel over
    6,000 chains in index order."""
    lens = _lengths(1, 1500, 61)
    x = gen.make_prefill(601, lens, H=2, dk=dk, dv=dv, dtype=dtype, state_std=0.02, packed=True)
    check_prefill(x, label=f"{len(lens)} sequences")


def _pooled(seed, lens, P, slots, dtype, packed):
    import torch
    import oracle
    import gated_delta_rule_prefill_amd as kda
    N, H, D = len(lens), 1, 128
    x = gen.make_prefill(seed, lens, H=H, dk=D, dv=D, dtype=dtype, packed=packed)
    pool = (0.02 * np.random.default_rng([31, seed]).standard_normal((P, H, D, D))).astype(np.float32)
    d = device_inputs(x)
    p = dev_f32(pool)
    sl = torch.from_numpy(np.asarray(slots, np.int32)).cuda()
    o = kda.decode_tokens(p, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state_indices=sl,
                          cu_seqlens=d["cu_seqlens"], num_seqs=N)
    torch.cuda.synchronize()
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, np.asarray(slots, np.int32), x.q, x.k, x.v, x.log_alpha,
                              x.beta, x.cu_seqlens, num_seqs=N)
    go, gp = host(o), host(p)
    # every slot's state on its own, and every sequence's o rows
    per_slot = [rel_l2(gp[s], ref_pool[s]) for s in range(P)]
    starts = np.concatenate([[0], np.cumsum(lens)])
    per_seq = [rel_l2(go[starts[i]:starts[i + 1]], ro[starts[i]:starts[i + 1]])
               for i in range(N) if lens[i] > 0 and 0 <= slots[i] < P]
    eo, ep = rel_l2(go, ro), rel_l2(gp, ref_pool)
    print(f"[many sequences] pooled {dtype} N={N} P={P} T={x.T}: o={eo:.3e} pool={ep:.3e} "
          f"worst slot={max(per_slot):.3e} worst sequence o={max(per_seq):.3e}", flush=True)
    assert eo <= TOL[dtype] and ep <= TOL[dtype]
    assert max(per_slot) <= TOL[dtype] and max(per_seq) <= TOL[dtype]
    for i in range(N):   # padding sequences leave zero rows
        if not 0 <= slots[i] < P:
            assert not np.any(go[starts[i]:starts[i + 1]]), i
    used = {s for s in slots if 0 <= s < P}
    for s in range(P):
        if s not in used:
            assert np.array_equal(gp[s], pool[s].astype(np.float64)), s


@pytest.mark.parametrize("case", ["eight_tokens", "one_token"])
def test_pooled_tokens_more_sequences_than_the_slot_walk(case):
    """5,000 sequences on a pool of 5,200 slots in permuted order with a few
    padding entries, H = 1, d = 128, bf16: 8 tokens each (the chunkwise MFMA
    form) or one each (the decode kernel with slot indirection), both walking
    the sequences."""
    N, P = 5000, 5200
    g = np.random.default_rng(32)
    slots = [int(s) for s in g.permutation(P)[:N]]
    for i in (3, 777, 4999):
        slots[i] = [-1, P, P + 11][i % 3]
    lens = [8 if case == "eight_tokens" else 1] * N
    _pooled(602 if case == "eight_tokens" else 603, lens, P, slots, "bf16", packed=False)


def test_pooled_tokens_packed_many_sequences():
    """5,000 packed sequences of 0..12 tokens on a pool of 5,100 slots (token
    steps with a per-sequence range from cu_seqlens), fp32."""
    N, P = 5000, 5100
    g = np.random.default_rng(33)
    lens = [int(x) for x in g.integers(0, 13, N)]
    slots = [int(s) for s in g.permutation(P)[:N]]
    slots[10] = -1
    _pooled(604, lens, P, slots, "f32", packed=True)
