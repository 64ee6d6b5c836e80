"""GPU parity of the optional paths against the fp64 oracle: chunk-state
export and resume, in-kernel q/k L2 normalisation and beta sigmoid, and the
pooled multi-token recurrent path (needs an MI355X)."""
import dataclasses

import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, dev_f32, device_inputs, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_prefill_amd.kda as k
    k.lib()


def _prefill(x, **kw):
    import torch
    import gated_delta_rule_prefill_amd as kda
    d = device_inputs(x)
    res = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                      d["cu_seqlens"], num_seqs=d["num_seqs"], **kw)
    torch.cuda.synchronize()
    return res


# -- chunk-state export ---------------------------------------------------------
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 64),
                                         ("bf16", 64, 128)])
def test_chunk_states_match_oracle(dtype, dk, dv):
    """Every chunk-start state against the oracle's state after 64c tokens
    (packed batch with an empty sequence and partial last chunks)."""
    x = gen.make_prefill(61, [130, 0, 64, 1, 200], H=3, dk=dk, dv=dv, dtype=dtype,
                         state_std=0.02, packed=True)
    o, fin, cs = _prefill(x, chunk_states=True)
    ro, rf, rs = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state,
                                x.cu_seqlens, states_every=64)
    assert tuple(cs.shape) == rs.shape, (tuple(cs.shape), rs.shape)
    errs = [rel_l2(host(o), ro), rel_l2(host(fin), rf), rel_l2(host(cs), rs)]
    print(f"[chunk states] {dtype} {dk}x{dv}: o={errs[0]:.3e} final={errs[1]:.3e} "
          f"chunk states={errs[2]:.3e}", flush=True)
    assert max(errs) <= TOL[dtype]
    # row 0 of each sequence is its initial state, exactly
    lens = x.lengths()
    row = 0
    for s, n in enumerate(lens):
        if n:
            assert np.array_equal(host(cs[row]), x.initial_state[s].astype(np.float64))
        row += (n + 63) // 64


def test_chunk_states_equal_rows_and_outputs_unchanged():
    """Asking for chunk states changes no other output (bit for bit)."""
    import torch
    x = gen.make_prefill(62, [256, 256], H=4, dk=128, dv=128, dtype="bf16", state_std=0.02)
    o1, f1 = _prefill(x)
    o2, f2, cs = _prefill(x, chunk_states=True)
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(f1.cpu(), f2.cpu())
    assert cs.shape[0] == 8
    _, _, rs = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state,
                              num_seqs=2, states_every=64)
    assert rel_l2(host(cs), rs) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_resume_from_chunk_state(dtype):
    """Prefill again from the exported state at token 64c: the tail's outputs
    and the final state match the single call."""
    x = gen.make_prefill(63, [300], H=2, dk=128, dv=128, dtype=dtype, state_std=0.02)
    o, fin, cs = _prefill(x, chunk_states=True)
    for c in (1, 3):
        a = 64 * c
        tail = dataclasses.replace(x, q=x.q[a:].copy(), k=x.k[a:].copy(), v=x.v[a:].copy(),
                                   log_alpha=x.log_alpha[a:].copy(), beta=x.beta[a:].copy(),
                                   initial_state=host(cs[c:c + 1]).astype(np.float32))
        o2, f2 = _prefill(tail)
        eo, ef = rel_l2(host(o2), host(o)[a:]), rel_l2(host(f2), host(fin))
        print(f"[resume] {dtype} c={c}: o={eo:.3e} final={ef:.3e}", flush=True)
        assert eo <= TOL[dtype] and ef <= TOL[dtype]


# -- in-kernel preprocessing ----------------------------------------------------
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64), ("f32", 128, 64),
                                         ("bf16", 64, 128)])
def test_prefill_preprocessing(dtype, dk, dv):
    """Raw q/k (arbitrary row norms) and beta logits with both flags against
    the oracle applying the same preprocessing in fp64."""
    x = gen.make_prefill(64, [150, 77], H=3, dk=dk, dv=dv, dtype=dtype, state_std=0.02,
                         packed=True, raw=True)
    o, fin = _prefill(x, l2norm_qk=True, beta_sigmoid=True)
    ro, rf = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens,
                            l2norm_qk=True, beta_logit=True)
    eo, ef = rel_l2(host(o), ro), rel_l2(host(fin), rf)
    print(f"[preprocess] {dtype} {dk}x{dv}: o={eo:.3e} final={ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


def test_prefill_normalisation_is_scale_invariant():
    """With L2 normalisation, power-of-two rescaling of q and k rows changes
    nothing (fp32 inputs: the scaled values are exact)."""
    x = gen.make_prefill(65, [200], H=2, dk=128, dv=128, dtype="f32", state_std=0.02, raw=True)
    g = np.random.default_rng(65)
    y = dataclasses.replace(
        x, q=(x.q * np.exp2(g.integers(-3, 4, (x.T, x.H, 1)))).astype(np.float32),
        k=(x.k * np.exp2(g.integers(-3, 4, (x.T, x.H, 1)))).astype(np.float32))
    o1, f1 = _prefill(x, l2norm_qk=True, beta_sigmoid=True)
    o2, f2 = _prefill(y, l2norm_qk=True, beta_sigmoid=True)
    assert rel_l2(host(o2), host(o1)) <= 1e-5 and rel_l2(host(f2), host(f1)) <= 1e-5


# -- pooled multi-token recurrent path -------------------------------------------
def _pool_case(seed, lens, dtype, dk=128, dv=128, H=4, P=7, raw=False, packed=True):
    x = gen.make_prefill(seed, lens, H=H, dk=dk, dv=dv, dtype=dtype, packed=packed, raw=raw)
    g = np.random.default_rng(seed)
    pool = (0.02 * g.standard_normal((P, H, dk, dv))).astype(np.float32)
    return x, pool


def _decode_tokens(x, pool, slots, **kw):
    import torch
    import gated_delta_rule_prefill_amd as kda
    d = device_inputs(x)
    p = dev_f32(pool)
    sl = None if slots is None else torch.from_numpy(np.asarray(slots, np.int32)).cuda()
    o = kda.decode_tokens(p, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state_indices=sl,
                          cu_seqlens=d["cu_seqlens"], num_seqs=d["num_seqs"], **kw)
    torch.cuda.synchronize()
    return o, p


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 64),
                                         ("bf16", 128, 64), ("bf16", 64, 128)])
@pytest.mark.parametrize("flags", [False, True])
def test_decode_tokens_match_oracle(dtype, dk, dv, flags):
    """Lengths 0..70 (several 16-token stages), permuted slots, two padding
    sequences (slot -1 and slot past the pool)."""
    lens = [5, 1, 0, 16, 17, 70, 3]
    slots = [4, -1, 0, 6, 2, 1, 9]
    x, pool = _pool_case(66, lens, dtype, dk, dv, raw=flags)
    kw = dict(l2norm_qk=flags, beta_sigmoid=flags)
    o, p = _decode_tokens(x, pool, slots, **kw)
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, np.asarray(slots, np.int32), x.q, x.k, x.v, x.log_alpha,
                              x.beta, x.cu_seqlens, l2norm_qk=flags, beta_logit=flags)
    eo, ep = rel_l2(host(o), ro), rel_l2(host(p), ref_pool)
    print(f"[decode tokens] {dtype} {dk}x{dv} flags={flags}: o={eo:.3e} pool={ep:.3e}", flush=True)
    assert eo <= TOL[dtype] and ep <= TOL[dtype]
    cu = x.cu_seqlens
    assert not np.any(host(o)[cu[1]:cu[2]]) and not np.any(host(o)[cu[6]:cu[7]])
    for untouched in (3, 5):   # slots no sequence names
        assert np.array_equal(host(p)[untouched], pool[untouched].astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lens", [[5, 1, 0, 16, 17, 70, 3], [1] * 7])
def test_decode_tokens_sparse_pool(dtype, lens):
    """A pool of 40 slots for 7 sequences: the kernels walk the sequences (the
    slot-order walk is for pools at most twice the batch), with permuted and
    padding slots, several tokens per sequence and one."""
    slots = [31, -1, 0, 12, 39, 7, 40]
    x, pool = _pool_case(72, lens, dtype, P=40, packed=len(set(lens)) > 1)
    o, p = _decode_tokens(x, pool, slots)
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, np.asarray(slots, np.int32), x.q, x.k, x.v, x.log_alpha,
                              x.beta, x.cu_seqlens, num_seqs=len(lens))
    go, gp = host(o), host(p)
    eo, ep = rel_l2(go, ro), rel_l2(gp, ref_pool)
    print(f"[decode tokens] sparse pool {dtype} lens={lens}: o={eo:.3e} pool={ep:.3e}", flush=True)
    assert eo <= TOL[dtype] and ep <= TOL[dtype]
    starts = np.concatenate([[0], np.cumsum(lens)])
    for pad in (1, 6):
        assert not np.any(go[starts[pad]:starts[pad + 1]])
    used = {sl for sl in slots if 0 <= sl < 40}
    for untouched in set(range(40)) - used:
        assert np.array_equal(gp[untouched], pool[untouched].astype(np.float64))


@pytest.mark.parametrize("R", [8, 1])
def test_decode_tokens_benchmark_shape(R):
    """The benchmark's pooled workloads in their launch configurations: 256
    sequences of 8 tokens (the chunkwise form) or of one token (the decode
    step through the slots) as equal rows, H = 32, d = 128, bf16, fp32 states
    in a permuted order of the pool's slots.  Gated per sequence (its output
    rows over all heads) and per (slot, head) state, besides the whole
    tensors."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    H, D, N = 32, 128, 256
    x = gen.make_prefill(9, [R] * N, H=H, dk=D, dv=D, dtype="bf16")
    pool = gen.decode_state(9, N, H, D, D)
    slots = np.random.default_rng(9).permutation(N).astype(np.int32)
    d = device_inputs(x)
    p = dev_f32(pool)
    o = kda.decode_tokens(p, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                          state_indices=torch.from_numpy(slots).cuda(), num_seqs=N)
    torch.cuda.synchronize()
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, slots, x.q, x.k, x.v, x.log_alpha, x.beta, num_seqs=N)
    go, gp = host(o), host(p)
    eo, ep = rel_l2(go, ro), rel_l2(gp, ref_pool)
    worst_o = max(rel_l2(go[R * s:R * s + R], ro[R * s:R * s + R]) for s in range(N))
    worst_p = max(rel_l2(gp[sl, h], ref_pool[sl, h]) for sl in range(N) for h in range(H))
    print(f"[decode tokens] benchmark shape, {R} token(s): o={eo:.3e} (worst sequence {worst_o:.3e}) "
          f"pool={ep:.3e} (worst state {worst_p:.3e})", flush=True)
    assert eo <= TOL["bf16"] and ep <= TOL["bf16"]
    assert worst_o <= TOL["bf16"] and worst_p <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_tokens_equal_prefill(dtype):
    """The recurrent path and the chunkwise prefill compute the same function
    (equal rows, identity slots)."""
    x = gen.make_prefill(67, [40, 40, 40], H=3, dk=128, dv=128, dtype=dtype, state_std=0.02)
    o_p, f_p = _prefill(x)
    o_r, pool = _decode_tokens(x, x.initial_state, None)
    assert rel_l2(host(o_r), host(o_p)) <= TOL[dtype]
    assert rel_l2(host(pool), host(f_p)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 64),
                                         ("bf16", 128, 64), ("bf16", 64, 128)])
@pytest.mark.parametrize("flags", [False, True])
def test_decode_tokens_one_token_per_sequence(dtype, dk, dv, flags):
    """One token per sequence as equal rows (the serving step on a pool):
    permuted slots, a slot of -1 and one past the pool pad; without options
    this takes the decode step's kernel with slot indirection, with them the
    token loop."""
    N, P, H = 9, 12, 3
    slots = [7, 0, -1, 11, 3, 12, 5, 1, 9]
    x, pool = _pool_case(71, [1] * N, dtype, dk, dv, H=H, P=P, raw=flags, packed=False)
    assert x.cu_seqlens is None
    kw = dict(l2norm_qk=flags, beta_sigmoid=flags)
    o, p = _decode_tokens(x, pool, slots, **kw)
    ref_pool = pool.astype(np.float64)
    ro = oracle.decode_tokens(ref_pool, np.asarray(slots, np.int32), x.q, x.k, x.v, x.log_alpha,
                              x.beta, num_seqs=N, l2norm_qk=flags, beta_logit=flags)
    go, gp = host(o), host(p)
    eo, ep = rel_l2(go, ro), rel_l2(gp, ref_pool)
    worst_o = max(rel_l2(go[s], ro[s]) for s in range(N) if 0 <= slots[s] < P)
    print(f"[decode tokens] one token {dtype} {dk}x{dv} flags={flags}: o={eo:.3e} "
          f"(worst sequence {worst_o:.3e}) pool={ep:.3e}", flush=True)
    assert eo <= TOL[dtype] and ep <= TOL[dtype] and worst_o <= TOL[dtype]
    assert not np.any(go[2]) and not np.any(go[5])
    for untouched in (2, 4, 6, 8, 10):   # slots no sequence names
        assert np.array_equal(gp[untouched], pool[untouched].astype(np.float64))


def test_decode_tokens_one_token_equals_decode_step():
    """One token per sequence with identity slots and no options is
    kda_decode_step, bit for bit (the same kernel)."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    t = gen.decode_token(68, 0, 16, 4, 128, 128, dtype="bf16")
    d = device_inputs(t)
    S0 = gen.decode_state(68, 16, 4, 128, 128)
    s1, s2 = dev_f32(S0), dev_f32(S0)
    o1 = kda.decode_step(s1, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    o2 = kda.decode_tokens(s2, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], num_seqs=16)
    torch.cuda.synchronize()
    assert np.array_equal(host(o2), host(o1)) and np.array_equal(host(s2), host(s1))
