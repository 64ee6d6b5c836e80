"""Property tests of the oracle over random small shapes (hypothesis; no GPU).

The fixed pins in pins.py check the oracle against independent references
on chosen cases; these draw the shapes, lengths, dtypes, decay strengths and
seeds at random and check the same independent facts on each draw:
  * every head equals the dense product of its transition matrices (numpy);
  * the chunkwise form (tests/chunkwise_mirror.py, written from the chunk
    algebra, not from the oracle) reproduces it for a random chunk size;
  * a packed batch equals separate calls per sequence, bit for bit;
  * token-by-token decode steps reproduce the prefill;
  * pooled tokens are decode steps on each sequence's slot (padding and
    unnamed slots untouched).
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import chunkwise_mirror
import oracle
from pins import _case, _f64, rel_err, transition_reference

SETTINGS = dict(max_examples=25, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow])

dims = st.integers(min_value=1, max_value=9)
dtypes = st.sampled_from(["f32", "bf16"])
mus = st.sampled_from([-1.0, 0.0, 1.0, 3.0])
seeds = st.integers(min_value=0, max_value=10_000)


@settings(**SETTINGS)
@given(seed=seeds, T=st.integers(min_value=1, max_value=14), H=st.integers(1, 3), dk=dims,
       dv=dims, dtype=dtypes, mu=mus)
def test_prefill_is_the_transition_product(seed, T, H, dk, dv, dtype, mu):
    x = _case(seed, T, H, dk, dv, dtype=dtype, mu=mu)
    o, fin = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    for h in range(H):
        ro, rS = transition_reference(_f64(x.q[:, h]), _f64(x.k[:, h]), _f64(x.v[:, h]),
                                      x.log_alpha[:, h].astype(np.float64),
                                      x.beta[:, h].astype(np.float64),
                                      x.initial_state[0, h].astype(np.float64))
        assert rel_err(o[:, h], ro) < 1e-11
        assert rel_err(fin[0, h], rS) < 1e-11


@settings(**SETTINGS)
@given(seed=seeds, lengths=st.lists(st.integers(0, 90), min_size=1, max_size=4), dk=dims, dv=dims,
       C=st.integers(1, 40), mu=st.sampled_from([0.0, 2.0, 4.0]))
def test_chunkwise_form_matches_for_any_chunk_size(seed, lengths, dk, dv, C, mu):
    x = _case(seed, 0, 2, dk, dv, mu=mu, lengths=lengths)
    o, fin = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens,
                            num_seqs=x.num_seqs)
    mo, mS = chunkwise_mirror.prefill(x, C)
    if o.size:
        assert rel_err(mo, o) < 1e-10
    assert rel_err(mS, fin) < 1e-10


@settings(**SETTINGS)
@given(seed=seeds, lengths=st.lists(st.integers(0, 20), min_size=2, max_size=5), dk=dims,
       dv=dims, dtype=dtypes)
def test_packed_batch_is_separate_calls(seed, lengths, dk, dv, dtype):
    x = _case(seed, 0, 2, dk, dv, dtype=dtype, lengths=lengths)
    o, fin = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    for s in range(x.num_seqs):
        y = x.select_seqs([s])
        os_, fs = oracle.prefill(y.q, y.k, y.v, y.log_alpha, y.beta, y.initial_state)
        a, b = x.cu_seqlens[s], x.cu_seqlens[s + 1]
        assert np.array_equal(o[a:b], os_)
        assert np.array_equal(fin[s], fs[0])


@settings(**SETTINGS)
@given(seed=seeds, T=st.integers(1, 12), H=st.integers(1, 3), dk=dims, dv=dims, dtype=dtypes)
def test_decode_steps_reproduce_prefill(seed, T, H, dk, dv, dtype):
    x = _case(seed, T, H, dk, dv, dtype=dtype)
    o, fin = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    S = x.initial_state.astype(np.float64).copy()
    for t in range(T):
        ot = oracle.decode_step(S, x.q[t][None], x.k[t][None], x.v[t][None],
                                x.log_alpha[t][None], x.beta[t][None])
        assert rel_err(ot[0], o[t]) < 1e-12
    assert rel_err(S, fin) < 1e-12


@settings(**SETTINGS)
@given(seed=seeds, lengths=st.lists(st.integers(0, 8), min_size=1, max_size=6), dk=dims, dv=dims,
       extra_slots=st.integers(0, 6), n_pad=st.integers(0, 2))
def test_pooled_tokens_are_decode_steps_on_the_slots(seed, lengths, dk, dv, extra_slots, n_pad):
    """Each sequence starts from its slot's state and leaves its final state
    there; padding sequences (a slot outside the pool) give zero output and
    touch nothing; slots no sequence names are unchanged."""
    x = _case(seed, 0, 2, dk, dv, lengths=lengths)
    N = x.num_seqs
    g = np.random.default_rng(seed)
    P = N + extra_slots
    slots = g.permutation(P)[:N].astype(np.int32)
    for i in g.choice(N, size=min(n_pad, N), replace=False):
        slots[i] = g.choice([-1, P, P + 3])
    pool = 0.3 * g.standard_normal((P, x.H, dk, dv))
    got = pool.copy()
    o = oracle.decode_tokens(got, slots, x.q, x.k, x.v, x.log_alpha, x.beta, x.cu_seqlens,
                             num_seqs=N)
    ref = pool.copy()
    cu = x.cu_seqlens if x.cu_seqlens is not None else np.arange(N + 1) * (x.T // N)
    for s in range(N):
        a, b = int(cu[s]), int(cu[s + 1])
        if not 0 <= slots[s] < P:
            assert not np.any(o[a:b])
            continue
        S = ref[slots[s]][None].copy()
        for t in range(a, b):
            ot = oracle.decode_step(S, x.q[t][None], x.k[t][None], x.v[t][None],
                                    x.log_alpha[t][None], x.beta[t][None])
            assert rel_err(ot[0], o[t]) < 1e-12
        ref[slots[s]] = S[0]
    assert rel_err(got, ref) < 1e-12
    unused = sorted(set(range(P)) - {int(v) for v in slots if 0 <= v < P})
    assert np.array_equal(got[unused], pool[unused])
