"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` takes an oracle handle (an object with ``prefill`` and
``decode_step``) and raises AssertionError when the handle disagrees with an
independent statement of what KDA computes.  The references here are written
from the pages and from mathematics, not from the oracle's code:

* the explicit product of dense transition matrices (Kimi Linear paper notes,
  section 2: the state update is a dk x dk transition applied to S plus a
  rank-1 write, so S_T is a sum of transition products);
* exact rational arithmetic on the matrix form of the recurrence;
* the reductions the pages name: alpha = 1 gives DeltaNet's error-correcting
  delta rule, a scalar alpha per head gives Gated DeltaNet (hnts03 KDA
  summary, "Kimi Delta Attention"; paper notes, section 2);
* closed forms: pure decay, one-hot keys (causal linear attention), beta = 1
  with unit keys (exact recall);
* the chunkwise algebra of ``chunkwise_mirror`` (paper notes, section 3).

Every pin is also run against deliberately broken copies of the oracle
(``test_oracle_mutants.py``) to show that it can fail.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction

import numpy as np

import chunkwise_mirror
from gated_delta_rule_prefill_amd import inputs as gen


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def _case(seed, T, H, dk, dv, dtype="f32", mu=1.0, state_std=0.3, lengths=None, raw=False):
    lengths = lengths or [T]
    return gen.make_prefill(seed, lengths, H=H, dk=dk, dv=dv, dtype=dtype, mu=mu,
                            state_std=state_std, packed=len(lengths) > 1 or None, raw=raw)


def _f64(x):
    return gen.as_f32(x).astype(np.float64)


# --------------------------------------------------------------------------
# reference 1: dense transition matrices (numpy fp64)
# --------------------------------------------------------------------------
def transition_reference(q, k, v, la, beta, S0):
    """One head.  M_t = (I - beta_t k_t k_t^T) Diag(exp la_t);
    S_t = (M_t ... M_0) S0 + sum_i (M_t ... M_{i+1}) beta_i k_i v_i^T; o_t = S_t^T q_t."""
    T, dk = k.shape
    M = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(la[t])) for t in range(T)]
    o = np.zeros((T, v.shape[1]))
    S_last = S0
    for t in range(T):
        Phi = np.eye(dk)                      # Phi_{t,t}
        S = beta[t] * np.outer(k[t], v[t])
        for i in range(t - 1, -1, -1):
            Phi = Phi @ M[i + 1]              # Phi_{t,i} = M_t ... M_{i+1}
            S = S + Phi @ (beta[i] * np.outer(k[i], v[i]))
        Phi = Phi @ M[0]                      # Phi_{t,-1} = M_t ... M_0
        S = S + Phi @ S0
        o[t] = S.T @ q[t]
        S_last = S
    return o, S_last


def pin_transition_product(orc):
    for seed, (T, H, dk, dv, dtype) in enumerate([(9, 2, 4, 3, "f32"), (12, 1, 6, 6, "f32"),
                                                  (7, 3, 5, 8, "bf16"), (1, 1, 3, 2, "f32")]):
        x = _case(100 + seed, T, H, dk, dv, dtype=dtype)
        o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
        for h in range(H):
            ro, rS = transition_reference(_f64(x.q[:, h]), _f64(x.k[:, h]), _f64(x.v[:, h]),
                                          x.log_alpha[:, h].astype(np.float64),
                                          x.beta[:, h].astype(np.float64),
                                          x.initial_state[0, h].astype(np.float64))
            assert rel_err(o[:, h], ro) < 1e-12, ("transition o", seed, h, rel_err(o[:, h], ro))
            assert rel_err(fin[0, h], rS) < 1e-12, ("transition S", seed, h)


# --------------------------------------------------------------------------
# reference 2: exact rationals, matrix form of the recurrence
# --------------------------------------------------------------------------
def _fr(x):
    return Fraction(float(x))


def exact_reference(q, k, v, alpha, beta, S0):
    dk, dv = len(k[0]), len(v[0])
    S = [[_fr(S0[c][j]) for j in range(dv)] for c in range(dk)]
    outs = []
    for t in range(len(q)):
        kt = [_fr(x) for x in k[t]]
        bt = _fr(beta[t])
        # M = (I - beta k k^T) Diag(alpha)
        M = [[((1 if r == c else 0) - bt * kt[r] * kt[c]) * alpha[t][c] for c in range(dk)]
             for r in range(dk)]
        S = [[sum(M[r][c] * S[c][j] for c in range(dk)) + bt * kt[r] * _fr(v[t][j])
              for j in range(dv)] for r in range(dk)]
        outs.append([sum(S[c][j] * _fr(q[t][c]) for c in range(dk)) for j in range(dv)])
    return outs, S


def pin_exact_rational(orc):
    x = _case(7, 5, 1, 3, 2, mu=0.5)
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    # alpha exactly as an IEEE double exp of the fp32 log-decay (C library exp)
    alpha = [[Fraction(math.exp(float(a))) for a in row] for row in x.log_alpha[:, 0]]
    outs, S = exact_reference(x.q[:, 0], x.k[:, 0], x.v[:, 0], alpha, x.beta[:, 0],
                              x.initial_state[0, 0])
    ref_o = np.array([[float(z) for z in row] for row in outs])
    ref_S = np.array([[float(z) for z in row] for row in S])
    assert rel_err(o[:, 0], ref_o) < 1e-14, rel_err(o[:, 0], ref_o)
    assert rel_err(fin[0, 0], ref_S) < 1e-14


# --------------------------------------------------------------------------
# reductions and closed forms
# --------------------------------------------------------------------------
def pin_identity_no_write(orc):
    """alpha = 1, beta = 0: nothing is written or forgotten; o_t = S0^T q_t."""
    x = _case(11, 20, 2, 8, 5)
    la = np.zeros_like(x.log_alpha)
    be = np.zeros_like(x.beta)
    o, fin = orc.prefill(x.q, x.k, x.v, la, be, x.initial_state)
    S0 = x.initial_state[0].astype(np.float64)
    assert np.array_equal(fin[0], S0)
    ref = np.einsum("hcj,thc->thj", S0, _f64(x.q))
    assert rel_err(o, ref) < 1e-14


def pin_pure_decay(orc):
    """beta = 0: S_t = Diag(exp(G_t)) S0 with G_t the running sum of log alpha."""
    x = _case(12, 30, 2, 6, 4, mu=1.0)
    be = np.zeros_like(x.beta)
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, be, x.initial_state)
    G = np.cumsum(x.log_alpha.astype(np.float64), axis=0)       # [T,H,dk]
    S0 = x.initial_state[0].astype(np.float64)                   # [H,dk,dv]
    ref_o = np.einsum("hcj,thc->thj", S0, np.exp(G) * _f64(x.q))
    ref_S = np.exp(G[-1])[:, :, None] * S0
    assert rel_err(o, ref_o) < 1e-12
    assert rel_err(fin[0], ref_S) < 1e-12


def pin_deltanet(orc):
    """alpha = 1 reduces to DeltaNet: S <- S + beta k (v - S^T k)^T (error-correcting write)."""
    x = _case(13, 25, 2, 7, 5)
    la = np.zeros_like(x.log_alpha)
    o, fin = orc.prefill(x.q, x.k, x.v, la, x.beta, x.initial_state)
    q, k, v = _f64(x.q), _f64(x.k), _f64(x.v)
    for h in range(x.H):
        S = x.initial_state[0, h].astype(np.float64)
        for t in range(x.T):
            err = v[t, h] - S.T @ k[t, h]             # prediction error of the memory
            S = S + float(x.beta[t, h]) * np.outer(k[t, h], err)
            assert rel_err(o[t, h], S.T @ q[t, h]) < 1e-12
        assert rel_err(fin[0, h], S) < 1e-12


def pin_gated_deltanet(orc):
    """One scalar decay a_t per head reduces to Gated DeltaNet:
    S <- a_t (I - beta k k^T) S + beta k v^T."""
    x = _case(14, 25, 2, 6, 6, mu=1.5)
    la = np.repeat(x.log_alpha[:, :, :1], x.dk, axis=2)       # same rate on every channel
    o, fin = orc.prefill(x.q, x.k, x.v, la, x.beta, x.initial_state)
    q, k, v = _f64(x.q), _f64(x.k), _f64(x.v)
    for h in range(x.H):
        S = x.initial_state[0, h].astype(np.float64)
        for t in range(x.T):
            a = math.exp(float(la[t, h, 0]))
            b = float(x.beta[t, h])
            S = a * (np.eye(x.dk) - b * np.outer(k[t, h], k[t, h])) @ S + b * np.outer(k[t, h], v[t, h])
        assert rel_err(fin[0, h], S) < 1e-12
    # the per-channel case must differ from the scalar case (the gating is per channel)
    o2, _ = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    assert rel_err(o2, o) > 1e-3


def pin_exact_recall(orc):
    """beta = 1 and unit k_t: the write makes S_t^T k_t = v_t exactly; with q_t = k_t, o_t = v_t.
    Keys are +-1/2 on four random channels, so |k| = 1 holds exactly in binary."""
    T, H, dk, dv = 40, 2, 16, 8
    x = _case(15, T, H, dk, dv, mu=2.0)
    g = np.random.default_rng(15)
    k = np.zeros((T, H, dk), np.float32)
    for t in range(T):
        for h in range(H):
            k[t, h, g.permutation(dk)[:4]] = g.choice([-0.5, 0.5], size=4)
    o, _ = orc.prefill(k, k, x.v, x.log_alpha, np.ones_like(x.beta), x.initial_state)
    assert rel_err(o, _f64(x.v)) < 1e-14


def pin_one_hot_linear_attention(orc):
    """One-hot keys k_i = e_{c_i}, distinct c_i, alpha = beta = 1, S0 = 0:
    causal linear attention as a lookup, o_t = sum_{i<=t} q_t[c_i] v_i."""
    T, dk, dv = 12, 16, 5
    g = np.random.default_rng(16)
    cs = g.permutation(dk)[:T]
    k = np.zeros((T, 1, dk), np.float32)
    k[np.arange(T), 0, cs] = 1.0
    q = g.standard_normal((T, 1, dk)).astype(np.float32)
    v = g.standard_normal((T, 1, dv)).astype(np.float32)
    o, _ = orc.prefill(q, k, v, np.zeros((T, 1, dk), np.float32), np.ones((T, 1), np.float32))
    ref = np.array([sum(q[t, 0, cs[i]] * v[i, 0].astype(np.float64) for i in range(t + 1))
                    for t in range(T)])
    assert rel_err(o[:, 0], ref) < 1e-14


def pin_one_hot_rows(orc):
    """One-hot keys with decay: only row c_t is corrected,
    S[c_t] <- (1 - beta) alpha_{c_t} S[c_t] + beta v_t; every other row only decays."""
    T, dk, dv = 15, 6, 4
    g = np.random.default_rng(17)
    cs = g.integers(0, dk, size=T)
    k = np.zeros((T, 1, dk), np.float32)
    k[np.arange(T), 0, cs] = 1.0
    x = _case(17, T, 1, dk, dv, mu=1.0)
    o, fin = orc.prefill(x.q, k, x.v, x.log_alpha, x.beta, x.initial_state)
    S = x.initial_state[0, 0].astype(np.float64)
    for t in range(T):
        a = np.exp(x.log_alpha[t, 0].astype(np.float64))
        b = float(x.beta[t, 0])
        S = a[:, None] * S
        S[cs[t]] = (1.0 - b) * S[cs[t]] + b * x.v[t, 0].astype(np.float64)
        assert rel_err(o[t, 0], S.T @ x.q[t, 0].astype(np.float64)) < 1e-13
    assert rel_err(fin[0, 0], S) < 1e-13


def pin_single_token(orc):
    """T = 1 written out: o = (D S0 + beta k (v - (D S0)^T k)^T)^T q with D = Diag(alpha)."""
    x = _case(18, 1, 1, 4, 3)
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    q, k, v = _f64(x.q)[0, 0], _f64(x.k)[0, 0], _f64(x.v)[0, 0]
    D = np.diag(np.exp(x.log_alpha[0, 0].astype(np.float64)))
    b = float(x.beta[0, 0])
    DS = D @ x.initial_state[0, 0].astype(np.float64)
    S1 = DS + b * np.outer(k, v - DS.T @ k)
    assert rel_err(fin[0, 0], S1) < 1e-14
    assert rel_err(o[0, 0], S1.T @ q) < 1e-14


def pin_chunkwise_algebra(orc):
    """The chunkwise form (cumulative log-decay, A_kk / A_qk, UT transform, state
    hand-off) reproduces the recurrence for every chunk size, including chunks
    cut short by the end of a sequence."""
    x = _case(19, 0, 2, 8, 6, mu=2.0, lengths=[150, 1, 64, 37])
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    for C in (1, 2, 3, 16, 64):
        mo, mS = chunkwise_mirror.prefill(x, C)
        assert rel_err(mo, o) < 1e-11, (C, rel_err(mo, o))
        assert rel_err(mS, fin) < 1e-11, C


def pin_chunk_transition_form(orc):
    """Folding W and U into each chunk's transition (S' = Diag(gamma_C) S + PM S
    + Hc) and read-out (O = QM S + OI) reproduces the recurrence."""
    x = _case(26, 0, 2, 8, 6, mu=2.0, lengths=[150, 64, 37])
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    for C in (1, 5, 16, 64):
        mo, mS = chunkwise_mirror.prefill(x, C, transition=True)
        assert rel_err(mo, o) < 1e-11, (C, rel_err(mo, o))
        assert rel_err(mS, fin) < 1e-11, C


def pin_packing(orc):
    """A packed batch equals separate calls per sequence; equal rows equal cu_seqlens."""
    x = _case(20, 0, 2, 5, 4, lengths=[7, 0, 13, 1])
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    for s in range(x.num_seqs):
        y = x.select_seqs([s])
        os_, fs = orc.prefill(y.q, y.k, y.v, y.log_alpha, y.beta, y.initial_state)
        a, b = x.cu_seqlens[s], x.cu_seqlens[s + 1]
        assert np.array_equal(o[a:b], os_)
        assert np.array_equal(fin[s], fs[0])
    # zero-length sequence: final state = initial state
    assert np.array_equal(fin[1], x.initial_state[1].astype(np.float64))
    z = _case(21, 0, 1, 3, 3, lengths=[6, 6, 6])
    o1, f1 = orc.prefill(z.q, z.k, z.v, z.log_alpha, z.beta, z.initial_state, z.cu_seqlens)
    o2, f2 = orc.prefill(z.q, z.k, z.v, z.log_alpha, z.beta, z.initial_state, None, num_seqs=3)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def pin_decode_matches_prefill(orc):
    """T decode steps give the same o and S as one prefill (one mode, two paths)."""
    x = _case(22, 9, 3, 5, 4, dtype="bf16")
    o, fin = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    S = x.initial_state.astype(np.float64).copy()
    for t in range(x.T):
        ot = orc.decode_step(S, x.q[t][None], x.k[t][None], x.v[t][None], x.log_alpha[t][None],
                             x.beta[t][None])
        assert rel_err(ot[0], o[t]) < 1e-13
    assert rel_err(S, fin) < 1e-13


def pin_linearity(orc):
    """For fixed q, k, alpha, beta, (o, S_T) is linear in (S0, V)."""
    x = _case(23, 16, 2, 6, 5)
    y = _case(24, 16, 2, 6, 5)
    a, b = 0.75, -1.25
    V = a * x.v + b * y.v
    S0 = (a * x.initial_state.astype(np.float64) + b * y.initial_state.astype(np.float64))
    # the combination is exactly representable in fp32 only approximately: compare in fp64
    o1, f1 = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state)
    o2, f2 = orc.prefill(x.q, x.k, y.v, x.log_alpha, x.beta, y.initial_state)
    o3, f3 = orc.prefill(x.q, x.k, V.astype(np.float32), x.log_alpha, x.beta,
                         S0.astype(np.float32))
    # fp32 rounding of the combined inputs bounds the residual
    assert rel_err(o3, a * o1 + b * o2) < 1e-6
    assert rel_err(f3, a * f1 + b * f2) < 1e-6


def pin_non_expansive(orc):
    """beta in [0,1], |k| = 1, alpha <= 1: ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    x = _case(25, 60, 2, 8, 8, mu=2.0, dtype="f32")
    S = x.initial_state.astype(np.float64).copy() * 10
    for t in range(x.T):
        before = np.linalg.norm(S.reshape(x.H, -1), axis=1)
        orc.decode_step(S, x.q[t][None], x.k[t][None], x.v[t][None], x.log_alpha[t][None],
                        x.beta[t][None])
        after = np.linalg.norm(S.reshape(x.H, -1), axis=1)
        bound = before + x.beta[t] * np.linalg.norm(x.v[t].astype(np.float64), axis=1)
        # fp32 unit keys carry |k|^2 = 1 +- 1e-7; the slack covers only that
        assert np.all(after <= bound * (1 + 1e-6))


# --------------------------------------------------------------------------
# options: state snapshots, in-call q/k normalisation and beta logits, pools
# --------------------------------------------------------------------------
def pin_state_snapshots(orc):
    """The state entering every C-th token of a sequence is the final state of
    the same sequence cut after that many tokens (the initial state at 0);
    rows follow the sequences in order, ceil(len / C) per sequence."""
    x = _case(27, 0, 2, 5, 4, lengths=[13, 0, 8, 1, 17])
    C = 4
    _, _, snaps = orc.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state,
                              x.cu_seqlens, states_every=C)
    row = 0
    for s, n in enumerate(x.lengths()):
        y = x.select_seqs([s])
        for c in range((n + C - 1) // C):
            if c == 0:
                expect = y.initial_state[0].astype(np.float64)
            else:
                _, f = orc.prefill(y.q[:C * c], y.k[:C * c], y.v[:C * c], y.log_alpha[:C * c],
                                   y.beta[:C * c], y.initial_state)
                expect = f[0]
            assert np.array_equal(snaps[row], expect), (s, c)
            row += 1
    assert row == snaps.shape[0]


def pin_qk_l2_normalisation(orc):
    """In-call L2 normalisation of q and k (per token and head, over dk):
    power-of-two rescaling of any row changes nothing but the regulariser's
    share; rows that are unit vectors already give the plain result; and with
    beta = 1 and q_t parallel to k_t the read-out recalls v_t exactly."""
    x = _case(28, 24, 2, 8, 5, raw=True)
    be = gen.as_f32(x.beta)
    q, k = x.q * np.float32(8), x.k * np.float32(8)        # exact; rows have |x|^2 >= 1e-2
    o1, f1 = orc.prefill(q, k, x.v, x.log_alpha, be, x.initial_state, l2norm_qk=True)
    g = np.random.default_rng(28)
    sq = np.exp2(g.integers(0, 7, (x.T, x.H, 1))).astype(np.float32)
    sk = np.exp2(g.integers(0, 7, (x.T, x.H, 1))).astype(np.float32)
    o2, f2 = orc.prefill(q * sq, k * sk, x.v, x.log_alpha, be, x.initial_state,
                         l2norm_qk=True)
    # the regulariser moves a row by at most 1e-6 / (2 |x|^2) relative
    bound = 1e-6 / min(np.einsum("thc,thc->th", q, q).min(), np.einsum("thc,thc->th", k, k).min())
    assert rel_err(o2, o1) < 4 * bound and rel_err(f2, f1) < 4 * bound, bound
    # unit rows: only the 1e-6 regulariser separates the two calls
    u = _case(29, 24, 2, 8, 5)
    o3, f3 = orc.prefill(u.q, u.k, u.v, u.log_alpha, u.beta, u.initial_state, l2norm_qk=True)
    o4, f4 = orc.prefill(u.q, u.k, u.v, u.log_alpha, u.beta, u.initial_state)
    assert rel_err(o3, o4) < 2e-6 and rel_err(f3, f4) < 2e-6
    # recall: |k|^2 ~ 1e4, so the normalised key has |k|^2 = 1 - 1e-10
    k = (x.k * np.float32(30.0)).astype(np.float32)
    o5, _ = orc.prefill((k * np.float32(0.5)).astype(np.float32), k, x.v, x.log_alpha,
                        np.ones_like(be), x.initial_state, l2norm_qk=True)
    assert rel_err(o5, _f64(x.v)) < 1e-8


def pin_beta_logit(orc):
    """beta given as a logit x: beta = sigmoid(x), so x = ln(p / (1 - p)) gives
    the plain call with beta = p."""
    x = _case(30, 20, 2, 6, 4)
    g = np.random.default_rng(30)
    p = g.choice([0.2, 0.25, 0.5, 0.75, 0.8], size=x.beta.shape)
    logit = np.log(p / (1.0 - p)).astype(np.float32)
    o1, f1 = orc.prefill(x.q, x.k, x.v, x.log_alpha, logit, x.initial_state, beta_logit=True)
    o2, f2 = orc.prefill(x.q, x.k, x.v, x.log_alpha, p.astype(np.float32), x.initial_state)
    # the logit is rounded to fp32: beta moves by ~1e-8
    assert rel_err(o1, o2) < 1e-6 and rel_err(f1, f2) < 1e-6


def pin_pooled_tokens(orc):
    """Recurrent tokens on a state pool: each sequence starts from its slot's
    state and leaves its final state there; a slot outside the pool marks a
    padding sequence (zero output, pool untouched).  Checked against
    token-by-token decode steps on copies of the slots."""
    x = _case(31, 0, 2, 5, 4, lengths=[4, 3, 0, 2, 5])
    P = 6
    g = np.random.default_rng(31)
    pool = 0.3 * g.standard_normal((P, x.H, x.dk, x.dv))
    slots = np.array([3, -1, 0, 7, 2], dtype=np.int32)
    got = pool.copy()
    o = orc.decode_tokens(got, slots, x.q, x.k, x.v, x.log_alpha, x.beta, x.cu_seqlens)
    ref = pool.copy()
    cu = x.cu_seqlens
    for s in range(x.num_seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        if not 0 <= slots[s] < P:
            assert not np.any(o[a:b])
            continue
        S = ref[slots[s]][None].copy()
        for t in range(a, b):
            ot = orc.decode_step(S, x.q[t][None], x.k[t][None], x.v[t][None],
                                 x.log_alpha[t][None], x.beta[t][None])
            assert rel_err(ot[0], o[t]) < 1e-13, (s, t)
        ref[slots[s]] = S[0]
    assert rel_err(got, ref) < 1e-13
    assert np.array_equal(got[[1, 4, 5]], pool[[1, 4, 5]])   # slots no sequence names


# --------------------------------------------------------------------------
# gradients: reverse mode against finite differences and an exact identity
# --------------------------------------------------------------------------
def _loss(orc, x, d_o, d_fin, **over):
    a = dict(q=x.q, k=x.k, v=x.v, log_alpha=x.log_alpha, beta=x.beta,
             initial_state=x.initial_state)
    a.update(over)
    o, fin = orc.prefill(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["initial_state"],
                         x.cu_seqlens, num_seqs=x.num_seqs)
    return float(np.sum(d_o * o) + np.sum(d_fin * fin))


def pin_backward_finite_differences(orc):
    """Every gradient entry of L = <dO, o> + <dS, S_T> against a central
    difference of the forward oracle (fp32 inputs perturbed by 2^-12; the
    step actually taken after fp32 rounding is the denominator)."""
    x = _case(32, 0, 1, 4, 3, mu=1.0, lengths=[5, 3])
    x = dataclasses.replace(x, v=(x.v * np.float32(0.5)).astype(np.float32))
    g = np.random.default_rng(32)
    d_o = g.standard_normal((x.T, x.H, x.dv))
    d_fin = g.standard_normal((x.num_seqs, x.H, x.dk, x.dv))
    gr = orc.backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens, d_o, d_fin)
    h = 2.0 ** -12
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_alpha", "dlog_alpha"),
                      ("beta", "dbeta"), ("initial_state", "dinitial_state")):
        base = getattr(x, name)
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] = np.float32(base[idx] + h)
            minus[idx] = np.float32(base[idx] - h)
            step = float(plus[idx]) - float(minus[idx])
            fd[idx] = (_loss(orc, x, d_o, d_fin, **{name: plus}) -
                       _loss(orc, x, d_o, d_fin, **{name: minus})) / step
        assert rel_err(gr[key], fd) < 1e-5, (name, rel_err(gr[key], fd))


def pin_backward_linear_part(orc):
    """o and S_T are linear in (S0, V) for fixed q, k, alpha, beta, so
    L(S0, V) = <dL/dS0, S0> + <dL/dV, V> exactly (Euler's identity)."""
    x = _case(33, 0, 2, 6, 5, mu=1.0, lengths=[9, 0, 14])
    g = np.random.default_rng(33)
    d_o = g.standard_normal((x.T, x.H, x.dv))
    d_fin = g.standard_normal((x.num_seqs, x.H, x.dk, x.dv))
    gr = orc.backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens, d_o, d_fin)
    L = _loss(orc, x, d_o, d_fin)
    euler = float(np.sum(gr["dinitial_state"] * x.initial_state) + np.sum(gr["dv"] * x.v))
    assert abs(L - euler) <= 1e-12 * max(1.0, abs(L)), (L, euler)
    # an empty sequence passes its final-state gradient straight through
    assert np.array_equal(gr["dinitial_state"][1], d_fin[1])


def pin_chunkwise_backward(orc):
    """The reverse mode of the chunkwise form (chunkwise_mirror.chunk_backward:
    entering-state gradients chained through the transposed chunk
    transitions, every input gradient chunk-local) gives the oracle's
    token-by-token gradients, for chunk sizes that do and do not divide the
    lengths."""
    x = _case(34, 0, 2, 8, 6, mu=1.0, lengths=[37, 0, 20, 64])
    g = np.random.default_rng(34)
    d_o = g.standard_normal((x.T, x.H, x.dv))
    d_fin = g.standard_normal((x.num_seqs, x.H, x.dk, x.dv))
    gr = orc.backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens, d_o, d_fin)
    q, k, v = (_f64(a) for a in (x.q, x.k, x.v))
    la, be = x.log_alpha.astype(np.float64), x.beta.astype(np.float64)
    offs = np.concatenate([[0], np.cumsum(x.lengths())])
    for C in (7, 16, 64):
        got = {n: np.zeros(gr[n].shape) for n in gr}
        for s in range(x.num_seqs):
            a, b = offs[s], offs[s + 1]
            for h in range(x.H):
                r = chunkwise_mirror.head_backward(q[a:b, h], k[a:b, h], v[a:b, h], la[a:b, h],
                                                   be[a:b, h], x.initial_state[s, h].astype(np.float64),
                                                   d_o[a:b, h], d_fin[s, h], C)
                for n, val in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta"), r[:5]):
                    got[n][a:b, h] = val
                got["dinitial_state"][s, h] = r[5]
        for n in gr:
            assert rel_err(got[n], gr[n]) < 1e-12, (C, n, rel_err(got[n], gr[n]))


ALL_PINS = [pin_transition_product, pin_exact_rational, pin_identity_no_write, pin_pure_decay,
            pin_deltanet, pin_gated_deltanet, pin_exact_recall, pin_one_hot_linear_attention,
            pin_one_hot_rows, pin_single_token, pin_chunkwise_algebra, pin_chunk_transition_form,
            pin_packing,
            pin_decode_matches_prefill, pin_linearity, pin_non_expansive,
            pin_state_snapshots, pin_qk_l2_normalisation, pin_beta_logit, pin_pooled_tokens,
            pin_backward_finite_differences, pin_backward_linear_part, pin_chunkwise_backward]
