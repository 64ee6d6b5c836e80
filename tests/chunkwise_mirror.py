"""fp64 NumPy statement of the chunkwise form of KDA (test reference).

The pages describe the prefill as a chunkwise-parallel computation: inside a
chunk of C tokens the C rank-1 transitions are folded into a dense WY/UT-style
form (matrices W and U), the output splits into an inter-chunk term (read-out
of the state entering the chunk) and an intra-chunk term, and only the fixed
dk x dv state passes from one chunk to the next (Kimi Linear paper notes,
section 3 "chunkwise parallel"; the listed chunk intermediates are the
cumulative log-decay g, A_qk, A_kk, w, u, the decayed q and k, the corrected
values v_new and the chunk states h).

The equations, derived from the recurrence by unrolling it inside a chunk
(exact algebra, no approximation), for one head and one chunk of rows
r = 1..C entering with state S0:

    g_r   = sum_{j<=r} log alpha_j               (per channel, restarts per chunk)
    A_kk[r,i] = beta_r sum_c k_rc k_ic exp(g_rc - g_ic)   for i < r
    A_qk[r,i] =        sum_c q_rc k_ic exp(g_rc - g_ic)   for i <= r
    T     = (I + A_kk)^{-1} Diag(beta)
    W     = T (exp(g) * K),   U = T V
    N     = U - W S0                               (corrected values)
    O     = (exp(g) * Q) S0 + A_qk N               (inter + intra)
    S_C   = Diag(exp(g_C)) S0 + (exp(g_C - g) * K)^T N

Folding W and U into the chunk gives the equivalent transition / read-out
form used by the GPU's sequential pass:

    S_C = Diag(exp(g_C)) S0 + PM S0 + Hc,     O = QM S0 + OI
    PM = -Khat^T W,  Hc = Khat^T U,  QM = Qg - A_qk W,  OI = A_qk U

This module is test infrastructure: it is not the oracle (the oracle is the
token-by-token recurrence) and it shares no code with the GPU library.  The
pins check it against the oracle for several chunk sizes; GPU stage tests
may compare intermediates with it.
"""
from __future__ import annotations

import numpy as np

from gated_delta_rule_prefill_amd import inputs as gen


def chunk_terms(q, k, v, la, beta):
    """Intermediates of one chunk (fp64): g, A_kk, A_qk, T, W, U, Khat, Qg."""
    n = k.shape[0]
    g = np.cumsum(la, axis=0)
    gam = np.exp(g)
    D = g[:, None, :] - g[None, :, :]                     # D[r, i, c] = g_rc - g_ic
    with np.errstate(over="ignore", invalid="ignore"):
        E = np.exp(D)
        L = np.einsum("rc,ic,ric->ri", k, k, E)
        Aqk = np.einsum("rc,ic,ric->ri", q, k, E)
    Akk = np.where(np.tri(n, k=-1, dtype=bool), beta[:, None] * L, 0.0)
    Aqk = np.where(np.tri(n, dtype=bool), Aqk, 0.0)
    Tm = np.linalg.solve(np.eye(n) + Akk, np.diag(beta))
    W = Tm @ (gam * k)
    U = Tm @ v
    Khat = np.exp(g[-1][None, :] - g) * k
    Qg = gam * q
    return dict(g=g, Akk=Akk, Aqk=Aqk, T=Tm, W=W, U=U, Khat=Khat, Qg=Qg, gC=gam[-1])


def head_sequence(q, k, v, la, beta, S0, C):
    """One head of one sequence in chunks of C tokens.  Returns (O, S_final)."""
    T = q.shape[0]
    S = S0.copy()
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        t = chunk_terms(q[sl], k[sl], v[sl], la[sl], beta[sl])
        N = t["U"] - t["W"] @ S
        O[sl] = t["Qg"] @ S + t["Aqk"] @ N
        S = t["gC"][:, None] * S + t["Khat"].T @ N
    return O, S


def head_sequence_transition(q, k, v, la, beta, S0, C):
    """The same chunks in transition / read-out form.  Returns (O, S_final)."""
    T = q.shape[0]
    S = S0.copy()
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        t = chunk_terms(q[sl], k[sl], v[sl], la[sl], beta[sl])
        PM = -t["Khat"].T @ t["W"]
        Hc = t["Khat"].T @ t["U"]
        QM = t["Qg"] - t["Aqk"] @ t["W"]
        OI = t["Aqk"] @ t["U"]
        O[sl] = QM @ S + OI
        S = t["gC"][:, None] * S + PM @ S + Hc
    return O, S


def prefill(x: "gen.KDAInputs", C: int, transition: bool = False):
    """The whole packed batch in chunks of C tokens (fp64)."""
    q, k, v = (gen.as_f32(a).astype(np.float64) for a in (x.q, x.k, x.v))
    la = x.log_alpha.astype(np.float64)
    be = x.beta.astype(np.float64)
    lens = x.lengths()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    O = np.zeros((x.T, x.H, x.dv))
    F = np.zeros((x.num_seqs, x.H, x.dk, x.dv))
    for s in range(x.num_seqs):
        a, b = offs[s], offs[s + 1]
        for h in range(x.H):
            S0 = np.zeros((x.dk, x.dv)) if x.initial_state is None else \
                x.initial_state[s, h].astype(np.float64)
            fn = head_sequence_transition if transition else head_sequence
            O[a:b, h], F[s, h] = fn(q[a:b, h], k[a:b, h], v[a:b, h], la[a:b, h], be[a:b, h],
                                    S0, C)
    return O, F


def chunk_backward(q, k, v, la, beta, S, dS, dO):
    """Reverse mode through one chunk (fp64).  S: state entering the chunk,
    dS: gradient of the loss with respect to the state leaving it, dO: with
    respect to the chunk's outputs.  Returns (dq, dk, dv, dla, dbeta, dS_in),
    dS_in being the gradient with respect to the entering state.

    Every input gradient of a chunk depends only on the chunk, S and dS; the
    entering-state gradient follows the transpose of the forward transition,
    dS_in = Diag(gamma_C) dS + Qg^T dO - W^T dN = (Diag(gamma_C) + PM^T) dS + QM^T dO.
    """
    n = k.shape[0]
    t = chunk_terms(q, k, v, la, beta)
    g, Aqk, Tm, W, U, Khat, Qg = (t[a] for a in ("g", "Aqk", "T", "W", "U", "Khat", "Qg"))
    gam, gC = np.exp(g), t["gC"]
    E = np.exp(g[:, None, :] - g[None, :, :])              # E[r, i, c] = exp(g_rc - g_ic)
    strict = np.tri(n, k=-1, dtype=bool)
    L = np.where(strict, np.einsum("rc,ic,ric->ri", k, k, E), 0.0)   # A_kk without beta
    X = np.linalg.inv(np.eye(n) + beta[:, None] * L)
    N = U - W @ S
    # through O = Qg S + A_qk N and S_C = Diag(gamma_C) S + Khat^T N
    dN = Aqk.T @ dO + Khat @ dS
    dS_in = gC[:, None] * dS + Qg.T @ dO - W.T @ dN
    dQg = dO @ S.T
    dAqk = np.tril(dO @ N.T)
    dKhat = N @ dS.T
    # through N = U - W S, W = T (e^g K), U = T V, T = X Diag(beta), X = (I + A_kk)^{-1}
    dW = -dN @ S.T
    dT = np.tril(dW @ (gam * k).T + dN @ v.T)
    dKg = Tm.T @ dW
    dv = Tm.T @ dN
    dbeta = np.sum(dT * X, axis=0)
    dA = np.where(strict, -(X.T @ (dT * beta[None, :]) @ X.T), 0.0)
    dbeta += np.sum(dA * L, axis=1)
    dL = beta[:, None] * dA
    # the decayed products M[r, i] = sum_c a_rc b_ic exp(g_rc - g_ic)
    def through(dM, a, b):
        da = np.einsum("ri,ic,ric->rc", dM, b, E)
        db = np.einsum("ri,rc,ric->ic", dM, a, E)
        return da, db
    daL, dbL = through(dL, k, k)
    daQ, dbQ = through(dAqk, q, k)
    eh = np.exp(g[-1][None, :] - g)                       # exp(g_C - g); gC is exp(g_C)
    dq = gam * dQg + daQ
    dk = gam * dKg + eh * dKhat + daL + dbL + dbQ
    dg = q * gam * dQg + k * gam * dKg - k * eh * dKhat + k * daL - k * dbL + q * daQ - k * dbQ
    dg[-1] += np.sum(k * eh * dKhat, axis=0) + gC * np.sum(S * dS, axis=1)
    dla = np.cumsum(dg[::-1], axis=0)[::-1]
    return dq, dk, dv, dla, dbeta, dS_in


def head_backward(q, k, v, la, beta, S0, dO, dSf, C):
    """One head of one sequence, chunk by chunk in reverse (fp64).  Returns
    (dq, dk, dv, dla, dbeta, dS0)."""
    T = q.shape[0]
    starts = list(range(0, T, C))
    states, S = [], S0.copy()
    for c0 in starts:                        # chunk-entry states (forward)
        sl = slice(c0, min(c0 + C, T))
        t = chunk_terms(q[sl], k[sl], v[sl], la[sl], beta[sl])
        states.append(S)
        S = t["gC"][:, None] * S + t["Khat"].T @ (t["U"] - t["W"] @ S)
    out = [np.zeros_like(a) for a in (q, k, v, la)] + [np.zeros_like(beta)]
    dS = dSf.copy()
    for c0, S in zip(reversed(starts), reversed(states)):
        sl = slice(c0, min(c0 + C, T))
        r = chunk_backward(q[sl], k[sl], v[sl], la[sl], beta[sl], S, dS, dO[sl])
        for o, g in zip(out, r[:5]):
            o[sl] = g
        dS = r[5]
    return (*out, dS)
