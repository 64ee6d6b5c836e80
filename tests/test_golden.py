"""The oracle against the hand-worked example of tests/golden/ (CPU)."""
import numpy as np

import oracle
from golden_case import load


def test_oracle_matches_hand_worked_example():
    for d in (2, 64):
        x, o_ref, fin_ref = load(d=d, H=2)
        o, fin = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta)
        assert np.abs(o - o_ref).max() < 2e-6
        assert np.abs(fin - fin_ref).max() < 2e-6


def test_oracle_decode_matches_hand_worked_example():
    x, o_ref, fin_ref = load(d=64, H=1)
    S = np.zeros((1, 1, 64, 64))
    for t in range(2):
        o = oracle.decode_step(S, x.q[t:t + 1], x.k[t:t + 1], x.v[t:t + 1],
                               x.log_alpha[t:t + 1], x.beta[t:t + 1])
        assert np.abs(o[0] - o_ref[t]).max() < 2e-6
    assert np.abs(S - fin_ref).max() < 2e-6
