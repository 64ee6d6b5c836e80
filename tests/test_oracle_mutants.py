"""The pins can fail: each plausible mistake planted in a copy of the oracle
(on the CPU, in a temporary build) must be caught by at least one pin."""
import pytest

import oracle
import pins

# (name, text in kda_oracle.c, replacement)
MUTANTS = [
    ("no decay", "S[(int64_t)c * dv + j] *= a;", "S[(int64_t)c * dv + j] *= 1.0;"),
    ("decay sign", "double a = exp(la[c]);", "double a = exp(-la[c]);"),
    ("query in correction", "y[j] += k[c] * S[(int64_t)c * dv + j];",
     "y[j] += q[c] * S[(int64_t)c * dv + j];"),
    ("correction with undecayed state", "y[j] += k[c] * S[(int64_t)c * dv + j];",
     "y[j] += k[c] * S[(int64_t)c * dv + j] / exp(la[c]);"),
    ("correction sign", "(v[j] - y[j]);", "(v[j] + y[j]);"),
    ("beta dropped on erase", "S[(int64_t)c * dv + j] += beta * k[c] * (v[j] - y[j]);",
     "S[(int64_t)c * dv + j] += beta * k[c] * v[j] - k[c] * y[j];"),
    ("read-out with key", "o[j] += q[c] * S[(int64_t)c * dv + j];",
     "o[j] += k[c] * S[(int64_t)c * dv + j];"),
    ("read-out before write", "o[j] += q[c] * S[(int64_t)c * dv + j];",
     "o[j] += q[c] * (S[(int64_t)c * dv + j] - beta * k[c] * (v[j] - y[j]));"),
    ("bf16 widening", "<< 16;", "<< 15;"),
    ("initial state ignored", "S[i] = (double)S0[i];", "S[i] = 0.0 * S0[i];"),
    ("packed offset", "t0 = cu_seqlens[s];", "t0 = cu_seqlens[s] + (s > 0 && cu_seqlens[s] < cu_seqlens[s + 1]);"),
    ("scalar decay", "lv[c] = (double)log_alpha[rk + c];", "lv[c] = (double)log_alpha[rk];"),
    ("decode beta", "(double)beta[u]", "(double)beta[0]"),
    ("q not normalised", "l2_normalise(qv, dk);", ";"),
    ("k not normalised", "l2_normalise(kv, dk);", ";"),
    ("norm over half the channels", "l2_normalise(kv, dk);", "l2_normalise(kv, dk / 2);"),
    ("sigmoid sign", "b = 1.0 / (1.0 + exp(-b));", "b = 1.0 / (1.0 + exp(b));"),
    ("snapshot one token late", "(t - t0) % every == 0", "(t - t0) % every == 1 % every"),
    ("snapshot rows", "snap_base[s + 1] = snap_base[s] +", "snap_base[s + 1] = snap_base[s] * 0 +"),
    ("backward: key term of the correction dropped", "acc += X[(int64_t)c2 * dv + j] * dy[j];", "acc += 0.0 * dy[j];"),
    ("backward: decay gradient from the undecayed state", "acc += G[(int64_t)c2 * dv + j] * X[(int64_t)c2 * dv + j];",
     "acc += G[(int64_t)c2 * dv + j] * Sprev[(int64_t)c2 * dv + j];"),
    ("backward: decay not applied to the carried gradient", "G[(int64_t)c2 * dv + j] *= av[c2];", "G[(int64_t)c2 * dv + j] *= 1.0;"),
    ("backward: correction sign", "dy[j] = -bt * gk[j];", "dy[j] = bt * gk[j];"),
    ("backward: read-out from the pre-update state", "acc += Snew[(int64_t)c2 * dv + j] * dov[j];",
     "acc += Sprev[(int64_t)c2 * dv + j] * dov[j];"),
    ("backward: beta gradient without the prediction", "db += gk[j] * (vv[j] - y[j]);", "db += gk[j] * vv[j];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = oracle.source()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    mutant = oracle.compile_variant(src.replace(old, new, 1), str(tmp_path / "libmutant.so"))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # AssertionError, or the mutant rejecting valid input
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {name!r}"
