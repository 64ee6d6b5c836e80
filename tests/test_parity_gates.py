"""The GPU tests' per-unit gates catch faults that a pooled error would hide
(CPU only: the faults are planted in copies of the oracle's own output)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, unit_errors


@pytest.fixture(scope="module")
def case():
    lens = [1100, 300, 0, 64]
    x = gen.make_prefill(81, lens, H=4, dk=64, dv=64, dtype="f32", state_std=0.02, packed=True)
    ro, rf = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens)
    return x, ro, rf


def _bf16_round(a):
    return gen.bf16_to_f32(gen.bf16_bits(a.astype(np.float32))).astype(np.float64)


def test_clean_bf16_rounding_passes(case):
    x, ro, rf = case
    e = unit_errors(_bf16_round(ro), ro, rf, rf, x.lengths())
    assert max(e["o"], e["seq_head_o"], e["chunk_o"]) < 4e-3 and e["row_o"] < 1e-2, e


def test_one_wrong_row_is_caught_per_row_and_chunk(case):
    x, ro, rf = case
    o = _bf16_round(ro)
    o[700, 2] *= 1.3                  # one (token, head) row 30 % off
    e = unit_errors(o, ro, rf, rf, x.lengths())
    assert e["o"] <= TOL["bf16"]      # the pooled error alone would pass
    assert e["row_o"] > 0.25 and e["worst_row"] == (700, 2)
    assert e["chunk_o"] > TOL["bf16"]


def test_wrong_column_slice_in_one_chunk_is_caught(case):
    x, ro, rf = case
    o = _bf16_round(ro)
    o[1200:1264, 1, 16:32] *= 1.2     # 16 value columns of one chunk of sequence 1
    e = unit_errors(o, ro, rf, rf, x.lengths())
    assert e["o"] <= TOL["bf16"]
    assert e["chunk_o"] > TOL["bf16"]


def test_wrong_final_state_of_one_head_is_caught(case):
    x, ro, rf = case
    f = rf.copy()
    f[1, 3, :, :8] *= 1.5
    e = unit_errors(ro, ro, f, rf, x.lengths())
    assert e["seq_head_state"] > TOL["bf16"]


def test_short_units_fall_under_the_row_bound(case):
    """A 5 % error on one row moves the 64-row unit that holds it by well
    under the tolerance, while the row gate still reports it."""
    x, ro, rf = case
    lens = x.lengths()
    o = _bf16_round(ro)
    a = int(np.sum(lens)) - lens[-1]       # the 64-token sequence: its largest row
    last = a + int(np.argmax(np.linalg.norm(ro[a:, 0], axis=1)))
    o[last, 0] *= 1.05
    e = unit_errors(o, ro, rf, rf, lens)
    assert e["row_o"] > 0.04 and e["chunk_o"] < TOL["bf16"]
