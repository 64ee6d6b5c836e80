"""Equal-row batches whose records exceed the segment budget run in token
segments, the fp32 state passing from one segment to the next.  A child
process with a tiny budget (KDA_SEGMENT_RECORD_BYTES, read once per process)
makes small inputs take many segments; outputs, final states and chunk
states are compared with the fp64 oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import sys, numpy as np, torch
root = sys.argv[1]
sys.path.insert(0, root); sys.path.insert(0, root + '/tests')
import oracle
import gated_delta_rule_prefill_amd as kda
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import assert_units, device_inputs, host, rel_l2, unit_errors, TOL
ok = 0
for dtype, dk, dv, lens, alias, want_final in (
        ("bf16", 128, 128, [1000, 1000], False, True),
        ("bf16", 128, 128, [700], True, True),
        ("f32", 64, 64, [1000, 1000, 1000], False, False),
        ("f32", 128, 64, [129, 129], False, True)):
    x = gen.make_prefill(95, lens, H=4, dk=dk, dv=dv, dtype=dtype, state_std=0.02)
    d = device_inputs(x)
    s0 = d["initial_state"]
    fin = s0 if alias else (torch.empty_like(s0) if want_final else None)
    s0_host = x.initial_state.copy()
    o, f, cs = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s0, None,
                           num_seqs=x.num_seqs, final_state=fin, output_final_state=want_final,
                           chunk_states=True)
    torch.cuda.synchronize()
    ro, rf, rs = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, s0_host, None,
                                num_seqs=x.num_seqs, states_every=64)
    label = f"segments {dtype} {dk}x{dv} lens={lens} alias={alias} final={want_final}"
    if want_final:
        assert_units(unit_errors(host(o), ro, host(f), rf, x.lengths()), dtype, label)
    else:
        assert_units(unit_errors(host(o), ro, rf, rf, x.lengths()), dtype, label)
    ecs = rel_l2(host(cs), rs)
    print(f"[segments] {label}: chunk states {ecs:.3e}", flush=True)
    assert ecs <= TOL[dtype], ecs
    ok += 1
print(f"RESULT|{ok}", flush=True)
"""


def test_segmented_equal_rows_match_oracle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, KDA_SEGMENT_RECORD_BYTES=str(2_500_000))
    r = subprocess.run([sys.executable, "-u", "-c", _CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=600)
    print(r.stdout[-6000:], flush=True)
    assert r.returncode == 0 and "RESULT|4" in r.stdout, (r.returncode, r.stderr[-3000:])
