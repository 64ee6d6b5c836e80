"""GPU parity of kda_backward against the oracle's reverse-mode gradients
(needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, dev_f32, dev_qkv, device_inputs, host, rel_l2

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_prefill_amd.kda as k
    k.lib()


def _case(seed, lens, H, dk, dv, dtype, packed=True):
    x = gen.make_prefill(seed, lens, H=H, dk=dk, dv=dv, dtype=dtype, state_std=0.02,
                         packed=packed)
    g = np.random.default_rng(seed)
    d_o = g.standard_normal((x.T, H, dv)).astype(np.float32)
    if dtype == "bf16":
        d_o = gen.bf16_bits(d_o)
    d_fin = g.standard_normal((x.num_seqs, H, dk, dv)).astype(np.float32)
    return x, d_o, d_fin


def _gpu_backward(x, d_o, d_fin, **kw):
    import torch
    import gated_delta_rule_prefill_amd as kda
    d = device_inputs(x)
    g = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dev_qkv(d_o),
                     d["initial_state"], d["cu_seqlens"], num_seqs=d["num_seqs"],
                     d_final_state=dev_f32(d_fin), **kw)
    torch.cuda.synchronize()
    return g


def _check(x, d_o, d_fin, label):
    g = _gpu_backward(x, d_o, d_fin)
    ref = oracle.backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens,
                          gen.as_f32(d_o).astype(np.float64), d_fin.astype(np.float64),
                          num_seqs=x.num_seqs)
    errs = {n: rel_l2(host(g[n]), ref[n]) for n in GRADS}
    print(f"[backward] {label} {x.dtype} dk={x.dk} dv={x.dv}: " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL[x.dtype], (label, n, e)
    return g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_backward_matches_oracle(dtype, dk, dv):
    """Packed batch with an empty and a one-token sequence, chunks cut short,
    nonzero initial states and final-state gradient."""
    x, d_o, d_fin = _case(71, [70, 0, 130, 1, 64], 2, dk, dv, dtype)
    _check(x, d_o, d_fin, "packed")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_ragged_pieces(dtype):
    """Chunks whose last 8-token piece is cut short after full pieces (22, 13
    and 9 tokens): the tail of the piece past the chunk's end must leave every
    gradient alone."""
    x, d_o, d_fin = _case(75, [150, 77, 9], 2, 128, 128, dtype)
    _check(x, d_o, d_fin, "ragged pieces")


def test_backward_equal_rows_long():
    """Two equal sequences of 1,000 tokens (16 chunks each), bf16, d = 128."""
    x, d_o, d_fin = _case(72, [1000, 1000], 3, 128, 128, "bf16", packed=False)
    _check(x, d_o, d_fin, "equal rows")


def test_backward_given_chunk_states_is_the_same():
    """Chunk states exported by the forward give bit-for-bit the gradients the
    call computes when it recomputes them; and two runs are identical."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x, d_o, d_fin = _case(73, [150, 77], 2, 128, 128, "bf16")
    d = device_inputs(x)
    _, _, cs = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                           d["cu_seqlens"], chunk_states=True)
    g1 = _gpu_backward(x, d_o, d_fin, chunk_states=cs)
    g2 = _gpu_backward(x, d_o, d_fin)
    g3 = _gpu_backward(x, d_o, d_fin)
    for n in GRADS:
        assert torch.equal(g1[n].cpu(), g2[n].cpu()), n
        assert torch.equal(g2[n].cpu(), g3[n].cpu()), n


def test_backward_without_final_gradient_fp32():
    """d_final_state = NULL means zero; no initial state means zero."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x = gen.make_prefill(74, [90], H=2, dk=64, dv=64, dtype="f32")
    g = np.random.default_rng(74)
    d_o = g.standard_normal((x.T, 2, 64)).astype(np.float32)
    d = device_inputs(x)
    gr = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dev_qkv(d_o))
    torch.cuda.synchronize()
    ref = oracle.backward(x.q, x.k, x.v, x.log_alpha, x.beta, None, None, d_o.astype(np.float64))
    for n in GRADS:
        assert rel_l2(host(gr[n]), ref[n]) <= TOL["f32"], n
