"""GPU parity of kda_backward against the oracle's reverse-mode gradients
(needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import MIN_UNIT_ROWS, TOL, dev_f32, dev_qkv, device_inputs, host, rel_l2

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_prefill_amd.kda as k
    k.lib()


def _case(seed, lens, H, dk, dv, dtype, packed=True, mu=3.0, fixed=None):
    x = gen.make_prefill(seed, lens, H=H, dk=dk, dv=dv, dtype=dtype, state_std=0.02,
                         packed=packed, mu=mu, fixed_even_log_alpha=fixed)
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
    # per sequence as well (sequences of at least MIN_UNIT_ROWS tokens: on
    # shorter ones the bf16 rounding of a few products is the whole signal)
    lens = np.diff(x.cu_seqlens) if x.cu_seqlens is not None else [x.T // x.num_seqs] * x.num_seqs
    at = 0
    for s, n_tok in enumerate(lens):
        if n_tok >= MIN_UNIT_ROWS:
            for n in GRADS[:5]:
                e = rel_l2(host(g[n])[at:at + n_tok], ref[n][at:at + n_tok])
                assert e <= TOL[x.dtype], (label, "sequence", s, n, e)
        at += n_tok
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
    call computes when it recomputes them; two runs are identical, and so is a
    run in a caller workspace whose bytes start as garbage (nothing is read
    before it is written)."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x, d_o, d_fin = _case(73, [150, 77], 2, 128, 128, "bf16")
    d = device_inputs(x)
    _, _, cs = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                           d["cu_seqlens"], chunk_states=True)
    g1 = _gpu_backward(x, d_o, d_fin, chunk_states=cs)
    g2 = _gpu_backward(x, d_o, d_fin)
    g3 = _gpu_backward(x, d_o, d_fin)
    need = kda.backward_workspace_bytes(x.T, x.num_seqs, x.H, x.dk, x.dv, True)
    ws = torch.full((need,), 0xA7, dtype=torch.uint8, device="cuda")
    g4 = _gpu_backward(x, d_o, d_fin, workspace=ws)
    for n in GRADS:
        assert torch.equal(g1[n].cpu(), g2[n].cpu()), n
        assert torch.equal(g2[n].cpu(), g3[n].cpu()), n
        assert torch.equal(g2[n].cpu(), g4[n].cpu()), n


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


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 128), ("bf16", 64)])
@pytest.mark.parametrize("mu,fixed", [(0.0, None), (-1.0, None), (3.0, -3.0)],
                         ids=["mu0", "mu-1", "fixed-3"])
def test_backward_strong_decay(dtype, dk, mu, fixed):
    """Strong per-channel decay (paper notes section 2: every key channel has its
    own forgetting rate): log_alpha = logsigmoid(N(mu, 1)) with mu = 0 or -1
    (16-token block sums near -13 and -22), or the even channels fixed at -3
    (block sums of -48); the chunkwise gradients' block-referenced decay
    factors run near their range.  Packed with empty, one-token and cut chunks."""
    x, d_o, d_fin = _case(81, [200, 1, 64, 0, 131, 77], 2, dk, dk, dtype, mu=mu, fixed=fixed)
    _check(x, d_o, d_fin, f"strong decay mu={mu} fixed={fixed}")


def test_backward_long_packed():
    """About 4,000 tokens in four sequences (one a single chunk), H = 4, bf16,
    d = 128: the reverse chain over up to 32 chunks and the gradient kernel on
    every chunk."""
    x, d_o, d_fin = _case(82, [1500, 64, 2000, 531], 4, 128, 128, "bf16")
    _check(x, d_o, d_fin, "long packed")


_SERIAL_CHILD = r"""
import sys, numpy as np, torch
root = sys.argv[1]
sys.path.insert(0, root); sys.path.insert(0, root + '/tests')
import oracle
import gated_delta_rule_prefill_amd as kda
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, dev_f32, dev_qkv, device_inputs, host, rel_l2
x = gen.make_prefill(83, [150, 1, 77], H=2, dk=128, dv=128, dtype="bf16", state_std=0.02)
g = np.random.default_rng(83)
d_o = gen.bf16_bits(g.standard_normal((x.T, 2, 128)).astype(np.float32))
d_fin = g.standard_normal((x.num_seqs, 2, 128, 128)).astype(np.float32)
d = device_inputs(x)
gr = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], dev_qkv(d_o),
                  d["initial_state"], d["cu_seqlens"], num_seqs=x.num_seqs,
                  d_final_state=dev_f32(d_fin))
torch.cuda.synchronize()
ref = oracle.backward(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens,
                      gen.as_f32(d_o).astype(np.float64), d_fin.astype(np.float64),
                      num_seqs=x.num_seqs)
for n in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dinitial_state"):
    e = rel_l2(host(gr[n]), ref[n])
    print(f"[backward serial] {n}={e:.2e}", flush=True)
    assert e <= TOL["bf16"], (n, e)
print("RESULT|ok", flush=True)
"""


def test_backward_token_walk_selected_by_environment():
    """KDA_BACKWARD_SERIAL=1 (read once per process) sends bf16 at d = 128
    through the token-serial kernels; a child process checks them against the
    oracle on a packed batch with a one-token sequence."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, KDA_BACKWARD_SERIAL="1")
    r = subprocess.run([sys.executable, "-u", "-c", _SERIAL_CHILD, root], env=env,
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0 and "RESULT|ok" in r.stdout


def test_backward_long_context_sampled_heads():
    """The headline length: one 65,536-token sequence, H = 32, bf16, d = 128
    (1,024 chunks: the reverse chain over the whole sequence).  Two heads,
    the first and the last, are compared with the oracle over every token,
    together with their initial-state gradients."""
    T, H = 65536, 32
    x = gen.make_prefill(84, [T], H=H, dk=128, dv=128, dtype="bf16", mu=4.0, state_std=0.02)
    g = np.random.default_rng(84)
    d_o = gen.bf16_bits(g.standard_normal((T, H, 128)).astype(np.float32))
    d_fin = g.standard_normal((1, H, 128, 128)).astype(np.float32)
    gr = _gpu_backward(x, d_o, d_fin)
    heads = [0, H - 1]

    def sub(a):
        return np.ascontiguousarray(a[:, heads])

    ref = oracle.backward(sub(x.q), sub(x.k), sub(x.v), sub(x.log_alpha), sub(x.beta),
                          sub(x.initial_state), None, gen.as_f32(sub(d_o)).astype(np.float64),
                          sub(d_fin).astype(np.float64), num_seqs=1)
    for n in GRADS:
        got = host(gr[n][:, heads])
        for j, hd in enumerate(heads):
            e = rel_l2(got[:, j], ref[n][:, j])
            print(f"[backward long] head {hd} {n}={e:.2e}", flush=True)
            assert e <= TOL["bf16"], (hd, n, e)


@pytest.mark.parametrize("seed", range(8))
def test_backward_random_configuration(seed):
    """Seeded random batches across the axes the backward branches on: the
    chunkwise path (bf16, d = 128) or the token walk, head counts that are
    not a multiple of 8, packed or equal rows with empty, one-token and
    partial-chunk sequences, and the decay strength."""
    g = np.random.default_rng([23, seed])
    if seed < 4:   # the chunkwise path
        dtype, dk, dv = "bf16", 128, 128
    else:
        dtype = ["f32", "bf16"][int(g.integers(2))]
        dk, dv = [(64, 64), (128, 64), (64, 128), (128, 128)][int(g.integers(4))]
    H = int(g.choice([1, 2, 3, 5, 8]))
    packed = seed % 2 == 1
    N = int(g.integers(2 if packed else 1, 9))
    if packed:
        lens = [int(x) for x in g.integers(0, 300, N)]
        lens[int(g.integers(N))] = int(g.choice([0, 1, 63, 65]))
    else:
        lens = [int(g.choice([64, 97, 200]))] * N
    mu = float(g.choice([0.0, 3.0, 4.0]))
    x, d_o, d_fin = _case(600 + seed, lens, H, dk, dv, dtype, packed=packed, mu=mu)
    _check(x, d_o, d_fin, f"random case {seed} (H={H}, N={N}, {'packed' if packed else 'equal rows'}, mu={mu})")
