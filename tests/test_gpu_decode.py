"""GPU parity of kda_decode_step against the fp64 oracle (needs an MI355X)."""
import numpy as np
import pytest

import oracle
from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import ROW_TOL, TOL, dev_f32, dev_qkv, host, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_decode(seed, N, H, dk, dv, steps, dtype):
    """Run `steps` decode tokens on the GPU and on the oracle for every
    (sequence, head).  Returns the worst whole-step o error, the worst
    (sequence, head) o error over all steps, the worst single o row, and the
    whole and worst (sequence, head) state errors after the last step."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    S0 = gen.decode_state(seed, N, H, dk, dv)
    state = dev_f32(S0)
    ref_state = S0.astype(np.float64)
    worst_step = worst_row = 0.0
    e2 = np.zeros((N, H))
    r2 = np.zeros((N, H))
    for step in range(steps):
        x = gen.decode_token(seed, step, N, H, dk, dv, dtype=dtype)
        o = kda.decode_step(state, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v),
                            dev_f32(x.log_alpha), dev_f32(x.beta))
        ro = oracle.decode_step(ref_state, x.q, x.k, x.v, x.log_alpha, x.beta)
        go = host(o)
        worst_step = max(worst_step, rel_l2(go, ro))
        de = ((go - ro) ** 2).sum(axis=2)
        dr = (ro ** 2).sum(axis=2)
        e2 += de
        r2 += dr
        worst_row = max(worst_row, float(np.max(np.sqrt(de) / np.maximum(np.sqrt(dr), 1e-300))))
    torch.cuda.synchronize()
    gs = host(state)
    es = rel_l2(gs, ref_state)
    unit_s = np.sqrt(((gs - ref_state) ** 2).sum(axis=(2, 3)) / (ref_state ** 2).sum(axis=(2, 3)))
    unit_o = np.sqrt(e2 / r2)
    return worst_step, float(unit_o.max()), worst_row, es, float(unit_s.max())


def _gate(res, dtype, label):
    eo, uo, ro, es, us = res
    print(f"[parity] decode {label} {dtype}: worst step o={eo:.3e}, worst (seq,head) o={uo:.3e}, "
          f"worst row={ro:.3e}; state={es:.3e}, worst (seq,head) state={us:.3e}", flush=True)
    assert max(eo, uo, es, us) <= TOL[dtype], res
    assert ro <= ROW_TOL[dtype], res


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_small(dtype, dk, dv):
    _gate(run_decode(41, N=3, H=2, dk=dk, dv=dv, steps=8, dtype=dtype), dtype, f"{dk}x{dv}")


def test_decode_256x32_full():
    """256 sequences x 32 heads, 128 steps; the oracle follows every one of the
    8,192 (sequence, head) states through all 128 steps."""
    c = gen.DECODE_WORKLOAD
    _gate(run_decode(c["seed"], c["N"], c["H"], c["dk"], c["dv"], c["steps"], c["dtype"]),
          c["dtype"], "256 x 32 decode (all 8192 units, 128 steps)")


def test_hand_worked_example():
    """The two-token example of tests/golden/ as two decode steps."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    from golden_case import load
    x, o_ref, fin_ref = load(d=64, H=2)
    state = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    for t in range(2):
        o = kda.decode_step(state, dev_qkv(x.q[t:t + 1]), dev_qkv(x.k[t:t + 1]),
                            dev_qkv(x.v[t:t + 1]), dev_f32(x.log_alpha[t:t + 1]),
                            dev_f32(x.beta[t:t + 1]))
        assert np.abs(host(o)[0] - o_ref[t]).max() < 1e-5
    assert np.abs(host(state) - fin_ref).max() < 1e-5


# -- closed forms at the batched-decode size ---------------------------------------
# Properties of the recurrence that hold exactly, checked on every
# (sequence, head) of a 256 x 32-head batch against numpy on the same inputs
# (no oracle): they pin the step's decay, write and read-out separately.

def _batch(seed, dtype, N=256, H=32, D=128):
    return gen.decode_token(seed, 0, N, H, D, D, dtype=dtype), gen.decode_state(seed, N, H, D, D)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_without_write_only_decays(dtype):
    """beta = 0: nu = 0, so the step writes nothing; the state becomes
    Diag(alpha) S and o = (Diag(alpha) S)^T q."""
    import gated_delta_rule_prefill_amd as kda
    x, S0 = _batch(51, dtype)
    state = dev_f32(S0)
    o = kda.decode_step(state, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v), dev_f32(x.log_alpha),
                        dev_f32(np.zeros_like(x.beta)))
    S1 = S0.astype(np.float64) * np.exp(x.log_alpha.astype(np.float64))[..., None]
    o_ref = np.einsum("nhkv,nhk->nhv", S1, gen.as_f32(x.q).astype(np.float64))
    gs = host(state)
    unit = np.sqrt(((gs - S1) ** 2).sum(axis=(2, 3)) / (S1 ** 2).sum(axis=(2, 3)))
    eo = rel_l2(host(o), o_ref)
    print(f"[closed form] decode, beta = 0, {dtype}: worst state {unit.max():.2e}, o {eo:.2e}", flush=True)
    assert unit.max() <= 1e-6
    assert eo <= (1e-5 if dtype == "f32" else TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_unit_key_recall(dtype):
    """alpha = 1, beta = 1 and a unit key e_j: the delta rule replaces what
    the state held under k by v, so row j of the new state is v and every
    other row is unchanged (bit for bit)."""
    import gated_delta_rule_prefill_amd as kda
    x, S0 = _batch(52, dtype)
    N, H, D = S0.shape[:3]
    jj = np.random.default_rng(52).integers(0, D, size=(N, H))
    k = np.zeros((N, H, D), np.float32)
    np.put_along_axis(k, jj[..., None], 1.0, axis=2)
    k = gen.bf16_bits(k) if dtype == "bf16" else k
    state = dev_f32(S0)
    kda.decode_step(state, dev_qkv(x.q), dev_qkv(k), dev_qkv(x.v), dev_f32(np.zeros_like(x.log_alpha)),
                    dev_f32(np.ones_like(x.beta)))
    gs = host(state)
    v = gen.as_f32(x.v).astype(np.float64)
    row = np.take_along_axis(gs, jj[..., None, None], axis=2)[:, :, 0]
    er = float(np.max(np.abs(row - v)) / np.max(np.abs(v)))
    mask = np.ones((N, H, D), bool)
    np.put_along_axis(mask, jj[..., None], False, axis=2)
    rest_equal = np.array_equal(gs[mask], S0.astype(np.float64)[mask])
    print(f"[closed form] decode, unit-key recall, {dtype}: row j vs v {er:.2e}, "
          f"other rows unchanged: {rest_equal}", flush=True)
    assert er <= 1e-6 and rest_equal


def test_decode_tokens_without_write_only_decay():
    """The pooled path's chunkwise form (256 sequences x 8 tokens, bf16) with
    beta = 0: each state becomes Diag(prod alpha) S, and token t reads out
    (Diag(alpha_1 .. alpha_t) S)^T q_t."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    H, D, N, R = 32, 128, 256, 8
    x = gen.make_prefill(53, [R] * N, H=H, dk=D, dv=D, dtype="bf16")
    pool = gen.decode_state(53, N, H, D, D)
    slots = np.random.default_rng(53).permutation(N).astype(np.int32)
    p = dev_f32(pool)
    o = kda.decode_tokens(p, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v), dev_f32(x.log_alpha),
                          dev_f32(np.zeros_like(x.beta)), state_indices=torch.from_numpy(slots).cuda(),
                          num_seqs=N)
    torch.cuda.synchronize()
    la = x.log_alpha.astype(np.float64).reshape(N, R, H, D)
    g = np.cumsum(la, axis=1)                                   # per sequence, token, head, channel
    S = pool.astype(np.float64)[slots]                          # [N, H, D, D], sequence order
    q = gen.as_f32(x.q).astype(np.float64).reshape(N, R, H, D)
    o_ref = np.einsum("nhkv,ntkh->nthv", S, (np.exp(g) * q).transpose(0, 1, 3, 2)).reshape(N * R, H, D)
    S_end = S * np.exp(g[:, -1])[..., None]                     # [N, H, D, D]
    gp = host(p)[slots]
    unit = np.sqrt(((gp - S_end) ** 2).sum(axis=(2, 3)) / (S_end ** 2).sum(axis=(2, 3)))
    eo = rel_l2(host(o), o_ref)
    print(f"[closed form] pooled tokens, beta = 0: worst state {unit.max():.2e}, o {eo:.2e}", flush=True)
    assert unit.max() <= 1e-5
    assert eo <= TOL["bf16"]


def test_decode_paths_are_deterministic():
    """Two runs of the decode step and of the pooled path on the same inputs
    and states give the same bits (no atomics, no order-dependent sums)."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x, S0 = _batch(54, "bf16")
    outs = []
    for _ in range(2):
        state = dev_f32(S0)
        o = kda.decode_step(state, dev_qkv(x.q), dev_qkv(x.k), dev_qkv(x.v), dev_f32(x.log_alpha),
                            dev_f32(x.beta))
        torch.cuda.synchronize()
        outs.append((o.cpu(), state.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    N, H, D, R = 64, 32, 128, 8
    y = gen.make_prefill(55, [R] * N, H=H, dk=D, dv=D, dtype="bf16")
    pool = gen.decode_state(55, N, H, D, D)
    slots = torch.from_numpy(np.random.default_rng(55).permutation(N).astype(np.int32)).cuda()
    outs = []
    for _ in range(2):
        p = dev_f32(pool)
        o = kda.decode_tokens(p, dev_qkv(y.q), dev_qkv(y.k), dev_qkv(y.v), dev_f32(y.log_alpha),
                              dev_f32(y.beta), state_indices=slots, num_seqs=N)
        torch.cuda.synchronize()
        outs.append((o.cpu(), p.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
