"""Properties of the GPU prefill that hold exactly or within tolerance at any
size: split/resume, decode = prefill, packing, head permutation, aliasing,
determinism, the linear-attention special case, exact recall and linearity."""
import dataclasses

import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import TOL, check_prefill, device_inputs, gpu_prefill, host, oracle_prefill, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_prefill_amd.kda as k
    k.lib()


def _raw(x, **kw):
    """GPU prefill returning device tensors (o, final)."""
    import torch
    o, fin = gpu_prefill(x, **kw)
    torch.cuda.synchronize()
    return o, fin


def _rows(x, a, b, state=None):
    """Tokens [a, b) of a single-sequence input, entering with `state`."""
    return dataclasses.replace(x, q=x.q[a:b].copy(), k=x.k[a:b].copy(), v=x.v[a:b].copy(),
                               log_alpha=x.log_alpha[a:b].copy(), beta=x.beta[a:b].copy(),
                               initial_state=state, cu_seqlens=None, num_seqs=1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_resume(dtype):
    """prefill(x[:a]) then prefill(x[a:], S_a) equals prefill(x); a is not a
    multiple of the chunk size, so the second call's chunk grid is shifted."""
    x = gen.make_prefill(41, [300], H=2, dk=128, dv=128, dtype=dtype, state_std=0.02)
    o_full, f_full = _raw(x)
    ro, rf = oracle_prefill(x)
    for a in (1, 137, 299):
        o1, f1 = _raw(_rows(x, 0, a, x.initial_state))
        o2, f2 = _raw(_rows(x, a, 300, host(f1).astype(np.float32)))
        o_cat = np.concatenate([host(o1), host(o2)])
        eo, ef = rel_l2(o_cat, ro), rel_l2(host(f2), rf)
        print(f"[split] {dtype} a={a}: o={eo:.3e} state={ef:.3e}", flush=True)
        assert eo <= TOL[dtype] and ef <= TOL[dtype]
        assert rel_l2(o_cat, host(o_full)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_equals_prefill(dtype):
    """T recurrent decode steps give the prefill's outputs and final state."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    T = 70
    x = gen.make_prefill(42, [T], H=2, dk=128, dv=64, dtype=dtype, state_std=0.02)
    o_p, f_p = _raw(x)
    d = device_inputs(x)
    state = d["initial_state"].clone()
    outs = []
    for t in range(T):
        # slices are copied: one token's beta row is 8 bytes, and every pointer
        # passed to the library must be 16-byte aligned
        tok = [d[n][t:t + 1].clone() for n in ("q", "k", "v", "log_alpha", "beta")]
        outs.append(kda.decode_step(state, *tok))
    torch.cuda.synchronize()
    o_d = np.concatenate([host(o) for o in outs])
    ro, rf = oracle_prefill(x)
    assert rel_l2(o_d, ro) <= TOL[dtype] and rel_l2(host(state), rf) <= TOL[dtype]
    assert rel_l2(o_d, host(o_p)) <= TOL[dtype]
    assert rel_l2(host(state), host(f_p)) <= TOL[dtype]


def test_packing_is_exact():
    """Chunks never span sequences, so a packed batch gives bit-for-bit the
    results of one call per sequence."""
    import torch
    lens = [65, 1, 200, 64, 0, 129]
    x = gen.make_prefill(43, lens, H=3, dk=128, dv=128, dtype="bf16", state_std=0.02,
                         packed=True)
    o, fin = _raw(x)
    o, fin = o.cpu(), fin.cpu()
    offs = np.concatenate([[0], np.cumsum(lens)])
    for s, n in enumerate(lens):
        y = x.select_seqs([s])
        oy, fy = _raw(y)
        assert torch.equal(oy.cpu(), o[offs[s]:offs[s + 1]]), s
        assert torch.equal(fy.cpu()[0], fin[s]), s


def test_head_permutation_is_exact():
    import torch
    x = gen.make_prefill(44, [150, 77], H=5, dk=64, dv=128, dtype="bf16", state_std=0.02)
    perm = [3, 0, 4, 1, 2]
    o, fin = _raw(x)
    op, fp = _raw(x.select_heads(perm))
    assert torch.equal(op.cpu(), o.cpu()[:, perm])
    assert torch.equal(fp.cpu(), fin.cpu()[:, perm])


def test_deterministic_and_workspace_forms():
    """Two runs, with the internal workspace and with a caller workspace, are
    bit-for-bit identical."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x = gen.make_prefill(45, [500, 3, 260], H=4, dk=128, dv=128, dtype="bf16", state_std=0.02)
    o1, f1 = _raw(x)
    o2, f2 = _raw(x)
    ws = torch.empty(kda.workspace_bytes(x.T, x.num_seqs, x.H, x.dk, x.dv, True),
                     dtype=torch.uint8, device="cuda")
    o3, f3 = _raw(x, workspace=ws)
    for a, b in ((o1, o2), (f1, f2), (o1, o3), (f1, f3)):
        assert torch.equal(a.cpu(), b.cpu())


def test_final_state_may_alias_initial_state():
    import torch
    import gated_delta_rule_prefill_amd as kda
    x = gen.make_prefill(46, [190, 64, 5], H=3, dk=128, dv=128, dtype="bf16", state_std=0.02)
    o1, f1 = _raw(x)
    d = device_inputs(x)
    s = d["initial_state"].clone()
    o2, f2 = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s, d["cu_seqlens"],
                         final_state=s)
    torch.cuda.synchronize()
    assert f2.data_ptr() == s.data_ptr()
    assert torch.equal(o1.cpu(), o2.cpu()) and torch.equal(f1.cpu(), s.cpu())


def test_no_write_linear_attention_fp32():
    """alpha = 1, beta = 0: the state never changes and o_t = S0^T q_t."""
    x = gen.make_prefill(47, [150, 70], H=2, dk=128, dv=64, dtype="f32", state_std=0.5)
    x = dataclasses.replace(x, log_alpha=np.zeros_like(x.log_alpha),
                            beta=np.zeros_like(x.beta))
    o, fin = _raw(x)
    assert np.array_equal(host(fin), x.initial_state.astype(np.float64))
    lens = x.lengths()
    offs = np.concatenate([[0], np.cumsum(lens)])
    S0 = x.initial_state.astype(np.float64)
    ref = np.concatenate([np.einsum("thk,hkv->thv", x.q[offs[s]:offs[s + 1]].astype(np.float64),
                                    S0[s]) for s in range(len(lens))])
    assert rel_l2(host(o), ref) <= 1e-6


def test_exact_recall_fp32():
    """beta = 1 and unit keys: the state recalls each value, S_t^T k_t = v_t,
    so with q = k every output equals its token's value."""
    x = gen.make_prefill(48, [200], H=2, dk=128, dv=128, dtype="f32", state_std=0.02)
    x = dataclasses.replace(x, q=x.k.copy(), beta=np.ones_like(x.beta))
    o, _ = _raw(x)
    assert rel_l2(host(o), x.v.astype(np.float64)) <= 1e-4


def test_linear_in_state_and_values_fp32():
    """For fixed q, k, alpha, beta the map (S0, V) -> (o, S_T) is linear."""
    x = gen.make_prefill(49, [180, 33], H=2, dk=64, dv=64, dtype="f32", state_std=0.02)
    y = gen.make_prefill(50, [180, 33], H=2, dk=64, dv=64, dtype="f32", state_std=0.02)
    a, b = 0.75, -1.5
    z = dataclasses.replace(x, v=(a * x.v + b * y.v).astype(np.float32),
                            initial_state=(a * x.initial_state + b * y.initial_state).astype(np.float32))
    y = dataclasses.replace(x, v=y.v, initial_state=y.initial_state)
    ox, fx = (host(t) for t in _raw(x))
    oy, fy = (host(t) for t in _raw(y))
    oz, fz = (host(t) for t in _raw(z))
    assert rel_l2(oz, a * ox + b * oy) <= 1e-5
    assert rel_l2(fz, a * fx + b * fy) <= 1e-5


def test_bf16_max_head_count_small_T():
    """Many heads with few tokens (grid wider than one XCD round)."""
    x = gen.make_prefill(51, [70, 9], H=67, dk=128, dv=128, dtype="bf16", state_std=0.02)
    check_prefill(x, label="67 heads")
