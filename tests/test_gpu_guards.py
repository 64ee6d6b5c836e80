"""Guard bytes around every output and workspace (out-of-bounds writes).

Each buffer the library writes -- o, final states, chunk states, state pools,
gradients and the caller's workspace -- is the middle of a larger device
allocation whose 4 KiB before and after are filled with a byte pattern.  After
the call the pattern must be intact: a kernel that writes past the end (or
before the start) of any output, at ragged lengths, empty sequences, padding
slots or segment boundaries, fails here even where the values it leaves in
bounds are right.  In-place buffers (decode states, pools) get the same
guards."""
import numpy as np
import pytest

from gated_delta_rule_prefill_amd import inputs as gen
from gpu_util import device_inputs, dev_f32, dev_qkv

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Guarded:
    """A device tensor of `shape` and `dtype` with guard bytes on both sides."""

    def __init__(self, shape, dtype, init=None):
        import torch
        self.n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + self.n].view(dtype).view(*shape)
        if init is not None:
            self.t.copy_(init)

    def intact(self) -> bool:
        h = self.buf.cpu().numpy()
        return bool((h[:GUARD] == PATTERN).all() and (h[GUARD + self.n:] == PATTERN).all())


def _check(bufs, label):
    import torch
    torch.cuda.synchronize()
    bad = [name for name, g in bufs.items() if not g.intact()]
    print(f"[guards] {label}: {len(bufs)} buffers, intact={not bad}", flush=True)
    assert not bad, f"{label}: writes outside {bad}"


PAIRINGS = [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 128, 64), ("f32", 128, 128),
            ("f32", 64, 64)]


@pytest.mark.parametrize("dtype,dk,dv", PAIRINGS)
def test_prefill_writes_stay_in_bounds(dtype, dk, dv):
    """Packed lengths with an empty sequence, one token, chunk edges and a
    ragged tail; o, final state, chunk states and workspace guarded."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    x = gen.make_prefill(301, [0, 1, 63, 64, 65, 130, 7], H=3, dk=dk, dv=dv, dtype=dtype,
                         state_std=0.02, packed=True)
    d = device_inputs(x)
    T, H, N = x.T, x.H, x.num_seqs
    nc = kda.num_chunk_states(T, N, d["cu_seqlens"])
    tdt = d["q"].dtype
    g = dict(o=Guarded((T, H, dv), tdt), fin=Guarded((N, H, dk, dv), torch.float32),
             cs=Guarded((nc, H, dk, dv), torch.float32),
             ws=Guarded((kda.workspace_bytes(T, N, H, dk, dv, dtype == "bf16"),), torch.uint8))
    kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                d["cu_seqlens"], out=g["o"].t, final_state=g["fin"].t, chunk_states=g["cs"].t,
                workspace=g["ws"].t)
    _check(g, f"prefill {dtype} {dk}x{dv}")
    assert torch.isfinite(g["o"].t.float()).all() and torch.isfinite(g["fin"].t).all()


def test_segmented_prefill_writes_stay_in_bounds():
    """Two sequences of 4,160 tokens at H = 32 (65 chunks each), which run in
    two segments; without a final state the state between segments lives in
    the workspace's carry area, which the guards bound too."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    N, rows, H, D = 2, 4160, 32, 128
    x = gen.make_prefill(302, [rows] * N, H=H, dk=D, dv=D, dtype="bf16", state_std=0.02)
    d = device_inputs(x)
    T = N * rows
    for with_final in (False, True):
        g = dict(o=Guarded((T, H, D), torch.bfloat16),
                 ws=Guarded((kda.workspace_bytes(T, N, H, D, D, True),), torch.uint8))
        kw = dict(output_final_state=False)
        if with_final:
            g["fin"] = Guarded((N, H, D, D), torch.float32)
            kw = dict(final_state=g["fin"].t)
        kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                    num_seqs=N, out=g["o"].t, workspace=g["ws"].t, **kw)
        _check(g, f"segmented prefill, final state {with_final}")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64), ("bf16", 64, 128)])
def test_decode_step_writes_stay_in_bounds(dtype, dk, dv):
    import torch
    import gated_delta_rule_prefill_amd as kda
    N, H = 5, 3
    t = gen.decode_token(303, 0, N, H, dk, dv, dtype=dtype)
    g = dict(state=Guarded((N, H, dk, dv), torch.float32,
                           init=dev_f32(gen.decode_state(303, N, H, dk, dv))),
             o=Guarded((N, H, dv), torch.bfloat16 if dtype == "bf16" else torch.float32))
    kda.decode_step(g["state"].t, dev_qkv(t.q), dev_qkv(t.k), dev_qkv(t.v), dev_f32(t.log_alpha),
                    dev_f32(t.beta), out=g["o"].t)
    _check(g, f"decode step {dtype} {dk}x{dv}")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 64)])
@pytest.mark.parametrize("case", ["packed", "one_token"])
def test_decode_tokens_writes_stay_in_bounds(dtype, dk, dv, case):
    """Pooled states with padding slots (-1 and one past the pool): packed
    lengths 0..70, and one token per sequence as equal rows."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    P, H = 6, 2
    if case == "packed":
        lens, slots = [5, 0, 17, 70, 1], [3, 0, -1, 5, 6]
        x = gen.make_prefill(304, lens, H=H, dk=dk, dv=dv, dtype=dtype, packed=True)
    else:
        lens, slots = [1] * 5, [2, -1, 0, 6, 4]
        x = gen.make_prefill(305, lens, H=H, dk=dk, dv=dv, dtype=dtype, packed=False)
    d = device_inputs(x)
    pool0 = (0.02 * np.random.default_rng(306).standard_normal((P, H, dk, dv))).astype(np.float32)
    g = dict(pool=Guarded((P, H, dk, dv), torch.float32, init=dev_f32(pool0)),
             o=Guarded((x.T, H, dv), d["q"].dtype))
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    kda.decode_tokens(g["pool"].t, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                      state_indices=sl, cu_seqlens=d["cu_seqlens"], num_seqs=len(lens),
                      out=g["o"].t)
    _check(g, f"decode tokens {case} {dtype} {dk}x{dv}")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 64)])
def test_backward_writes_stay_in_bounds(dtype, dk, dv):
    """Every gradient output and the workspace guarded (chunkwise path for
    bf16 at d = 128, the token walk for fp32), through the C ABI."""
    import torch
    import gated_delta_rule_prefill_amd as kda
    from gated_delta_rule_prefill_amd import kda as b
    x = gen.make_prefill(307, [0, 65, 1, 130], H=2, dk=dk, dv=dv, dtype=dtype, state_std=0.02,
                         packed=True)
    d = device_inputs(x)
    T, H, N = x.T, x.H, x.num_seqs
    tdt = d["q"].dtype
    d_o = dev_qkv(gen.make_prefill(308, [T], H=H, dk=dk, dv=dv, dtype=dtype).v)
    d_fin = dev_f32(0.1 * gen.decode_state(309, N, H, dk, dv))
    g = dict(dq=Guarded((T, H, dk), tdt), dk=Guarded((T, H, dk), tdt), dv=Guarded((T, H, dv), tdt),
             dla=Guarded((T, H, dk), torch.float32), dbeta=Guarded((T, H), torch.float32),
             dinit=Guarded((N, H, dk, dv), torch.float32),
             ws=Guarded((kda.backward_workspace_bytes(T, N, H, dk, dv, dtype == "bf16"),),
                        torch.uint8))
    st = b.lib().kda_backward(
        b._ptr(d["q"]), b._ptr(d["k"]), b._ptr(d["v"]), b._ptr(d["log_alpha"]), b._ptr(d["beta"]),
        b._ptr(d["initial_state"]), b._ptr(d["cu_seqlens"]), T, N, H, dk, dv, b._dtype_code(d["q"]),
        b._ptr(d_o), b._ptr(d_fin), None, b._ptr(g["dq"].t), b._ptr(g["dk"].t), b._ptr(g["dv"].t),
        b._ptr(g["dla"].t), b._ptr(g["dbeta"].t), b._ptr(g["dinit"].t), b._ptr(g["ws"].t), g["ws"].n,
        b._stream(d["q"].device, None))
    assert st == b.KDA_OK, b.last_error()
    _check(g, f"backward {dtype} {dk}x{dv}")


def test_noalloc_writes_stay_in_bounds():
    import torch
    from gated_delta_rule_prefill_amd import kda as b
    x = gen.make_prefill(310, [300, 0, 65], H=4, dk=128, dv=128, dtype="bf16", state_std=0.02,
                         packed=True)
    d = device_inputs(x)
    g = dict(o=Guarded((x.T, x.H, x.dv), torch.bfloat16),
             fin=Guarded((x.num_seqs, x.H, x.dk, x.dv), torch.float32))
    st = b.lib().kda_prefill_noalloc(
        b._ptr(d["q"]), b._ptr(d["k"]), b._ptr(d["v"]), b._ptr(d["log_alpha"]), b._ptr(d["beta"]),
        b._ptr(d["initial_state"]), b._ptr(d["cu_seqlens"]), x.T, x.num_seqs, x.H, x.dk, x.dv,
        b.KDA_DTYPE_BF16, b._ptr(g["o"].t), b._ptr(g["fin"].t), b._stream(d["q"].device, None))
    assert st == b.KDA_OK, b.last_error()
    _check(g, "noalloc prefill")
