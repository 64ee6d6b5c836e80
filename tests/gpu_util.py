"""Helpers for the GPU parity tests: move seeded inputs to the device, run
libkda through its binding, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
from gated_delta_rule_prefill_amd import inputs as gen

# Tolerances on relative L2 error (whole tensor, fp64): fp32 inputs, bf16 inputs.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def dev_qkv(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def dev_f32(a, device="cuda"):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return gen.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def device_inputs(x: "gen.KDAInputs", device="cuda"):
    import torch
    d = dict(q=dev_qkv(x.q, device), k=dev_qkv(x.k, device), v=dev_qkv(x.v, device),
             log_alpha=dev_f32(x.log_alpha, device), beta=dev_f32(x.beta, device),
             initial_state=dev_f32(x.initial_state, device), cu_seqlens=None,
             num_seqs=x.num_seqs)
    if x.cu_seqlens is not None:
        d["cu_seqlens"] = torch.from_numpy(np.ascontiguousarray(x.cu_seqlens, dtype=np.int32)).to(device)
    return d


def gpu_prefill(x: "gen.KDAInputs", device="cuda", **kw):
    import gated_delta_rule_prefill_amd as kda
    d = device_inputs(x, device)
    o, fin = kda.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["initial_state"],
                         d["cu_seqlens"], num_seqs=d["num_seqs"], **kw)
    return o, fin


def oracle_prefill(x: "gen.KDAInputs"):
    return oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state, x.cu_seqlens,
                          num_seqs=x.num_seqs)


def check_prefill(x: "gen.KDAInputs", tol=None, label=""):
    """Run GPU and oracle on the same inputs; return (err_o, err_state)."""
    import torch
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    ro, rf = oracle_prefill(x)
    eo, ef = rel_l2(host(o), ro), rel_l2(host(fin), rf)
    tol = tol if tol is not None else TOL[x.dtype]
    print(f"[parity] {label} T={x.T} H={x.H} dk={x.dk} dv={x.dv} {x.dtype}: "
          f"rel_l2 o={eo:.3e} state={ef:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and ef <= tol, (label, eo, ef, tol)
    return eo, ef
