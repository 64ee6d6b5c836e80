"""Helpers for the GPU parity tests: move seeded inputs to the device, run
libkda through its binding, and compare with the fp64 oracle.

Every prefill comparison is gated at several granularities, so that a fault
confined to one place cannot hide in a pooled error:
  * the whole o and final-state tensors (relative L2, the stated tolerance);
  * every (sequence, head): its o rows and its final state;
  * every 64-token chunk of every (sequence, head): its o rows;
  * every single o row (token, head), at a looser bound (ROW_TOL) since one
    row has only dv elements: its error against the larger of its own norm
    and the RMS row norm of its (sequence, head), so that a row whose exact
    value nearly vanishes (the first token of a zero-state sequence is
    beta (q . k) v, and q . k of two random unit vectors can be close to 0)
    is not held to a relative bound on a near-zero number.
A sequence or chunk of fewer than MIN_UNIT_ROWS tokens is a few rows, not a
tensor: its o is held to the row bound, its final state to the tolerance.
(On the bf16 path the decayed q and k operands are rounded to bf16, so one
entry q_r . k_i of a small dot product carries a relative error of a few
percent; a one-token sequence's output is that one entry times v plus the
read-out of its entering state, and shows it undiluted.)
"""
from __future__ import annotations

import numpy as np

import oracle
from gated_delta_rule_prefill_amd import inputs as gen

# Tolerances on relative L2 error (fp64): fp32 inputs, bf16 inputs.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# One output row (dv elements) against its own norm.  A wholly wrong row gives
# an error of order 1; bf16 rounding of the row alone gives about 2e-3.
ROW_TOL = {"f32": 1e-3, "bf16": 1e-1}
MIN_UNIT_ROWS = 8
CHUNK = 64


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def _rel_rows(err_sq: np.ndarray, ref_sq: np.ndarray) -> np.ndarray:
    """Relative L2 from summed squares; an all-zero reference gives the absolute error."""
    den = np.sqrt(ref_sq)
    num = np.sqrt(err_sq)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def unit_errors(o, ro, fin, rf, lengths):
    """Errors of a packed prefill at every granularity (see the module docstring).

    o, ro: [T, H, dv]; fin, rf: [N, H, dk, dv] (fp64).  Returns a dict with
    the whole-tensor errors and the worst (sequence, head), chunk and row."""
    o = np.asarray(o, dtype=np.float64)
    ro = np.asarray(ro, dtype=np.float64)
    T, H, _ = ro.shape
    e2 = ((o - ro) ** 2).sum(axis=2)        # [T, H]
    r2 = (ro ** 2).sum(axis=2)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    scale2 = r2.copy()                      # max(own, unit-mean) squared row norm
    for s, n in enumerate(lengths):
        a = int(offs[s])
        if n:
            scale2[a:a + n] = np.maximum(r2[a:a + n], r2[a:a + n].mean(axis=0, keepdims=True))
    row = _rel_rows(e2, scale2)
    seq_o, chunk_o = [], []      # units of at least MIN_UNIT_ROWS rows
    for s, n in enumerate(lengths):
        a = int(offs[s])
        if n < MIN_UNIT_ROWS:
            continue
        seq_o.append(_rel_rows(e2[a:a + n].sum(0), r2[a:a + n].sum(0)))   # [H]
        for c0 in range(0, n, CHUNK):
            b = a + min(n, c0 + CHUNK)
            if b - (a + c0) >= MIN_UNIT_ROWS:
                chunk_o.append(_rel_rows(e2[a + c0:b].sum(0), r2[a + c0:b].sum(0)))
    fin = np.asarray(fin, dtype=np.float64)
    rf = np.asarray(rf, dtype=np.float64)
    seq_s = _rel_rows(((fin - rf) ** 2).sum(axis=(2, 3)), (rf ** 2).sum(axis=(2, 3)))  # [N, H]
    worst_row = np.unravel_index(int(np.argmax(row)), row.shape) if T else (0, 0)
    return {
        "o": rel_l2(o, ro), "state": rel_l2(fin, rf),
        "seq_head_o": float(np.max(seq_o)) if seq_o else 0.0,
        "seq_head_state": float(np.max(seq_s)) if seq_s.size else 0.0,
        "chunk_o": float(np.max(chunk_o)) if chunk_o else 0.0,
        "row_o": float(row[worst_row]) if T else 0.0,
        "worst_row": tuple(int(i) for i in worst_row),
    }


def assert_units(errs: dict, dtype: str, label: str = "", tol=None, row_tol=None) -> None:
    tol = TOL[dtype] if tol is None else tol
    row_tol = ROW_TOL[dtype] if row_tol is None else row_tol
    print(f"[parity] {label} ({dtype}): rel_l2 o={errs['o']:.3e} state={errs['state']:.3e}; "
          f"worst (seq,head) o={errs['seq_head_o']:.3e} state={errs['seq_head_state']:.3e}; "
          f"worst chunk o={errs['chunk_o']:.3e}; worst row o={errs['row_o']:.3e} at "
          f"(token, head) {errs['worst_row']} (tol {tol:g}, row tol {row_tol:g})", flush=True)
    for key in ("o", "state", "seq_head_o", "seq_head_state", "chunk_o"):
        assert errs[key] <= tol, (label, key, errs[key], tol)
    assert errs["row_o"] <= row_tol, (label, "row_o", errs["row_o"], errs["worst_row"], row_tol)


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
    """Run GPU and oracle on the same inputs and gate every granularity;
    return (err_o, err_state) over the whole tensors."""
    import torch
    o, fin = gpu_prefill(x)
    torch.cuda.synchronize()
    ro, rf = oracle_prefill(x)
    errs = unit_errors(host(o), ro, host(fin), rf, x.lengths())
    assert_units(errs, x.dtype, f"{label} T={x.T} H={x.H} dk={x.dk} dv={x.dv}", tol=tol)
    return errs["o"], errs["state"]
