"""fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the GPU library and its Python
binding never do, and the two share no code.

The oracle is the plain token-by-token recurrence (Kimi Linear paper notes,
section 2, "KDA recurrence"), in IEEE double, on the exact input values the GPU
receives:

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t,          alpha_t = exp(log_alpha_t)  (per key channel)

It is implemented in plain C (``kda_oracle.c``) and called through ctypes.
Every function here is argument marshalling only.  Pins that tie the oracle to
the pages and to mathematics it does not itself use live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP; no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes handle on one build of the oracle library (the default build, or
    a deliberately altered copy that a test compiles to check the pins)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.oracle_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                       i32, vp, vp, i32]
        lib.oracle_prefill.restype = ctypes.c_int
        lib.oracle_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                          i32, i32, i32, vp, vp, vp, i32]
        lib.oracle_prefill_ex.restype = ctypes.c_int
        lib.oracle_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           vp, i32]
        lib.oracle_decode_step.restype = ctypes.c_int
        lib.oracle_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32,
                                        vp, vp, vp, vp, vp, vp, vp, vp, i32]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = [ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def prefill(self, *args, **kwargs):
        return _prefill(self.lib, *args, **kwargs)

    def decode_step(self, *args, **kwargs):
        return _decode_step(self.lib, *args, **kwargs)

    def decode_tokens(self, *args, **kwargs):
        return _decode_tokens(self.lib, *args, **kwargs)

    def backward(self, *args, **kwargs):
        return _backward(self.lib, *args, **kwargs)


_default: Optional[Oracle] = None


def _load():
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _default = Oracle(_LIB)
    return _default.lib


def compile_variant(source_text: str, out_path: str) -> Oracle:
    """Compile a (test-altered) copy of the oracle source and load it."""
    src = out_path[:-3] + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-o", out_path, src, "-lm"])
    return Oracle(out_path)


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def max_threads(nthreads: Optional[int] = None) -> int:
    return _load().oracle_max_threads(int(nthreads or default_threads()))


def _qkv_dtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError(f"q/k/v must be float32 or uint16 (bf16 bit patterns), got {x.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(*args, **kwargs) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token fp64 recurrence over a packed batch (see ``_prefill``)."""
    return _prefill(_load(), *args, **kwargs)


def decode_step(*args, **kwargs) -> np.ndarray:
    """One recurrent token for every (sequence, head) (see ``_decode_step``)."""
    return _decode_step(_load(), *args, **kwargs)


def decode_tokens(*args, **kwargs) -> np.ndarray:
    """Recurrent tokens of a packed batch on pooled states (see ``_decode_tokens``)."""
    return _decode_tokens(_load(), *args, **kwargs)


def backward(*args, **kwargs):
    """Gradients of the recurrence for given output gradients (see ``_backward``)."""
    return _backward(_load(), *args, **kwargs)


# option bits of oracle_prefill_ex
L2NORM_QK, BETA_LOGIT = 1, 2


def _prefill(lib, q: np.ndarray, k: np.ndarray, v: np.ndarray, log_alpha: np.ndarray,
             beta: np.ndarray, initial_state: Optional[np.ndarray] = None,
             cu_seqlens: Optional[np.ndarray] = None, num_seqs: Optional[int] = None,
             nthreads: Optional[int] = None, l2norm_qk: bool = False,
             beta_logit: bool = False, states_every: int = 0):
    """Token-by-token fp64 recurrence over a packed batch.

    q, k: [T, H, dk]; v: [T, H, dv] -- float32, or uint16 holding bf16 bits.
    log_alpha: [T, H, dk] float32; beta: [T, H] float32 (a logit if beta_logit).
    initial_state: [N, H, dk, dv] float32 or float64, or None (zeros).
    cu_seqlens: [N+1] int32 offsets, or None for N equal rows (num_seqs, default 1).
    l2norm_qk: L2-normalise q and k per (token, head) first (with 1e-6 added
    to the squared norm); beta_logit: beta = sigmoid(given value).
    Returns (o [T, H, dv] float64, final_state [N, H, dk, dv] float64), and
    with states_every = C > 0 also the state entering every C-th token of each
    sequence, [sum_s ceil(len_s / C), H, dk, dv] float64, in sequence order.
    """
    dtype = _qkv_dtype(q)
    assert k.dtype == q.dtype and v.dtype == q.dtype
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and v.shape == (T, H, dv)
    assert log_alpha.shape == (T, H, dk) and beta.shape == (T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = cu.shape[0] - 1
    else:
        cu = None
        N = int(num_seqs or 1)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    la = np.ascontiguousarray(log_alpha, dtype=np.float32)
    be = np.ascontiguousarray(beta, dtype=np.float32)
    s0 = s64 = None
    if initial_state is not None:
        if initial_state.dtype == np.float64:
            s64 = np.ascontiguousarray(initial_state)
        else:
            s0 = np.ascontiguousarray(initial_state, dtype=np.float32)
        assert initial_state.shape == (N, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    fin = np.zeros((N, H, dk, dv), dtype=np.float64)
    flags = (L2NORM_QK if l2norm_qk else 0) | (BETA_LOGIT if beta_logit else 0)
    if flags == 0 and states_every == 0 and s64 is None:
        rc = lib.oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
                                _ptr(cu), T, N, H, dk, dv, dtype, _ptr(o), _ptr(fin),
                                int(nthreads or default_threads()))
        if rc != 0:
            raise ValueError("oracle_prefill rejected its arguments")
        return o, fin
    snaps = None
    if states_every > 0:
        lens = np.diff(cu) if cu is not None else np.full(N, T // N)
        n_snap = int(sum((int(n) + states_every - 1) // states_every for n in lens))
        snaps = np.zeros((n_snap, H, dk, dv), dtype=np.float64)
    rc = lib.oracle_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
                               _ptr(s64), _ptr(cu), T, N, H, dk, dv, dtype, flags,
                               int(states_every), _ptr(snaps), _ptr(o), _ptr(fin),
                               int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_prefill_ex rejected its arguments")
    return (o, fin) if snaps is None else (o, fin, snaps)


def _decode_step(lib, state: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 log_alpha: np.ndarray, beta: np.ndarray,
                 nthreads: Optional[int] = None) -> np.ndarray:
    """One recurrent token for every (sequence, head); ``state`` (float64
    [N, H, dk, dv], C-contiguous) is updated in place.  Returns o [N, H, dv]."""
    assert state.dtype == np.float64 and state.flags.c_contiguous
    dtype = _qkv_dtype(q)
    N, H, dk, dv = state.shape
    assert q.shape == (N, H, dk) and k.shape == (N, H, dk) and v.shape == (N, H, dv)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    la = np.ascontiguousarray(log_alpha, dtype=np.float32)
    be = np.ascontiguousarray(beta, dtype=np.float32)
    assert la.shape == (N, H, dk) and be.shape == (N, H)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = lib.oracle_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                                _ptr(be), N, H, dk, dv, dtype, _ptr(o),
                                int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_decode_step rejected its arguments")
    return o


def _decode_tokens(lib, pool: np.ndarray, slots: Optional[np.ndarray], q: np.ndarray,
                   k: np.ndarray, v: np.ndarray, log_alpha: np.ndarray, beta: np.ndarray,
                   cu_seqlens: Optional[np.ndarray] = None, num_seqs: Optional[int] = None,
                   nthreads: Optional[int] = None, l2norm_qk: bool = False,
                   beta_logit: bool = False) -> np.ndarray:
    """Recurrent tokens of a packed batch, each sequence starting from and
    returning to its slot of a state pool (float64 [P, H, dk, dv], updated in
    place).  slots: [N] int32 slot per sequence (None = slot s for sequence s);
    a slot outside [0, P) marks a padding sequence: its output rows are zero
    and no state is read or written.  Returns o [T, H, dv] float64."""
    assert pool.dtype == np.float64 and pool.flags.c_contiguous
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = cu.shape[0] - 1
    else:
        N = int(num_seqs or 1)
        cu = np.arange(N + 1, dtype=np.int32) * (T // N)
    sl = np.arange(N, dtype=np.int64) if slots is None else np.asarray(slots, dtype=np.int64)
    assert sl.shape == (N,)
    o = np.zeros((T, H, dv), dtype=np.float64)
    for s in range(N):
        if not 0 <= sl[s] < pool.shape[0]:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        os_, fs = _prefill(lib, q[a:b], k[a:b], v[a:b], log_alpha[a:b], beta[a:b],
                           pool[sl[s]][None].copy(), None, 1, nthreads, l2norm_qk, beta_logit)
        o[a:b] = os_
        pool[sl[s]] = fs[0]
    return o


def _backward(lib, q: np.ndarray, k: np.ndarray, v: np.ndarray, log_alpha: np.ndarray,
              beta: np.ndarray, initial_state: Optional[np.ndarray], cu_seqlens: Optional[np.ndarray],
              d_o: np.ndarray, d_final: Optional[np.ndarray] = None,
              num_seqs: Optional[int] = None, nthreads: Optional[int] = None) -> dict:
    """Reverse-mode gradients of the token-by-token recurrence.

    Inputs as for ``prefill``; d_o [T, H, dv] and d_final [N, H, dk, dv] (or
    None) are the gradients of the loss with respect to o and the final state.
    Returns float64 arrays: dq, dk [T, H, dk]; dv [T, H, dv]; dlog_alpha
    [T, H, dk]; dbeta [T, H]; dinitial_state [N, H, dk, dv].
    """
    dtype = _qkv_dtype(q)
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = cu.shape[0] - 1
    else:
        cu = None
        N = int(num_seqs or 1)
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    la = np.ascontiguousarray(log_alpha, dtype=np.float32)
    be = np.ascontiguousarray(beta, dtype=np.float32)
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float32)
    do = np.ascontiguousarray(d_o, dtype=np.float64)
    df = None if d_final is None else np.ascontiguousarray(d_final, dtype=np.float64)
    assert do.shape == (T, H, dv)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dlog_alpha=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)),
               dinitial_state=np.zeros((N, H, dk, dv)))
    rc = lib.oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0), _ptr(cu),
                             T, N, H, dk, dv, dtype, _ptr(do), _ptr(df), _ptr(out["dq"]),
                             _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]),
                             _ptr(out["dbeta"]), _ptr(out["dinitial_state"]),
                             int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle_backward rejected its arguments")
    return out
