"""Python binding of libkda (ctypes).  Argument marshalling only: every step
of the computation runs in the HIP kernels behind the C ABI of
``include/kda.h``.  PyTorch provides device memory and the stream.

There is no fallback: if libkda.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_DTYPE_F32, KDA_DTYPE_BF16 = 0, 1
KDA_FLAG_L2NORM_QK, KDA_FLAG_BETA_SIGMOID = 1, 2
CHUNK = 64  # tokens per chunk of the chunkwise prefill (rows of chunk_states)

# name -> (restype, argtypes) for every entry point of include/kda.h
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "kda_prefill_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, ctypes.c_int]),
    "kda_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                   _i32, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "kda_prefill_ex": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                      _i32, _i32, ctypes.c_int, ctypes.c_uint32, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "kda_prefill_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                           _i32, _i32, ctypes.c_int, _vp, _vp, _vp]),
    "kda_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                       ctypes.c_int, _vp, _vp]),
    "kda_decode_tokens": (ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                         _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_uint32,
                                         _vp, _vp]),
    "kda_backward_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, ctypes.c_int]),
    "kda_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                    _i32, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _sz, _vp]),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error_message": (ctypes.c_char_p, []),
    "kda_version": (_i32, []),
    "kda_set_kernel_timing": (ctypes.c_int, [_i32]),
    "kda_prefill_kernel_times": (_i32, [ctypes.POINTER(ctypes.c_float),
                                        ctypes.POINTER(ctypes.c_char_p), _i32]),
}


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)} ({detail})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by ``gated_delta_rule_prefill_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m gated_delta_rule_prefill_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def last_error() -> str:
    return lib().kda_last_error_message().decode()


def _check(status: int, where: str) -> None:
    if status != KDA_OK:
        raise KDAError(status, where, last_error())


def workspace_bytes(total_tokens: int, num_seqs: int, H: int, dk: int, dv: int,
                    bf16: bool) -> int:
    return int(lib().kda_prefill_workspace_bytes(int(total_tokens), int(num_seqs), int(H),
                                                 int(dk), int(dv),
                                                 KDA_DTYPE_BF16 if bf16 else KDA_DTYPE_F32))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _flags(l2norm_qk: bool, beta_sigmoid: bool) -> int:
    return (KDA_FLAG_L2NORM_QK if l2norm_qk else 0) | (KDA_FLAG_BETA_SIGMOID if beta_sigmoid else 0)


def num_chunk_states(T: int, N: int, cu_seqlens=None) -> int:
    """Rows of ``chunk_states``: sum over sequences of ceil(len / 64)."""
    if cu_seqlens is None:
        return N * ((T // N + CHUNK - 1) // CHUNK)
    cu = [int(x) for x in cu_seqlens.tolist()]
    return sum((b - a + CHUNK - 1) // CHUNK for a, b in zip(cu[:-1], cu[1:]))


def prefill(q, k, v, log_alpha, beta, initial_state=None, cu_seqlens=None,
            num_seqs: Optional[int] = None, output_final_state: bool = True,
            final_state=None, out=None, workspace=None, stream=None,
            l2norm_qk: bool = False, beta_sigmoid: bool = False, chunk_states=None):
    """Chunkwise KDA prefill of a packed batch (``kda_prefill_ex``).

    q, k: [T, H, dk]; v: [T, H, dv] (bf16 or fp32, same dtype, CUDA/HIP device);
    log_alpha: [T, H, dk] fp32; beta: [T, H] fp32 (logits with beta_sigmoid);
    initial_state: [N, H, dk, dv] fp32 or None; cu_seqlens: [N+1] int32 or None
    (then ``num_seqs`` equal rows, default 1).  ``final_state`` may be the
    same tensor as ``initial_state``.  l2norm_qk / beta_sigmoid: in-kernel
    preprocessing (KDA_FLAG_*).  chunk_states: None, True (allocate) or an fp32
    [NC, H, dk, dv] tensor for the state entering every 64-token chunk.
    Returns (o [T, H, dv], final_state or None), plus chunk_states if asked.
    """
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1, "cu_seqlens: int32 [N+1]")
        N = cu_seqlens.shape[0] - 1
    else:
        N = int(num_seqs or 1)
    dev = q.device
    for name, t, shape, dt in (("k", k, (T, H, dk), q.dtype), ("v", v, (T, H, dv), q.dtype),
                               ("log_alpha", log_alpha, (T, H, dk), torch.float32),
                               ("beta", beta, (T, H), torch.float32)):
        _require(tuple(t.shape) == shape, f"{name}: expected shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt, f"{name}: expected dtype {dt}, got {t.dtype}")
    tensors = [q, k, v, log_alpha, beta]
    if initial_state is not None:
        _require(tuple(initial_state.shape) == (N, H, dk, dv) and
                 initial_state.dtype == torch.float32, "initial_state: fp32 [N, H, dk, dv]")
        tensors.append(initial_state)
    if cu_seqlens is not None:
        tensors.append(cu_seqlens)
    for t in tensors:
        _require(t.device == dev and t.is_contiguous(), "all inputs: contiguous, on one device")
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    want_cs = chunk_states is not None and chunk_states is not False
    if chunk_states is True:
        nc = num_chunk_states(T, N, cu_seqlens)
        chunk_states = torch.empty((nc, H, dk, dv), dtype=torch.float32, device=dev)
    elif want_cs:
        nc = num_chunk_states(T, N, cu_seqlens)
        _require(chunk_states.dtype == torch.float32 and chunk_states.is_contiguous() and
                 chunk_states.device == dev and chunk_states.numel() >= nc * H * dk * dv,
                 "chunk_states: contiguous fp32 with room for [NC, H, dk, dv]")
    else:
        chunk_states = None
    need = workspace_bytes(T, N, H, dk, dv, q.dtype == torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _require(workspace.numel() * workspace.element_size() >= need, "workspace too small")
    st = lib().kda_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                              _ptr(initial_state), _ptr(cu_seqlens), T, N, H, dk, dv,
                              _dtype_code(q), _flags(l2norm_qk, beta_sigmoid), _ptr(out),
                              _ptr(final_state), _ptr(chunk_states), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(st, "kda_prefill_ex")
    return (out, final_state, chunk_states) if want_cs else (out, final_state)


def decode_step(state, q, k, v, log_alpha, beta, out=None, stream=None):
    """One recurrent KDA token per sequence (``kda_decode_step``); ``state``
    (fp32 [N, H, dk, dv]) is updated in place.  Returns o [N, H, dv]."""
    import torch
    N, H, dk, dv = state.shape
    _require(state.dtype == torch.float32 and state.is_contiguous(), "state: contiguous fp32")
    for name, t, shape, dt in (("q", q, (N, H, dk), q.dtype), ("k", k, (N, H, dk), q.dtype),
                               ("v", v, (N, H, dv), q.dtype),
                               ("log_alpha", log_alpha, (N, H, dk), torch.float32),
                               ("beta", beta, (N, H), torch.float32)):
        _require(tuple(t.shape) == shape, f"{name}: expected shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt, f"{name}: expected dtype {dt}")
        _require(t.device == state.device and t.is_contiguous(), f"{name}: contiguous, same device")
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=state.device)
    st = lib().kda_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                               _ptr(beta), N, H, dk, dv, _dtype_code(q), _ptr(out),
                               _stream(state.device, stream))
    _check(st, "kda_decode_step")
    return out


def decode_tokens(state_pool, q, k, v, log_alpha, beta, state_indices=None, cu_seqlens=None,
                  num_seqs: Optional[int] = None, l2norm_qk: bool = False,
                  beta_sigmoid: bool = False, out=None, stream=None):
    """Recurrent KDA over the tokens of a packed batch on pooled states
    (``kda_decode_tokens``).  state_pool: fp32 [P, H, dk, dv], updated in
    place; state_indices: int32 [N] slot per sequence (None = slot s for
    sequence s; a slot outside [0, P) marks padding); tokens as for
    ``prefill``.  Returns o [T, H, dv]."""
    import torch
    P, H, dk, dv = state_pool.shape
    T = q.shape[0]
    dev = state_pool.device
    _require(state_pool.dtype == torch.float32 and state_pool.is_contiguous(),
             "state_pool: contiguous fp32")
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1, "cu_seqlens: int32 [N+1]")
        N = cu_seqlens.shape[0] - 1
    else:
        N = int(num_seqs or 1)
    for name, t, shape, dt in (("q", q, (T, H, dk), q.dtype), ("k", k, (T, H, dk), q.dtype),
                               ("v", v, (T, H, dv), q.dtype),
                               ("log_alpha", log_alpha, (T, H, dk), torch.float32),
                               ("beta", beta, (T, H), torch.float32)):
        _require(tuple(t.shape) == shape, f"{name}: expected shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt, f"{name}: expected dtype {dt}")
        _require(t.device == dev and t.is_contiguous(), f"{name}: contiguous, same device")
    if state_indices is not None:
        _require(state_indices.dtype == torch.int32 and tuple(state_indices.shape) == (N,) and
                 state_indices.device == dev and state_indices.is_contiguous(),
                 "state_indices: int32 [N] on the same device")
    if cu_seqlens is not None:
        _require(cu_seqlens.device == dev and cu_seqlens.is_contiguous(), "cu_seqlens: same device")
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    st = lib().kda_decode_tokens(_ptr(state_pool), P, _ptr(state_indices), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), T, N,
                                 H, dk, dv, _dtype_code(q), _flags(l2norm_qk, beta_sigmoid),
                                 _ptr(out), _stream(dev, stream))
    _check(st, "kda_decode_tokens")
    return out


def backward_workspace_bytes(total_tokens: int, num_seqs: int, H: int, dk: int, dv: int,
                             bf16: bool) -> int:
    return int(lib().kda_backward_workspace_bytes(int(total_tokens), int(num_seqs), int(H),
                                                  int(dk), int(dv),
                                                  KDA_DTYPE_BF16 if bf16 else KDA_DTYPE_F32))


def backward(q, k, v, log_alpha, beta, d_o, initial_state=None, cu_seqlens=None,
             num_seqs: Optional[int] = None, d_final_state=None, chunk_states=None,
             need_initial_state_grad: bool = True, workspace=None, stream=None) -> dict:
    """Gradients of ``prefill`` (``kda_backward``): for dL/do = d_o and
    dL/dfinal_state = d_final_state (or zero) returns dq, dk, dv (q/k/v dtype),
    dlog_alpha, dbeta and dinitial_state (fp32).  chunk_states: the forward's
    exported chunk states, or None to recompute them."""
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1, "cu_seqlens: int32 [N+1]")
        N = cu_seqlens.shape[0] - 1
    else:
        N = int(num_seqs or 1)
    dev = q.device
    for name, t, shape, dt in (("k", k, (T, H, dk), q.dtype), ("v", v, (T, H, dv), q.dtype),
                               ("log_alpha", log_alpha, (T, H, dk), torch.float32),
                               ("beta", beta, (T, H), torch.float32),
                               ("d_o", d_o, (T, H, dv), q.dtype)):
        _require(tuple(t.shape) == shape, f"{name}: expected shape {shape}, got {tuple(t.shape)}")
        _require(t.dtype == dt, f"{name}: expected dtype {dt}, got {t.dtype}")
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _require(tuple(t.shape) == (N, H, dk, dv) and t.dtype == torch.float32,
                     f"{name}: fp32 [N, H, dk, dv]")
    if chunk_states is not None:
        _require(chunk_states.dtype == torch.float32 and
                 chunk_states.numel() >= num_chunk_states(T, N, cu_seqlens) * H * dk * dv,
                 "chunk_states: fp32 [NC, H, dk, dv]")
    for t in (q, k, v, log_alpha, beta, d_o, initial_state, cu_seqlens, d_final_state, chunk_states):
        if t is not None:
            _require(t.device == dev and t.is_contiguous(), "all inputs: contiguous, on one device")
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dlog_alpha=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta),
               dinitial_state=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
               if need_initial_state_grad else None)
    need = backward_workspace_bytes(T, N, H, dk, dv, q.dtype == torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _require(workspace.numel() * workspace.element_size() >= need, "workspace too small")
    st = lib().kda_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                            _ptr(initial_state), _ptr(cu_seqlens), T, N, H, dk, dv,
                            _dtype_code(q), _ptr(d_o), _ptr(d_final_state), _ptr(chunk_states),
                            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]),
                            _ptr(out["dinitial_state"]), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(dev, stream))
    _check(st, "kda_backward")
    return out


def set_kernel_timing(enabled: bool) -> None:
    _check(lib().kda_set_kernel_timing(1 if enabled else 0), "kda_set_kernel_timing")


def prefill_kernel_times():
    """[(kernel name, ms)] of the last prefill recorded with timing enabled on
    this thread, in launch order (a long batch runs its kernels once per segment)."""
    ms = (ctypes.c_float * 256)()
    names = (ctypes.c_char_p * 256)()
    n = min(lib().kda_prefill_kernel_times(ms, names, 256), 256)
    if n < 0:
        raise RuntimeError("no timed prefill recorded")
    return [(names[i].decode(), float(ms[i])) for i in range(n)]
