"""Seeded synthetic inputs for KDA prefill and decode.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic, and it is the only code that the GPU path and the fp64
oracle both use.  Every tensor has its own NumPy PCG64 stream keyed by
``(seed, tensor_id[, step])`` so a tensor never depends on the order in which
the others were drawn.

Recipe (the workloads of the Kimi Linear KDA hot path):
  * q, k ~ N(0, 1) per element, L2-normalised over the head dimension in fp32
    (the layer normalises q and k before the recurrence), then cast to the
    input dtype (bf16 by round-to-nearest-even, or kept fp32);
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1)) in fp32 (the layer's write strength is a sigmoid);
  * log_alpha = log(sigmoid(N(mu, 1))) per key channel in fp32, mu = 3 (or 4
    for long-context memory), so alpha is a per-channel decay in (0, 1);
  * states ~ 0.02 * N(0, 1) in fp32, or zero;
  * packed batches list their sequence offsets in ``cu_seqlens`` (int32).

Tensor ids: q=1, k=2, v=3, log_alpha=4, beta=5, initial_state=6, lengths=7.
Decode step s uses the key (seed, 100 + s, tensor_id); decode states (seed, 6).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

Q, K, V, LOG_ALPHA, BETA, STATE, LENGTHS = 1, 2, 3, 4, 5, 6, 7


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(x) for x in key])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they denote (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(g: np.random.Generator, shape, loc: float = 0.0) -> np.ndarray:
    x = g.standard_normal(shape, dtype=np.float32)
    if loc:
        x += np.float32(loc)
    return x


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.einsum("...d,...d->...", x, x, dtype=np.float32))[..., None]
    return (x / n).astype(np.float32)


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (-(np.logaddexp(0.0, -x64))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclass
class KDAInputs:
    """Host-side inputs of one prefill call (or one decode step).

    q, k: [T, H, dk]; v: [T, H, dv] -- float32, or uint16 holding bf16 bits.
    log_alpha: [T, H, dk] float32; beta: [T, H] float32.
    initial_state: [N, H, dk, dv] float32 or None (zeros).
    cu_seqlens: [N+1] int32 or None (N equal rows).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: np.ndarray
    beta: np.ndarray
    initial_state: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    num_seqs: int
    dtype: str  # "f32" | "bf16"

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def dk(self) -> int:
        return self.q.shape[2]

    @property
    def dv(self) -> int:
        return self.v.shape[2]

    def lengths(self) -> List[int]:
        if self.cu_seqlens is None:
            return [self.T // self.num_seqs] * self.num_seqs
        return [int(b - a) for a, b in zip(self.cu_seqlens[:-1], self.cu_seqlens[1:])]

    def select_heads(self, heads: Sequence[int]) -> "KDAInputs":
        """The same inputs restricted to a subset of heads (heads are independent)."""
        h = np.asarray(list(heads), dtype=np.int64)
        return KDAInputs(
            q=np.ascontiguousarray(self.q[:, h]), k=np.ascontiguousarray(self.k[:, h]),
            v=np.ascontiguousarray(self.v[:, h]),
            log_alpha=np.ascontiguousarray(self.log_alpha[:, h]),
            beta=np.ascontiguousarray(self.beta[:, h]),
            initial_state=None if self.initial_state is None
            else np.ascontiguousarray(self.initial_state[:, h]),
            cu_seqlens=self.cu_seqlens, num_seqs=self.num_seqs, dtype=self.dtype)

    def select_seqs(self, seqs: Sequence[int]) -> "KDAInputs":
        """The same inputs restricted to a subset of packed sequences, repacked."""
        lens = self.lengths()
        offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        rows = np.concatenate([np.arange(offs[s], offs[s + 1]) for s in seqs]) if seqs else \
            np.zeros(0, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum([lens[s] for s in seqs])]).astype(np.int32)
        st = None if self.initial_state is None else \
            np.ascontiguousarray(self.initial_state[np.asarray(list(seqs), dtype=np.int64)])
        return KDAInputs(
            q=np.ascontiguousarray(self.q[rows]), k=np.ascontiguousarray(self.k[rows]),
            v=np.ascontiguousarray(self.v[rows]),
            log_alpha=np.ascontiguousarray(self.log_alpha[rows]),
            beta=np.ascontiguousarray(self.beta[rows]), initial_state=st, cu_seqlens=cu,
            num_seqs=len(seqs), dtype=self.dtype)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def make_prefill(seed: int, lengths: Sequence[int], H: int, dk: int, dv: int,
                 dtype: str = "bf16", mu: float = 3.0, state_std: float = 0.0,
                 packed: Optional[bool] = None, raw: bool = False,
                 fixed_even_log_alpha: Optional[float] = None) -> KDAInputs:
    """Inputs for one prefill call over sequences of the given lengths.

    ``fixed_even_log_alpha`` sets log_alpha of every even key channel to that
    value (strong, mixed per-channel decay next to the drawn odd channels).

    ``packed`` (default: more than one distinct length) selects cu_seqlens;
    otherwise the batch is N equal rows and cu_seqlens is None.  ``raw`` draws
    the layer's inputs before its own preprocessing: q and k rows N(0, 1) with
    a per-row scale 2^U(-3, 3) (not normalised) and beta as a N(0, 1) logit.
    """
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T = int(sum(lengths))
    if packed is None:
        packed = len(set(lengths)) > 1
    if not packed and len(set(lengths)) > 1:
        raise ValueError("unequal lengths need a packed batch")
    if raw:
        g = rng(seed, Q, 1)
        q = _normal(rng(seed, Q), (T, H, dk)) * np.exp2(g.uniform(-3, 3, (T, H, 1))).astype(np.float32)
        k = _normal(rng(seed, K), (T, H, dk)) * np.exp2(g.uniform(-3, 3, (T, H, 1))).astype(np.float32)
        beta = _normal(rng(seed, BETA), (T, H))
    else:
        q = _unit_rows(_normal(rng(seed, Q), (T, H, dk)))
        k = _unit_rows(_normal(rng(seed, K), (T, H, dk)))
        beta = _sigmoid(_normal(rng(seed, BETA), (T, H)))
    v = _normal(rng(seed, V), (T, H, dv))
    la = _log_sigmoid(_normal(rng(seed, LOG_ALPHA), (T, H, dk), loc=mu))
    if fixed_even_log_alpha is not None:
        la[:, :, 0::2] = np.float32(fixed_even_log_alpha)
    s0 = None
    if state_std:
        s0 = (np.float32(state_std) * _normal(rng(seed, STATE), (N, H, dk, dv))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if packed else None
    return KDAInputs(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), log_alpha=la,
                     beta=beta, initial_state=s0, cu_seqlens=cu, num_seqs=N, dtype=dtype)


# The named workloads (each with its own fixed seed).
WORKLOADS = {
    "tiny_T256": "tiny fp32 prefill B=1 T=256 H=2 d=64",
    "single_T4096": "single-sequence prefill B=1 T=4096 H=32 d=128 bf16",
    "packed_16": "packed varlen prefill 16 seqs U[256,4096] H=32 d=128 bf16, nonzero states",
    "long_T65536": "long-context prefill B=1 T=65536 H=32 d=128 bf16",
    "decode_256x32": "batched decode 256 seqs H=32 d=128, 128 steps",
}


def packed_16_lengths() -> List[int]:
    """The 16 sequence lengths of the packed workload, uniform in [256, 4096]."""
    return [int(x) for x in rng(3, LENGTHS).integers(256, 4096, size=16, endpoint=True)]


def workload_prefill(name: str) -> KDAInputs:
    """Inputs of a named prefill workload (see WORKLOADS)."""
    if name == "tiny_T256":
        return make_prefill(1, [256], H=2, dk=64, dv=64, dtype="f32", mu=3.0)
    if name == "single_T4096":
        return make_prefill(2, [4096], H=32, dk=128, dv=128, dtype="bf16", mu=3.0)
    if name == "packed_16":
        return make_prefill(3, packed_16_lengths(), H=32, dk=128, dv=128, dtype="bf16", mu=3.0,
                            state_std=0.02, packed=True)
    if name == "long_T65536":
        return make_prefill(4, [65536], H=32, dk=128, dv=128, dtype="bf16", mu=4.0)
    raise ValueError(name)


def decode_state(seed: int, N: int, H: int, dk: int, dv: int, std: float = 0.02) -> np.ndarray:
    return (np.float32(std) * _normal(rng(seed, STATE), (N, H, dk, dv))).astype(np.float32)


def decode_token(seed: int, step: int, N: int, H: int, dk: int, dv: int,
                 dtype: str = "bf16", mu: float = 3.0) -> KDAInputs:
    """Inputs of decode step ``step`` (one token per sequence), shapes [N, H, d]."""
    q = _unit_rows(_normal(rng(seed, 100 + step, Q), (N, H, dk)))
    k = _unit_rows(_normal(rng(seed, 100 + step, K), (N, H, dk)))
    v = _normal(rng(seed, 100 + step, V), (N, H, dv))
    la = _log_sigmoid(_normal(rng(seed, 100 + step, LOG_ALPHA), (N, H, dk), loc=mu))
    beta = _sigmoid(_normal(rng(seed, 100 + step, BETA), (N, H)))
    return KDAInputs(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), log_alpha=la,
                     beta=beta, initial_state=None, cu_seqlens=None, num_seqs=N, dtype=dtype)


# the batched decode workload
DECODE_WORKLOAD = dict(seed=5, N=256, H=32, dk=128, dv=128, steps=128, dtype="bf16", mu=3.0)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Values of a q/k/v array as float32 (bf16 bit patterns widened exactly)."""
    return bf16_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)
