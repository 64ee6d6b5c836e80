#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One JSON line on stdout.  The headline is the long-context prefill, the
largest single-GPU prefill workload (B=1, T=65536, H=32, dk=dv=128, bf16
q/k/v, fp32 log_alpha/beta/state, log_alpha = logsigmoid(N(4, 1))):

  value      prefill tokens/s over exactly --steps timed steps (after --warmup
             untimed ones), inputs resident in HBM, wall clock bracketed by
             device synchronisation;
  roofline   the dominant prefill kernel (most time per step) against the
             8 TB/s HBM peak: its algorithmic bytes per launch over its average
             launch duration, from HIP events each kernel records at its own
             start and end (the library's kernel timing); traffic from
             rocprofv3 counters when the committed measurement matches the
             current kernel sources, and the rate of that traffic against the
             copy ceilings;
  path       the whole step against its HBM roofline (1540 B per token-head
             plus the final state) from the wall clock, and the MFMA rate at
             the dense-tile flop count;
  ceilings   measured alongside: a plain device copy (HBM) and a large bf16
             GEMM (MFMA), each with its fraction of the datasheet peak;
  configs    the other prefill workloads: the single 4096-token sequence
             (rotated input sets, so no step reads what the previous one left
             in the 256 MB last-level cache) and the packed batch of 16
             sequences with nonzero initial states;
  decode     the batched decode workload (256 seqs x 32 heads, 128 steps), GB/s;
  options    chunk-state export, in-kernel preprocessing, the pooled recurrent
             path and the backward pass, on the 4096-token workload;
  cpu_baseline  the fp64 oracle on the host cores, on the headline's inputs;
  parity     the headline's output and final state against that oracle run
             (relative L2 of the whole tensors, every head and every 64-token
             chunk); the run exits with status 1 after its line if any is
             outside the tolerance.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Single workloads for profiling (one JSON object each): --decode-only,
--decode-tokens-only, --backward-only, --packed-only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # dense
METRIC = "KDA prefill tokens/s (H=32,d=128) + decode state GB/s, % of roofline"

# Algorithmic bytes per token-head at dk=dv=128 (bf16 q/k/v/o, fp32 log_alpha/beta).
CHUNK = 64
PATH_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 256          # 1540: q,k,v + log_alpha + beta + o
INTRA_READ = 3 * 256 + 512 + 4                                # 1284: q,k,v + log_alpha + beta
DECODE_BYTES_PER_UNIT = 2 * 128 * 128 * 4 + 3 * 256 + 512 + 4 + 256   # 132,612
FLOP_PER_TOKEN_HEAD_DENSE = 180224                             # chunkwise form, dense 64-tiles
STATE_BYTES = 128 * 128 * 4                                    # one head's fp32 state
CPU_MIN_SECONDS = 10.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM traffic of `kernel` on `workload` from the committed rocprofv3 counter
    summary, if it was measured on the current source of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload, {}).get(kernel)
        if not rec or rec.get("source_sha") != kernel_source_sha(rec["sources"]):
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


PARITY_TOL = 2e-2   # relative L2 for bf16 q/k/v: whole tensors, every head, every chunk


def headline_parity(head, ref):
    """The headline's output and final state (from its last timed step) against
    the oracle's, on the same inputs: relative L2 of the whole tensors, of every
    head, and of every (64-token chunk, head)."""
    o_ref, s_ref = ref[0], ref[1]
    o = head.out[0].float().cpu().numpy().astype(np.float64)
    fin = head.fin.cpu().numpy().astype(np.float64)
    e2 = ((o - o_ref) ** 2).sum(axis=2)          # [T, H]
    r2 = (o_ref ** 2).sum(axis=2)
    del o
    T, H = e2.shape
    nc = -(-T // CHUNK)
    pad = nc * CHUNK - T
    ce = np.pad(e2, ((0, pad), (0, 0))).reshape(nc, CHUNK, H).sum(1)
    cr = np.pad(r2, ((0, pad), (0, 0))).reshape(nc, CHUNK, H).sum(1)
    rel = lambda e, r: np.sqrt(e / np.maximum(r, 1e-300))  # noqa: E731
    res = {"o": float(rel(e2.sum(), r2.sum())),
           "final_state": float(rel(((fin - s_ref) ** 2).sum(), (s_ref ** 2).sum())),
           "worst_head_o": float(rel(e2.sum(0), r2.sum(0)).max()),
           "worst_chunk_o": float(rel(ce, cr).max())}
    ok = all(v <= PARITY_TOL for v in res.values())
    out = {k: float(f"{v:.3e}") for k, v in res.items()}
    out.update({"tol": PARITY_TOL, "ok": bool(ok),
                "against": "the fp64 oracle's output on the same inputs (the CPU leg's run)"})
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Prefill:
    """Device buffers of one prefill workload and a step that runs it."""

    def __init__(self, x, dev, sets=1):
        import torch
        import gated_delta_rule_prefill_amd as kdalib
        self.x, self.kdalib = x, kdalib
        T, H, dk, dv, N = x.T, x.H, x.dk, x.dv, x.num_seqs

        def dq(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

        # distinct buffers with identical contents: the work stays the same while
        # consecutive steps read different memory
        self.sets = [dict(q=dq(x.q), k=dq(x.k), v=dq(x.v),
                          la=torch.from_numpy(x.log_alpha).to(dev),
                          beta=torch.from_numpy(x.beta).to(dev)) for _ in range(sets)]
        self.s0 = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(dev)
        self.cu = None if x.cu_seqlens is None else \
            torch.from_numpy(np.ascontiguousarray(x.cu_seqlens, dtype=np.int32)).to(dev)
        self.out = [torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev) for _ in range(sets)]
        self.fin = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        self.ws = torch.empty(kdalib.workspace_bytes(T, N, H, dk, dv, True), dtype=torch.uint8,
                              device=dev)
        self.token_heads = T * H
        self.path_bytes = PATH_BYTES_PER_TOKEN_HEAD * T * H + N * H * STATE_BYTES * \
            (2 if x.initial_state is not None else 1)

    def step(self, i=0, **kw):
        s = self.sets[i % len(self.sets)]
        self.kdalib.prefill(s["q"], s["k"], s["v"], s["la"], s["beta"], self.s0, self.cu,
                            num_seqs=self.x.num_seqs, final_state=self.fin,
                            out=self.out[i % len(self.sets)], workspace=self.ws, **kw)

    def event_time_us(self, reps, warm=3, same_set=False):
        """Mean time per step from events; the steps rotate over the input sets
        unless same_set (then every step reads what the last one left cached)."""
        import torch
        pick = (lambda i: 0) if same_set else (lambda i: i)  # noqa: E731
        for i in range(warm):
            self.step(pick(i))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            self.step(pick(i))
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def kernel_us(self, reps, per_launch=False):
        """Time of each kernel per step (HIP events each kernel records at its own
        start and end); with per_launch, (average us per launch,
        launches per step) instead: a long batch runs its kernels per segment."""
        self.kdalib.set_kernel_timing(True)
        sums, counts = {}, {}
        try:
            for i in range(reps):
                self.step(i)
                for name, ms in self.kdalib.prefill_kernel_times():
                    sums[name] = sums.get(name, 0.0) + ms
                    counts[name] = counts.get(name, 0) + 1
        finally:
            self.kdalib.set_kernel_timing(False)
        if per_launch:
            return {k: (v * 1e3 / counts[k], counts[k] / reps) for k, v in sums.items()}
        return {k: v * 1e3 / reps for k, v in sums.items()}

    def summary(self, us):
        x = self.x
        tok_s = x.T / (us * 1e-6)
        roof_tok_s = x.T * HBM_PEAK_GBS * 1e9 / self.path_bytes
        return {"us_per_step": round(us, 2), "tokens_per_s": round(tok_s, 1),
                "algorithmic_bytes_per_step": self.path_bytes,
                "achieved_GBs": round(self.path_bytes / (us * 1e-6) / 1e9, 1),
                "roofline_tokens_per_s": round(roof_tok_s),
                "frac_of_roofline": round(tok_s / roof_tok_s, 4),
                "mfma_tflops_dense_count": round(FLOP_PER_TOKEN_HEAD_DENSE * self.token_heads /
                                                 (us * 1e-6) / 1e12, 1)}


def backward_option(single, cs, reps, timed):
    """kda_backward on the 4096-token workload (H=32, d=128, bf16) from its
    exported chunk states cs: the chunkwise path (reverse-chain records, the
    reverse chain, the per-chunk gradient kernel)."""
    import torch
    import gated_delta_rule_prefill_amd as kdalib
    x = single.x
    T, H, dk, dv = x.T, x.H, x.dk, x.dv
    dev = cs.device
    g = np.random.default_rng(11)
    d_o = torch.from_numpy(gen_bf16(g.standard_normal((T, H, dv)).astype(np.float32))).view(
        torch.bfloat16).to(dev)
    s0 = single.sets[0]
    bws = torch.empty(kdalib.backward_workspace_bytes(T, 1, H, dk, dv, True), dtype=torch.uint8,
                      device=dev)
    single.step(0, chunk_states=cs)
    us = timed(lambda i: kdalib.backward(s0["q"], s0["k"], s0["v"], s0["la"], s0["beta"], d_o,
                                         chunk_states=cs, need_initial_state_grad=False,
                                         workspace=bws), reps)
    # the same gradients when the caller kept no chunk states: the call
    # recomputes them with the forward kernels first
    us_rc = timed(lambda i: kdalib.backward(s0["q"], s0["k"], s0["v"], s0["la"], s0["beta"], d_o,
                                            need_initial_state_grad=False, workspace=bws), reps)
    nbytes = (PATH_BYTES_PER_TOKEN_HEAD + 768 + 512 + 4) * T * H
    return {"workload": "gradients of the 4096-token prefill (H=32, d=128, bf16) from its "
                        "exported chunk states", "path": "chunkwise", "us_per_call": round(us, 1),
            "tokens_per_s": round(T / (us * 1e-6), 1), "algorithmic_bytes": nbytes,
            "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "us_per_call_recomputing_chunk_states": round(us_rc, 1)}


def decode_option(dev, steps):
    """The batched decode workload: 256 sequences x 32 heads, dk = dv = 128, fp32
    states (512 MiB) updated in place by `steps` consecutive kda_decode_step calls
    (bf16 q/k/v, 16 token sets in rotation)."""
    import torch
    import gated_delta_rule_prefill_amd as kdalib
    from gated_delta_rule_prefill_amd import inputs as gen

    def dq(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    c = gen.DECODE_WORKLOAD
    N, Hd = c["N"], c["H"]
    state = torch.from_numpy(gen.decode_state(c["seed"], N, Hd, c["dk"], c["dv"])).to(dev)
    toks = []
    for s_ in range(min(steps, 16)):
        y = gen.decode_token(c["seed"], s_, N, Hd, c["dk"], c["dv"])
        toks.append((dq(y.q), dq(y.k), dq(y.v), torch.from_numpy(y.log_alpha).to(dev),
                     torch.from_numpy(y.beta).to(dev)))
    o_dec = torch.empty((N, Hd, c["dv"]), dtype=torch.bfloat16, device=dev)
    for s_ in range(4):
        kdalib.decode_step(state, *toks[s_ % len(toks)], out=o_dec)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s_ in range(steps):
        kdalib.decode_step(state, *toks[s_ % len(toks)], out=o_dec)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    gbs = DECODE_BYTES_PER_UNIT * N * Hd / (us * 1e-6) / 1e9
    # the same step as kda_decode_tokens on the states as a pool in permuted slot order
    slots = torch.from_numpy(np.random.default_rng(c["seed"]).permutation(N).astype(np.int32)).to(dev)

    def pooled(t):
        q_, k_, v_, la_, b_ = t
        kdalib.decode_tokens(state, q_, k_, v_, la_, b_, state_indices=slots, num_seqs=N, out=o_dec)
    for s_ in range(4):
        pooled(toks[s_ % len(toks)])
    torch.cuda.synchronize()
    e0.record()
    for s_ in range(steps):
        pooled(toks[s_ % len(toks)])
    e1.record()
    torch.cuda.synchronize()
    us_pool = e0.elapsed_time(e1) * 1e3 / steps
    return {"workload": "batched decode: 256 seqs x 32 heads, dk=dv=128, fp32 state "
                        "(512 MiB), bf16 q/k/v", "steps": steps,
            "us_per_step": round(us, 2), "value": round(gbs, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": DECODE_BYTES_PER_UNIT * N * Hd,
            "us_per_step_decode_tokens_permuted_slots": round(us_pool, 2)}


def decode_tokens_option(dev, reps, timed):
    """kda_decode_tokens on 256 sequences of 8 tokens (H=32, d=128, bf16), fp32
    states in a permuted order of pool slots."""
    import torch
    import gated_delta_rule_prefill_amd as kdalib
    from gated_delta_rule_prefill_amd import inputs as gen
    H, dk, dv, Nr, Tr = 32, 128, 128, 256, 8

    def dq(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    rr = gen.make_prefill(9, [Tr] * Nr, H=H, dk=dk, dv=dv, dtype="bf16")
    pool = torch.from_numpy(gen.decode_state(9, Nr, H, dk, dv)).to(dev)
    slots = torch.from_numpy(np.random.default_rng(9).permutation(Nr).astype(np.int32)).to(dev)
    rin = dict(q=dq(rr.q), k=dq(rr.k), v=dq(rr.v), la=torch.from_numpy(rr.log_alpha).to(dev),
               beta=torch.from_numpy(rr.beta).to(dev))
    o_r = torch.empty((Nr * Tr, H, dv), dtype=torch.bfloat16, device=dev)
    us = timed(lambda i: kdalib.decode_tokens(pool, rin["q"], rin["k"], rin["v"], rin["la"],
                                              rin["beta"], state_indices=slots, num_seqs=Nr,
                                              out=o_r), reps)
    nbytes = Nr * H * (2 * dk * dv * 4 + Tr * PATH_BYTES_PER_TOKEN_HEAD)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "pooled recurrent tokens: 256 seqs x 8 tokens, H=32, dk=dv=128, bf16, "
                        "fp32 states in permuted slots", "us_per_call": round(us, 2),
            "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def gen_bf16(a):
    from gated_delta_rule_prefill_amd import inputs as gen
    return gen.bf16_bits(a).view(np.int16)


def ceilings(dev):
    """Achievable rates measured in the same run: a device copy and a bf16 GEMM."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    n = 1 << 31
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    best = 1e9
    for i in range(8):
        e0, e1 = ev(), ev()
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    copy_gbs = 2 * n / (best * 1e-3) / 1e9
    del b
    f = a.view(torch.float32)   # in-place scale of the same 2 GiB: one read and one write
    best = 1e9
    for i in range(8):
        e0, e1 = ev(), ev()
        e0.record()
        f.mul_(1.0)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    scale_gbs = 2 * n / (best * 1e-3) / 1e9
    # The prefill kernels' own mix: inputs streamed once from HBM while a
    # fixed ~200 MB area (the record area of one segment, which every segment
    # reuses) is written and read back, so that area can stay in the 256 MB
    # last-level cache.  (1) a copy whose source rotates over 2 GiB of fresh
    # data and whose destination is one 192 MiB buffer; (2) a copy between two
    # 96 MiB buffers, both cache-resident after the first pass.
    src = a.view(torch.uint8)
    m = 192 << 20
    dst = torch.empty(m, dtype=torch.uint8, device=dev)
    best = 1e9
    for i in range(2 * (n // m)):
        j = i % (n // m)
        e0, e1 = ev(), ev()
        e0.record()
        dst.copy_(src[j * m:(j + 1) * m])
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    fresh_to_resident = 2 * m / (best * 1e-3) / 1e9
    h = m // 2
    best = 1e9
    for i in range(12):
        e0, e1 = ev(), ev()
        e0.record()
        dst[h:].copy_(dst[:h])
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    resident_copy = 2 * h / (best * 1e-3) / 1e9
    del dst, src
    del a, f
    copy_gbs = max(copy_gbs, scale_gbs)
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    y = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    best = 1e9
    for i in range(8):
        e0, e1 = ev(), ev()
        e0.record()
        torch.mm(x, y)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            best = min(best, e0.elapsed_time(e1))
    mm_tflops = 2 * m ** 3 / (best * 1e-3) / 1e12
    del x, y
    return {"hbm_copy_GBs": round(copy_gbs, 1), "hbm_copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "hbm_copy": "the faster of a torch copy of a 2 GiB device buffer and an in-place "
                        "scale of one (read + write counted), best of 6 runs each",
            "fresh_to_resident_copy_GBs": round(fresh_to_resident, 1),
            "fresh_to_resident_copy": "192 MiB copies from a source rotating over 2 GiB into one "
                                      "fixed 192 MiB destination (read + write counted), best",
            "resident_copy_GBs": round(resident_copy, 1),
            "resident_copy": "96 MiB copied between two halves of that destination, again and "
                             "again (last-level-cache resident), best of 10",
            "bf16_gemm_TFLOPs": round(mm_tflops, 1),
            "bf16_gemm_frac_of_peak": round(mm_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
            "bf16_gemm": "torch.mm of two 8192x8192 bf16 matrices (hipBLASLt), best of 6"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other prefill workloads, ceilings and optional paths")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the optional paths (chunk states, preprocessing, pooled tokens, backward)")
    ap.add_argument("--headline", choices=["long", "single"], default="long",
                    help="headline workload: the 65536-token sequence (default) or the 4096-token one")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the batched decode workload and print its JSON object")
    ap.add_argument("--decode-tokens-only", action="store_true",
                    help="time only the pooled-recurrent option (--steps calls after --warmup; "
                         "for profiling) and print its JSON")
    ap.add_argument("--packed-only", action="store_true",
                    help="time only the packed 16-sequence prefill (--steps steps after --warmup; "
                         "for profiling) and print its JSON")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward option (--steps calls after --warmup; for "
                         "profiling) and print its JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the KDA hot path here is built and timed on a "
              "single MI355X (no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_prefill_amd as kdalib
    from gated_delta_rule_prefill_amd import inputs as gen
    from gated_delta_rule_prefill_amd import kda as kbind

    kbind.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def dq(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    if args.decode_only:
        print(json.dumps(decode_option(dev, args.decode_steps)), flush=True)
        return
    if args.packed_only:
        packed = Prefill(gen.workload_prefill("packed_16"), dev)
        us = packed.event_time_us(args.steps, warm=args.warmup)
        c3 = packed.summary(us)
        c3["workload"] = (f"packed varlen prefill, 16 sequences U[256,4096] (T={packed.x.T}), H=32 "
                          f"dk=dv=128 bf16, nonzero fp32 initial states, per-sequence final states")
        c3["kernel_us"] = {k: round(v, 2) for k, v in packed.kernel_us(10).items()}
        c3["kernel_us_per_launch"] = {k: [round(v[0], 2), v[1]] for k, v in
                                      packed.kernel_us(10, per_launch=True).items()}
        print(json.dumps(c3), flush=True)
        return
    if args.backward_only or args.decode_tokens_only:
        def timed(fn, reps):
            for i in range(args.warmup):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        if args.decode_tokens_only:
            print(json.dumps(decode_tokens_option(dev, args.steps, timed)), flush=True)
            return
        single = Prefill(gen.workload_prefill("single_T4096"), dev)
        cs = torch.empty((kdalib.num_chunk_states(single.x.T, 1), single.x.H, single.x.dk,
                          single.x.dv), dtype=torch.float32, device=dev)
        print(json.dumps(backward_option(single, cs, args.steps, timed)), flush=True)
        return

    rec_extra = {}
    single = None
    if not args.no_extra or args.headline == "single":
        log("[bench] single-sequence workload T=4096 H=32 d=128, 3 rotated input sets")
        single = Prefill(gen.workload_prefill("single_T4096"), dev, sets=3)

    if not args.no_extra:
        rec_extra["ceilings"] = ceilings(dev)
        log(f"[bench] ceilings: {rec_extra['ceilings']}")
        # -- the other prefill workloads ------------------------------------
        us = single.event_time_us(100, warm=20)
        c2 = single.summary(us)
        c2["workload"] = "single-sequence prefill B=1 T=4096 H=32 dk=dv=128 bf16, zero initial state"
        c2["kernel_us"] = {k: round(v, 2) for k, v in single.kernel_us(50).items()}
        # the 204 MB a step moves fits the 256 MB last-level cache: the figure
        # above rotates three input sets (a step never finds its inputs cached);
        # this one repeats one set
        c2["us_per_step_one_input_set"] = round(single.event_time_us(100, warm=10, same_set=True), 2)
        log(f"[bench] T=4096: {us:.1f} us/step, {c2['tokens_per_s'] / 1e6:.2f} M tok/s, "
            f"{c2['frac_of_roofline']:.3f} of roofline")
        packed = Prefill(gen.workload_prefill("packed_16"), dev)
        us = packed.event_time_us(20)
        c3 = packed.summary(us)
        c3["workload"] = (f"packed varlen prefill, 16 sequences U[256,4096] (T={packed.x.T}), H=32 "
                          f"dk=dv=128 bf16, nonzero fp32 initial states, per-sequence final states")
        c3["kernel_us"] = {k: round(v, 2) for k, v in packed.kernel_us(10).items()}
        log(f"[bench] packed: {us:.1f} us/step, {c3['tokens_per_s'] / 1e6:.2f} M tok/s, "
            f"{c3['frac_of_roofline']:.3f} of roofline")
        rec_extra["configs"] = {"single_4096": c2, "packed_16": c3}
        del packed

    # ---------------- decode workload ----------------
    decode = None
    if not args.no_decode:
        decode = decode_option(dev, args.decode_steps)
        if "ceilings" in rec_extra:
            decode["frac_of_copy_ceiling"] = round(decode["value"] / rec_extra["ceilings"]["hbm_copy_GBs"], 4)
        log(f"[bench] decode: {decode['us_per_step']:.1f} us/step, {decode['value']:.0f} GB/s "
            f"({100 * decode['frac_of_hbm_peak']:.1f}% of peak)")

    # ---------------- optional paths (on the 4096-token workload) ----------------
    options = None
    if not args.no_options and not args.no_extra:
        options = {}
        x = single.x
        T, H, dk, dv = x.T, x.H, x.dk, x.dv
        ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

        def timed(fn, reps):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            for i in range(reps):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        reps = 50
        base_us = timed(single.step, reps)
        nc = kdalib.num_chunk_states(T, 1)
        cs = torch.empty((nc, H, dk, dv), dtype=torch.float32, device=dev)
        cs_us = timed(lambda i: single.step(i, chunk_states=cs), reps)
        options["chunk_states"] = {
            "workload": "the 4096-token prefill, also writing the fp32 state entering each of "
                        "its 64 chunks", "us_per_step": round(cs_us, 2),
            "extra_us": round(cs_us - base_us, 2), "extra_bytes": nc * H * dk * dv * 4,
            "tokens_per_s": round(T / (cs_us * 1e-6), 1)}
        r = gen.make_prefill(2, [T], H=H, dk=dk, dv=dv, dtype="bf16", raw=True)
        raw = Prefill(r, dev)
        pre_runs, plain_runs = [], []
        for _ in range(2):   # alternating runs, best of two each: the clock drifts
            pre_runs.append(timed(lambda i: raw.step(i, l2norm_qk=True, beta_sigmoid=True), reps))
            plain_runs.append(timed(raw.step, reps))
        options["preprocessing"] = {
            "workload": "the 4096-token prefill from raw q/k and beta logits, L2 normalisation "
                        "and sigmoid in the kernels (one input set, cache-warm; best of two "
                        "alternating runs with and without)",
            "us_per_step": round(min(pre_runs), 2), "us_per_step_without": round(min(plain_runs), 2)}
        del raw
        options["decode_tokens"] = decode_tokens_option(dev, reps, timed)
        rec_us, rec_gbs = options["decode_tokens"]["us_per_call"], options["decode_tokens"]["achieved_GBs"]
        options["backward"] = backward_option(single, cs, 20, timed)
        bwd_us = options["backward"]["us_per_call"]
        log(f"[bench] options: chunk states +{cs_us - base_us:.1f} us, preprocessing "
            f"{min(pre_runs):.1f} us (plain {min(plain_runs):.1f}), decode_tokens {rec_us:.1f} us "
            f"= {rec_gbs:.0f} GB/s, backward {bwd_us:.0f} us")
        del cs

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] ran 3 plain copies of 1 GiB (counter calibration)")
        del a, b

    # ---------------- headline: the long-context prefill ----------------
    if args.headline == "long":
        log("[bench] headline workload: B=1 T=65536 H=32 d=128 bf16 (generating inputs)")
        head = Prefill(gen.workload_prefill("long_T65536"), dev)
        workload = ("long-context KDA prefill B=1 T=65536 H=32 dk=dv=128, bf16 q/k/v, fp32 "
                    "log_alpha (logsigmoid(N(4,1)))/beta/state, chunk 64, zero initial state")
        wl_key = "long_65536"
    else:
        head = single
        workload = ("single-sequence KDA prefill B=1 T=4096 H=32 dk=dv=128, bf16 q/k/v, fp32 "
                    "log_alpha/beta/state, chunk 64, zero initial state")
        wl_key = "single_4096"
    T, H = head.x.T, head.x.H
    for i in range(args.warmup):
        head.step(i)
    torch.cuda.synchronize()
    # events between the steps (on the stream the library launches on) give the
    # spread of single steps; the wall clock over all of them gives `value`
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        head.step(i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_us = sorted(1e3 * marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_per_step = 1e3 * dt / args.steps
    tok_s = T / (dt / args.steps)
    log(f"[bench] headline: {ms_per_step * 1e3:.1f} us/step, {tok_s / 1e6:.2f} M tokens/s "
        f"({args.steps} timed steps after {args.warmup} warm-up steps)")
    kern = head.kernel_us(max(5, min(args.steps, 20)), per_launch=True)
    log("[bench] kernel averages per launch: " + ", ".join(
        f"{k}={v[0]:.1f}us x{v[1]:g}" for k, v in kern.items()))
    # The dominant kernel (most time per step) against HBM: its algorithmic bytes
    # per launch (its share of the path's 1540 B per token-head, times the
    # token-heads of one launch) over its average launch duration.
    seg_tokens = T / max(kern.get("prefill_intra", (0, 1))[1], 1)
    kern_bytes = {"prefill_intra": INTRA_READ * seg_tokens * H,
                  "prefill_state": 256 * seg_tokens * H + head.x.num_seqs * H * STATE_BYTES *
                  (2 if head.x.initial_state is not None else 1) / max(kern.get("prefill_state", (0, 1))[1], 1)}
    dom = max((k for k in kern if k in kern_bytes), key=lambda k: kern[k][0] * kern[k][1])
    achieved = kern_bytes[dom] / (kern[dom][0] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(dom, wl_key), "kernel": dom,
                "algorithmic_bytes_per_launch": int(kern_bytes[dom]),
                "avg_launch_us": round(kern[dom][0], 2), "launches_per_step": kern[dom][1],
                "kernels": {k: {"avg_launch_us": round(v[0], 2), "launches_per_step": v[1],
                                "us_per_step": round(v[0] * v[1], 1)} for k, v in kern.items()},
                "note": "the dominant kernel per launch; algorithmic bytes = its share of the "
                        "path's 1540 B per token-head (q, k, v, log_alpha, beta read by the intra "
                        "kernel; o and states by the sequential one); the records one kernel "
                        "hands to the other are in traffic, not in achieved"}
    if "ceilings" in rec_extra:
        roofline["frac_of_copy_ceiling"] = round(achieved / rec_extra["ceilings"]["hbm_copy_GBs"], 4)
    # The rate at which each kernel moves the bytes it really moves (the counted
    # traffic per launch over the launch time): set beside the copy ceiling, it
    # shows how much of a kernel's time its own traffic accounts for.
    rates = {}
    for k, v in kern.items():
        tb = traffic_for(k, wl_key)
        if tb is not None and v[0] > 0:
            rates[k] = {"traffic_bytes_per_launch": tb,
                        "traffic_GBs": round(tb / (v[0] * 1e-6) / 1e9, 1)}
            if "ceilings" in rec_extra:
                c = rec_extra["ceilings"]
                rates[k]["frac_of_copy_ceiling"] = round(rates[k]["traffic_GBs"] / c["hbm_copy_GBs"], 4)
                # the copy whose traffic mix matches the kernel's: the intra kernel
                # streams fresh inputs and writes the reused record area; the
                # sequential kernel reads that area back
                mix = {"prefill_intra": "fresh_to_resident_copy_GBs",
                       "prefill_state": "resident_copy_GBs"}.get(k)
                if mix and c.get(mix):
                    rates[k]["mix_ceiling"] = mix
                    rates[k]["frac_of_mix_ceiling"] = round(rates[k]["traffic_GBs"] / c[mix], 4)
    if rates:
        roofline["traffic_rate"] = rates
    path = head.summary(dt / args.steps * 1e6)
    if step_us:
        path["step_us_events"] = {"min": round(step_us[0], 1),
                                  "median": round(step_us[len(step_us) // 2], 1),
                                  "max": round(step_us[-1], 1)}
    path["mfma_frac_of_bf16_peak"] = round(path["mfma_tflops_dense_count"] / BF16_MFMA_PEAK_TFLOPS, 4)
    if "ceilings" in rec_extra:
        path["frac_of_copy_ceiling"] = round(path["achieved_GBs"] / rec_extra["ceilings"]["hbm_copy_GBs"], 4)

    # ---------------- CPU baseline: the oracle on the headline's inputs ----------------
    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        x = head.x
        threads = oracle.default_threads()
        used = min(oracle.max_threads(threads), H * x.num_seqs)
        reps, ct = 0, 0.0
        while ct < CPU_MIN_SECONDS and reps < 200:
            t1 = time.perf_counter()
            ref = oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.initial_state,
                                 x.cu_seqlens, num_seqs=x.num_seqs, nthreads=threads)
            ct += time.perf_counter() - t1
            reps += 1
        parity = headline_parity(head, ref)
        del ref
        log(f"[bench] parity of the headline against the oracle: {parity}")
        cpu = {"value": round(reps * T / ct, 1), "unit": "tokens/s", "cores": used,
               "kind": "oracle", "cpu_model": cpu_model(),
               "host_threads_available": len(os.sched_getaffinity(0)),
               "sample": f"the headline workload itself (T={T}, H={H}, dk=dv=128), fp64 token "
                         f"loop, run {reps} times back to back: {ct:.1f} s wall on {used} threads"}
        log(f"[bench] oracle: {reps} runs in {ct:.1f} s, {reps * T / ct:.0f} tokens/s "
            f"on {used} threads ({cpu['cpu_model']})")

    rec = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": workload, "global_batch": head.x.num_seqs, "seq_len": T,
                      "heads": H, "head_dim": 128, "parallelism": "single GPU"},
           "roofline": roofline, "path": path, **rec_extra, "decode": decode, "options": options,
           "cpu_baseline": cpu, "parity": parity}
    if cpu:
        cpu["gpu_over_oracle"] = round(tok_s / cpu["value"], 1)
    print(json.dumps(rec), flush=True)
    if parity is not None and not parity["ok"]:
        log("[bench] the headline's output is outside the parity tolerance")
        sys.exit(1)


if __name__ == "__main__":
    main()
