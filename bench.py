#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One JSON line on stdout:
  value    prefill tokens/s of the single-sequence workload (B=1, T=4096, H=32,
           dk=dv=128, bf16 q/k/v, fp32 log_alpha/beta/state), inputs resident in
           HBM, several input sets rotated so that no step reads what the
           previous one left in the 256 MB last-level cache;
  roofline the dominant prefill kernel: algorithmic bytes per launch divided by
           its average duration (HIP events the library records on its own
           stream), against the 8 TB/s HBM peak; traffic from rocprofv3 counters
           when the committed measurement matches the current kernel source;
  path     the whole prefill path against its HBM roofline (1540 B per token-head);
  decode   the batched decode workload (256 seqs x 32 heads, 128 steps) in GB/s;
  options  the optional paths: chunk-state export, in-kernel preprocessing and
           the pooled multi-token recurrent path;
  cpu_baseline  the fp64 oracle on the host cores, same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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

# Algorithmic bytes per token-head at H=32, dk=dv=128 (bf16 q/k/v/o, fp32 log_alpha/beta).
CHUNK = 64
PATH_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 256          # 1540: q,k,v + log_alpha + beta + o
INTRA_READ = 3 * 256 + 512 + 4                                # 1284: q,k,v + log_alpha + beta


def record_bytes(dk=128, dv=128, es=2):
    """Bytes of one chunk-head record the intra-chunk kernel writes and the sequential
    kernel reads: PM (dk x dk), Hc (dk x dv), QM (C x dk), OI (C x dv) in the I/O type,
    the chunk decay gamma_C (dk fp32), padded to 256 B."""
    b = (dk * dk + dk * dv + CHUNK * dk + CHUNK * dv) * es + dk * 4
    return (b + 255) // 256 * 256


RECORD_PER_TOKEN_HEAD = record_bytes() / CHUNK                # 1544
DECODE_BYTES_PER_UNIT = 2 * 128 * 128 * 4 + 3 * 256 + 512 + 4 + 256   # 132,612
FLOP_PER_TOKEN_HEAD_DENSE = 180224                             # chunkwise form, dense 64-tiles
CPU_MIN_SECONDS = 10.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_prefill_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str):
    """HBM traffic of `kernel` from the committed rocprofv3 counter summary, if it
    was measured on the current source of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
        if not rec or rec.get("source_sha") != kernel_source_sha(rec["sources"]):
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=3, help="rotated input sets (defeat the MALL)")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-options", action="store_true",
                    help="skip the optional paths (chunk states, preprocessing, pooled tokens)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
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

    # ---------------- prefill workload (config 2) ----------------
    x = gen.config_prefill(2)
    T, H, dk, dv = x.T, x.H, x.dk, x.dv
    log(f"[bench] prefill workload: B=1 T={T} H={H} dk={dk} dv={dv} bf16, {args.sets} input sets")

    def dq(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    sets = []
    for i in range(args.sets):
        # distinct buffers with identical contents (a different permutation of heads would
        # change the work; copies keep the work identical while defeating cache reuse)
        sets.append(dict(q=dq(x.q), k=dq(x.k), v=dq(x.v),
                         la=torch.from_numpy(x.log_alpha).to(dev),
                         beta=torch.from_numpy(x.beta).to(dev)))
    out = [torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev) for _ in range(args.sets)]
    fin = torch.empty((1, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(kdalib.workspace_bytes(T, 1, H, dk, dv, True), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % args.sets]
        kdalib.prefill(s["q"], s["k"], s["v"], s["la"], s["beta"], None, None, num_seqs=1,
                       final_state=fin, out=out[i % args.sets], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = 1e3 * dt / args.steps
    tok_s = T / (dt / args.steps)
    log(f"[bench] prefill: {ms_per_step * 1e3:.1f} us/step, {tok_s / 1e6:.2f} M tokens/s")

    # per-kernel durations from events recorded by the library on its stream
    kdalib.set_kernel_timing(True)
    sums = {}
    nrep = max(20, min(args.steps, 100))
    for i in range(nrep):
        step(i)
        for name, ms in kdalib.prefill_kernel_times():
            sums[name] = sums.get(name, 0.0) + ms
    kdalib.set_kernel_timing(False)
    kern_ms = {k: v / nrep for k, v in sums.items()}
    log("[bench] kernel averages (ms): " + ", ".join(f"{k}={v * 1e3:.1f}us" for k, v in kern_ms.items()))
    token_heads = T * H
    # Algorithmic bytes of each kernel: its share of the path's 1540 B per token-head
    # (the intra-chunk kernel reads q, k, v, log_alpha, beta; the sequential kernel writes
    # o and the final state).  The per-chunk records one kernel hands to the other are this
    # design's own traffic: they show up in `traffic`, not in `achieved`.
    kern_bytes = {"prefill_intra": INTRA_READ * token_heads,
                  "prefill_state": H * dk * dv * 4 + 256 * token_heads,
                  "chunk_table": 0}
    record_bytes_per_step = int(RECORD_PER_TOKEN_HEAD * token_heads)
    dom = max((k for k in kern_ms if kern_bytes.get(k)), key=lambda k: kern_ms[k])
    achieved = kern_bytes[dom] / (kern_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(dom), "kernel": dom,
                "algorithmic_bytes_per_launch": kern_bytes[dom],
                "record_bytes_per_launch": record_bytes_per_step,
                "avg_launch_us": round(kern_ms[dom] * 1e3, 2)}
    path_bytes = PATH_BYTES_PER_TOKEN_HEAD * token_heads
    path_roof_tok_s = HBM_PEAK_GBS * 1e9 / (PATH_BYTES_PER_TOKEN_HEAD * H)
    path = {"bound": "hbm", "algorithmic_bytes_per_step": path_bytes,
            "achieved_GBs": round(path_bytes / (dt / args.steps) / 1e9, 1),
            "roofline_tokens_per_s": round(path_roof_tok_s),
            "frac_of_roofline": round(tok_s / path_roof_tok_s, 4),
            "mfma_tflops_dense_count": round(FLOP_PER_TOKEN_HEAD_DENSE * token_heads /
                                             (dt / args.steps) / 1e12, 1),
            "mfma_frac_of_bf16_peak": round(FLOP_PER_TOKEN_HEAD_DENSE * token_heads /
                                            (dt / args.steps) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in kern_ms.items()}}

    # ---------------- decode workload (config 5) ----------------
    decode = None
    if not args.no_decode:
        c = gen.DECODE_CONFIG
        N, Hd = c["N"], c["H"]
        state = torch.from_numpy(gen.decode_state(c["seed"], N, Hd, c["dk"], c["dv"])).to(dev)
        toks = []
        for s_ in range(min(args.decode_steps, 16)):
            y = gen.decode_token(c["seed"], s_, N, Hd, c["dk"], c["dv"])
            toks.append((dq(y.q), dq(y.k), dq(y.v), torch.from_numpy(y.log_alpha).to(dev),
                         torch.from_numpy(y.beta).to(dev)))
        o_dec = torch.empty((N, Hd, c["dv"]), dtype=torch.bfloat16, device=dev)
        for s_ in range(4):
            kdalib.decode_step(state, *toks[s_ % len(toks)], out=o_dec)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s_ in range(args.decode_steps):
            kdalib.decode_step(state, *toks[s_ % len(toks)], out=o_dec)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.decode_steps
        gbs = DECODE_BYTES_PER_UNIT * N * Hd / (us * 1e-6) / 1e9
        decode = {"workload": "batched decode: 256 seqs x 32 heads, dk=dv=128, fp32 state "
                              "(512 MiB), bf16 q/k/v", "steps": args.decode_steps,
                  "us_per_step": round(us, 2), "value": round(gbs, 1), "unit": "GB/s",
                  "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                  "algorithmic_bytes_per_step": DECODE_BYTES_PER_UNIT * N * Hd}
        log(f"[bench] decode: {us:.1f} us/step, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)")
        del state

    # ---------------- optional paths ----------------
    options = None
    if not args.no_options:
        options = {}
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

        reps = max(20, min(args.steps, 100))
        base_us = timed(step, reps)
        # chunk-state export: fp32 state entering each of the 64 chunks, per head
        nc = kdalib.num_chunk_states(T, 1)
        cs = torch.empty((nc, H, dk, dv), dtype=torch.float32, device=dev)

        def step_cs(i):
            s = sets[i % args.sets]
            kdalib.prefill(s["q"], s["k"], s["v"], s["la"], s["beta"], None, None, num_seqs=1,
                           final_state=fin, out=out[i % args.sets], workspace=ws, chunk_states=cs)
        cs_us = timed(step_cs, reps)
        cs_bytes = nc * H * dk * dv * 4
        options["chunk_states"] = {
            "workload": "the prefill workload, also writing the fp32 state entering each of "
                        "its 64 chunks", "us_per_step": round(cs_us, 2),
            "extra_us": round(cs_us - base_us, 2), "extra_bytes": cs_bytes,
            "tokens_per_s": round(T / (cs_us * 1e-6), 1)}
        # in-kernel q/k normalisation and beta sigmoid on raw inputs
        r = gen.make_prefill(2, [T], H=H, dk=dk, dv=dv, dtype="bf16", raw=True)
        raw = dict(q=dq(r.q), k=dq(r.k), v=dq(r.v), la=torch.from_numpy(r.log_alpha).to(dev),
                   beta=torch.from_numpy(r.beta).to(dev))

        def step_pre(i):
            kdalib.prefill(raw["q"], raw["k"], raw["v"], raw["la"], raw["beta"], None, None,
                           num_seqs=1, final_state=fin, out=out[0], workspace=ws,
                           l2norm_qk=True, beta_sigmoid=True)

        def step_plain_same_buffers(i):
            kdalib.prefill(raw["q"], raw["k"], raw["v"], raw["la"], raw["beta"], None, None,
                           num_seqs=1, final_state=fin, out=out[0], workspace=ws)
        # alternating runs, best of two each: the clock drifts over a long run
        pre_runs, plain_runs = [], []
        for _ in range(2):
            pre_runs.append(timed(step_pre, reps))
            plain_runs.append(timed(step_plain_same_buffers, reps))
        pre_us, plain_us = min(pre_runs), min(plain_runs)
        options["preprocessing"] = {
            "workload": "the prefill workload from raw q/k and beta logits, L2 normalisation "
                        "and sigmoid in the kernels (one input set, cache-warm; best of two "
                        "alternating runs with and without)",
            "us_per_step": round(pre_us, 2), "us_per_step_without": round(plain_us, 2)}
        # pooled recurrent tokens: 256 sequences x 8 tokens (speculative verification)
        Nr, Tr, Hr = 256, 8, H
        rr = gen.make_prefill(9, [Tr] * Nr, H=Hr, dk=dk, dv=dv, dtype="bf16")
        pool = torch.from_numpy(gen.decode_state(9, Nr, Hr, dk, dv)).to(dev)
        slots = torch.from_numpy(np.random.default_rng(9).permutation(Nr).astype(np.int32)).to(dev)
        rin = dict(q=dq(rr.q), k=dq(rr.k), v=dq(rr.v), la=torch.from_numpy(rr.log_alpha).to(dev),
                   beta=torch.from_numpy(rr.beta).to(dev))
        o_r = torch.empty((Nr * Tr, Hr, dv), dtype=torch.bfloat16, device=dev)

        def step_rec(i):
            kdalib.decode_tokens(pool, rin["q"], rin["k"], rin["v"], rin["la"], rin["beta"],
                                 state_indices=slots, num_seqs=Nr, out=o_r)
        rec_us = timed(step_rec, reps)
        rec_bytes = Nr * Hr * (2 * dk * dv * 4 + Tr * PATH_BYTES_PER_TOKEN_HEAD)
        rec_gbs = rec_bytes / (rec_us * 1e-6) / 1e9
        options["decode_tokens"] = {
            "workload": "pooled recurrent tokens: 256 seqs x 8 tokens, H=32, dk=dv=128, bf16, "
                        "fp32 states in permuted slots", "us_per_call": round(rec_us, 2),
            "algorithmic_bytes": rec_bytes, "achieved_GBs": round(rec_gbs, 1),
            "frac_of_hbm_peak": round(rec_gbs / HBM_PEAK_GBS, 4)}
        # backward of the prefill workload from the exported chunk states
        g = np.random.default_rng(11)
        d_o = dq(gen.bf16_bits(g.standard_normal((T, H, dv)).astype(np.float32)))
        s0set = sets[0]
        bws = torch.empty(kdalib.backward_workspace_bytes(T, 1, H, dk, dv, True), dtype=torch.uint8,
                          device=dev)
        kdalib.prefill(s0set["q"], s0set["k"], s0set["v"], s0set["la"], s0set["beta"], None, None,
                       num_seqs=1, final_state=fin, out=out[0], workspace=ws, chunk_states=cs)

        def step_bwd(i):
            kdalib.backward(s0set["q"], s0set["k"], s0set["v"], s0set["la"], s0set["beta"], d_o,
                            chunk_states=cs, need_initial_state_grad=False, workspace=bws)
        bwd_us = timed(step_bwd, max(3, reps // 10))
        bwd_bytes = (PATH_BYTES_PER_TOKEN_HEAD + 768 + 512 + 4) * token_heads
        options["backward"] = {
            "workload": "gradients of the prefill workload (T=4096, H=32, d=128, bf16) from its "
                        "exported chunk states", "us_per_call": round(bwd_us, 1),
            "tokens_per_s": round(T / (bwd_us * 1e-6), 1),
            "algorithmic_bytes": bwd_bytes,
            "achieved_GBs": round(bwd_bytes / (bwd_us * 1e-6) / 1e9, 1)}
        log(f"[bench] options: chunk states {cs_us:.1f} us (+{cs_us - base_us:.1f}), "
            f"preprocessing {pre_us:.1f} us (plain {plain_us:.1f}), "
            f"decode_tokens 256x8 {rec_us:.1f} us = {rec_gbs:.0f} GB/s, backward {bwd_us:.0f} us")
        del pool, cs, bws

    if args.copy_calib:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] ran 3 plain copies of 1 GiB (counter calibration)")

    # ---------------- CPU baseline: the oracle on the same inputs ----------------
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = oracle.default_threads()
        used = min(oracle.max_threads(threads), H)
        reps, ct = 0, 0.0
        while ct < CPU_MIN_SECONDS and reps < 200:
            t0 = time.perf_counter()
            oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, None, None, num_seqs=1,
                           nthreads=threads)
            ct += time.perf_counter() - t0
            reps += 1
        cpu = {"value": round(reps * T / ct, 1), "unit": "tokens/s", "cores": used,
               "kind": "oracle",
               "sample": f"the single-sequence workload (T={T}, H={H}, dk=dv=128) in fp64, "
                         f"run {reps} times back to back: {ct:.1f} s wall on {used} threads"}
        log(f"[bench] oracle: {reps} runs in {ct:.1f} s, {reps * T / ct:.0f} tokens/s "
            f"on {used} threads")

    rec = {"metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "single-sequence KDA prefill B=1 T=4096 H=32 dk=dv=128, "
                                  "bf16 q/k/v, fp32 log_alpha/beta/state, chunk 64",
                      "global_batch": 1, "seq_len": T, "heads": H, "head_dim": dk,
                      "parallelism": "single GPU"},
           "roofline": roofline, "path": path, "decode": decode, "options": options,
           "cpu_baseline": cpu}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
