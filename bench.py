#!/usr/bin/env python3
"""Benchmark of the block-diffusion decoding step's hot path on one MI355X.

One step = one pass of the hot path over one batch of the batched-serving workload
(B=32 sequences, block S=16, Hq=32 query heads on Hkv=2 KV heads, head dim 128, context
lengths U[1024,8192] in storage padded to 8192, bf16): the denoiser block attention over
[context KV ; block KV] (tt_block_denoise_attn) followed by the gamma=0.8 confidence commit
over logits[32,16,131072] (tt_commit). Inputs are seeded synthetic data resident in HBM
before timing; the context KV and the logits rotate over several copies so that the
256 MB last-level cache cannot serve them.

Prints ONE JSON line on stdout. The metric is denoise-attention blocks per second (one
block = one sequence's S-query block through one attention layer) together with the
context-KV stream's achieved HBM bandwidth against the 8 TB/s peak.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "denoise-attn blocks/sec + context-KV HBM GB/s (% peak), S=16 ctx 8K bf16"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(x) -> float:
    n = x.ctx_len.astype(np.int64) + x.S
    return float(4 * x.S * x.Hq * x.D * int(n.sum()))


PROFILE_MD = os.path.join(ROOT, "profiles", "kernels_b32_s16_ctx8k_bf16.md")


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("attn_mfma.hip", "tt_internal.h"):
        with open(os.path.join(ROOT, "block_diffusion_lm_tt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by a plain copy's reading), or None when that summary was taken
    on another version of the kernel source than the one built here."""
    try:
        text = open(PROFILE_MD).read()
    except OSError:
        return None
    import re
    m = re.search(r"attention source sha256\[:16\][^`]*`([0-9a-f]+)`", text)
    t = re.search(kernel + r" traffic_bytes_per_launch: (\d+)", text)
    if not m or not t or m.group(1) != attn_source_hash():
        return None
    return int(t.group(1))


def profiled_avg_us(kernel: str):
    """The kernel's average duration in the committed rocprofv3 kernel-trace summary, when
    that summary was taken on the kernel source built here (else None)."""
    try:
        text = open(PROFILE_MD).read()
    except OSError:
        return None
    import re
    m = re.search(r"attention source sha256\[:16\][^`]*`([0-9a-f]+)`", text)
    t = re.search(r"\| " + kernel + r" \| \d+ \| ([0-9.]+) \|", text)
    if not m or not t or m.group(1) != attn_source_hash():
        return None
    return float(t.group(1))


def cpu_baseline(w, budget_s: float) -> dict:
    """The fp64 oracle as it stands, on this host, on a bounded sample of the workload."""
    from oracle import ttref_block_denoise_attn, ttref_threads
    x = w.attn()
    done, t_total, ctx_sum = 0, 0.0, 0
    # sequences in batch order, pass after pass, until the budget of CPU time is spent
    while t_total < budget_s:
        for b in range(x.B):
            xb = (x.q[b:b + 1], x.k_blk[b:b + 1], x.v_blk[b:b + 1], x.k_ctx[b:b + 1], x.v_ctx[b:b + 1],
                  x.ctx_len[b:b + 1].copy())
            t0 = time.perf_counter()
            ttref_block_denoise_attn(1, x.S, x.Hq, x.Hkv, x.D, x.Lmax, x.dtype, *xb)
            t_total += time.perf_counter() - t0
            done += 1
            ctx_sum += int(x.ctx_len[b])
            if t_total >= budget_s:
                break
    # scale: blocks/s over the sampled sequences, weighted to the full batch's mean context
    full_mean = float(x.ctx_len.mean()) + x.S
    samp_mean = ctx_sum / done + x.S
    rate = done / t_total * (samp_mean / full_mean)
    # the commit's oracle on the same workload's logits (one pass over the masked rows)
    from oracle import ttref_commit
    c = w.commit()
    t0 = time.perf_counter()
    ttref_commit(c.B, c.S, c.V, c.dtype, c.logits, c.mask, c.gamma)
    t_commit = time.perf_counter() - t0
    return {"value": rate, "unit": "blocks/s", "cores": ttref_threads(), "kind": "oracle",
            "sample": f"{done} sequence blocks of the timed workload ({done / x.B:.1f} passes over its "
                      f"{x.B} sequences, sum ctx_len {ctx_sum}), {t_total:.1f} s, rate rescaled to the "
                      f"batch's mean context length",
            "host_cpu_count": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "commit_pass_s": t_commit, "commit_masked_rows": int(c.mask.sum()),
            "single_thread_blocks_per_s": single_thread_rate(x)}


def single_thread_rate(x) -> float:
    """The attention oracle on one thread (a child process started with OMP_NUM_THREADS=1):
    the batch's first sequence, rescaled to the batch's mean context length."""
    import subprocess
    b = 0
    code = ("import sys, time; sys.path.insert(0, %r)\n"
            "from block_diffusion_lm_tt_amd import workloads as W\n"
            "from oracle import ttref_block_denoise_attn\n"
            "x = W.WORKLOADS[%d].attn(B=%d)\n"
            "t0 = time.perf_counter()\n"
            "ttref_block_denoise_attn(1, x.S, x.Hq, x.Hkv, x.D, x.Lmax, x.dtype, x.q[%d:%d], x.k_blk[%d:%d], "
            "x.v_blk[%d:%d], x.k_ctx[%d:%d], x.v_ctx[%d:%d], x.ctx_len[%d:%d].copy())\n"
            "print(time.perf_counter() - t0)\n") % (ROOT, 3, b + 1, b, b + 1, b, b + 1, b, b + 1, b, b + 1,
                                                      b, b + 1, b, b + 1)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return float("nan")
    t = float(r.stdout.strip().splitlines()[-1])
    return (float(x.ctx_len[b]) + x.S) / (float(x.ctx_len.mean()) + x.S) / t


def loop_bench(w, args, torch, tt, TZ, W):
    """Block loop (the block-loop workload): per block, T denoising steps; each step runs
    tt_block_denoise_attn on every layer (its own context KV, block Q/K/V drawn per
    (step, layer)) and then tt_commit on that step's logits; the still-masked set shrinks
    by the committed positions, and the last step commits whatever is left (the end of a
    block) and every layer's context cache takes the block's rows (tt_ctx_append, the last
    layer bumping ctx_len). Each block starts from the workload's context lengths again (the
    caches have S spare rows past Lmax for the update). Reported per gamma: blocks/s = B /
    (time of the T steps and the cache update) and the positions committed at each step.
    Inputs are generated and copied to HBM before timing."""
    dev = torch.device("cuda:0")
    T, L = w.steps, w.layers
    log(f"[loop] generating workload {w.cid}: {w.name}")
    ctx0 = torch.from_numpy(w.ctx_lens()).to(dev)
    ctx = ctx0.clone()
    kcs, vcs = [], []
    for l in range(L):
        x = w.attn(step=0, layer=l)
        _, _, _, kc, vc, _ = TZ.attn_to_device(x, dev)
        # S spare rows past Lmax: room for the committed block's rows
        kb = torch.empty((w.B, w.Lmax + w.S, w.Hkv, w.D), dtype=kc.dtype, device=dev)
        vb = torch.empty_like(kb)
        kb[:, :w.Lmax].copy_(kc)
        vb[:, :w.Lmax].copy_(vc)
        kcs.append(kb)
        vcs.append(vb)
        del x, kc, vc
    qkv = [[tuple(TZ.to_torch(a, w.dtype, dev) for a in w.block_qkv(t, l)) for l in range(L)]
           for t in range(T)]
    logits = [TZ.commit_to_device(w.commit(step=t), dev)[0] for t in range(T)]
    out = torch.empty_like(qkv[0][0][0])
    dt = 1 if w.dtype == W.BF16 else 0
    ws_a = torch.empty(max(1, tt.tt_block_denoise_attn_workspace(w.B, w.S, w.Hq, w.Hkv, w.D, w.Lmax + w.S, dt)),
                       dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, tt.tt_commit_workspace(w.B, w.S, w.V, dt)), dtype=torch.uint8, device=dev)
    tok = torch.empty((w.B, w.S), dtype=torch.int32, device=dev)
    com = torch.empty((w.B, w.S), dtype=torch.uint8, device=dev)
    mask = torch.empty((w.B, w.S), dtype=torch.uint8, device=dev)
    counts = torch.zeros((T,), dtype=torch.int64, device=dev)
    ones = torch.ones((w.B, w.S), dtype=torch.uint8, device=dev)

    def block(gamma: float):
        mask.copy_(ones)
        ctx.copy_(ctx0)
        for t in range(T):
            for l in range(L):
                q, kb, vb = qkv[t][l]
                tt.tt_block_denoise_attn(q, kb, vb, kcs[l], vcs[l], ctx, out=out, workspace=ws_a)
            tt.tt_commit(logits[t], mask, gamma, token_id=tok, committed=com, workspace=ws_c,
                         want_conf=False)
            if t == T - 1:
                com.copy_(mask)  # end of the block: every remaining masked position commits
            counts[t] += com.sum()
            mask.sub_(com)  # committed positions are masked ones: mask & ~committed
        # the committed block's rows enter every layer's context cache (stand-in rows: the
        # last step's block K/V of that layer); the last layer bumps ctx_len
        for l in range(L):
            _, kb, vb = qkv[T - 1][l]
            tt.tt_ctx_append(kb, vb, kcs[l], vcs[l], ctx, bump=(l == L - 1))

    results = []
    reps = max(1, args.steps // 10)
    for gamma in (0.5, 0.8, 0.95):
        for _ in range(max(1, args.warmup // 10)):
            block(gamma)
        torch.cuda.synchronize()
        counts.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            block(gamma)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        per_step = (counts.double() / reps / w.B).tolist()
        results.append({"gamma": gamma, "blocks_per_s": w.B / (ms * 1e-3), "ms_per_block": ms,
                        "tokens_per_step_per_sequence": per_step,
                        "threshold_commits_per_sequence": sum(per_step[:-1]),
                        "end_of_block_commits_per_sequence": per_step[-1]})
        log(f"[loop] gamma {gamma}: {ms:.3f} ms per block of {T} steps x {L} layers, "
            f"{w.B / (ms * 1e-3):.1f} blocks/s, committed per step per sequence {per_step}")
    # the cache update alone: L layer calls, timed back-to-back
    reps_a = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps_a):
        ctx.copy_(ctx0)
        for l in range(L):
            _, kb, vb = qkv[T - 1][l]
            tt.tt_ctx_append(kb, vb, kcs[l], vcs[l], ctx, bump=(l == L - 1))
    e1.record()
    torch.cuda.synchronize()
    append_us = e0.elapsed_time(e1) * 1e3 / (reps_a * L)
    append_bytes = 2 * 2 * w.B * w.S * w.Hkv * w.D * (2 if w.dtype == W.BF16 else 4)  # read + write, K and V
    log(f"[loop] context cache update: {append_us:.1f} us per layer ({append_bytes / append_us / 1e3:.1f} GB/s)")
    attn_flop = 4.0 * w.S * w.Hq * w.D * float((w.ctx_lens().astype(np.int64) + w.S).sum()) * L * T
    res = {"metric": "block-loop blocks/s and tokens committed per step", "unit": "blocks/s",
           "value": results[1]["blocks_per_s"], "n_gpus": 1, "higher_is_better": True,
           "dtype": "bf16", "data": "synthetic (seeded)",
           "config": {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                      "ctx_len": int(w.ctx_lens()[0]), "layers": L, "steps": T, "V": w.V,
                      "reps": reps},
           "attn_mfma_TFLOPs_gamma_0.8": attn_flop / (results[1]["ms_per_block"] * 1e-3) / 1e12,
           "ctx_append_us_per_layer": append_us,
           "ctx_append_GBps": append_bytes / append_us / 1e3,
           "sweep": results}
    print(json.dumps(res), flush=True)


def stream_read_ceiling(torch, dev) -> float:
    """A streaming read measured in the same run: a library reduction over 2 GiB of fp32
    (read once, a scalar written), best of five, in GB/s."""
    x = torch.ones((1 << 29,), dtype=torch.float32, device=dev)
    best = 0.0
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        x.sum()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x
    return best


def copy_probe(args, torch, dev):
    """A plain device-to-device copy of known size inside the profiled process (the reading
    that calibrates the FETCH_SIZE / WRITE_SIZE counters)."""
    if not args.copy_probe_mib:
        return
    n = args.copy_probe_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: {args.copy_probe_mib} MiB device-to-device copy x3")


def lmhead_bench(args, torch, tt, TZ, W):
    """The LM head fused with the commit (tt_lmhead_commit) on the batched-serving commit
    workload's positions: B=32, S=16, 4..16 masked positions per sequence, V=131072, with
    d_model K = Hq * D = 4096; hidden states N(0,1), head rows N(0, 3/sqrt(K)) (logits of
    standard deviation about 3) and token peaks of +8..+14 at 60% of the positions. Timed
    beside it: the unfused pair a plain pipeline would run (the head as one library GEMM over
    all B*S positions writing bf16 logits, then tt_commit), and the library GEMM over the
    masked rows alone. Prints one JSON line (an extra line, not the headline)."""
    dev = torch.device("cuda:0")
    w3 = W.WORKLOADS[3]
    K = w3.Hq * w3.D
    log(f"[lmhead] generating B={w3.B} S={w3.S} K={K} V={w3.V}")
    x = W.make_lmhead(w3.B, w3.S, K, w3.V, seed=w3.seed, gamma=w3.gamma,
                      mask=W.random_mask(w3.B, w3.S, 4, 16, seed=w3.seed),
                      peaks={"p": 0.6, "low": 8.0, "high": 14.0})
    h, wt, mk = TZ.lmhead_to_device(x, dev)
    R = int(x.mask.sum())
    ws = torch.empty(tt.tt_lmhead_commit_workspace(x.B, x.S, K, x.V), dtype=torch.uint8, device=dev)
    tok = torch.empty((x.B, x.S), dtype=torch.int32, device=dev)
    com = torch.empty((x.B, x.S), dtype=torch.uint8, device=dev)
    conf = torch.empty((x.B, x.S), dtype=torch.float32, device=dev)

    def fused():
        tt.tt_lmhead_commit(h, wt, mk, x.gamma, token_id=tok, committed=com, conf=conf, workspace=ws)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    reps = max(5, args.steps // 2)
    for _ in range(max(2, args.warmup // 2)):
        fused()
    tt.profile_enable(True)
    tt.profile_reset()
    t_events = timed(fused, reps)
    prof = tt.profile_read()
    tt.profile_enable(False)
    t_reduce = prof["lm_reduce_ms"] / max(1, prof["lm_calls"]) * 1e-3
    t_call = timed(fused, reps)

    h2 = h.reshape(-1, K)
    idx = torch.from_numpy(np.nonzero(x.mask.reshape(-1))[0]).to(dev)
    hm = h2.index_select(0, idx).contiguous()
    ws_c = torch.empty(tt.tt_commit_workspace(x.B, x.S, x.V, 1), dtype=torch.uint8, device=dev)
    tok2, com2 = torch.empty_like(tok), torch.empty_like(com)

    def unfused():
        lg = torch.nn.functional.linear(h2, wt).reshape(x.B, x.S, x.V)
        tt.tt_commit(lg, mk, x.gamma, token_id=tok2, committed=com2, want_conf=False, workspace=ws_c)

    def gemm_masked():
        torch.nn.functional.linear(hm, wt)

    for _ in range(2):
        unfused()
        gemm_masked()
    t_unfused = timed(unfused, reps)
    t_gemm = timed(gemm_masked, reps)
    copy_probe(args, torch, dev)
    mb = mk.bool()
    agree = float((tok[mb] == tok2[mb]).double().mean().item()) if R else 1.0  # bf16 logits round
    log(f"[lmhead] fused {t_call*1e6:.1f} us/call (kernel {t_reduce*1e6:.1f} us), unfused "
        f"{t_unfused*1e6:.1f} us, library GEMM over the {R} masked rows {t_gemm*1e6:.1f} us; "
        f"tokens equal to the unfused pair (bf16 logits) at {100 * agree:.1f}% of masked positions")

    wbytes = x.V * K * 2
    alg_bytes = wbytes + R * K * 2
    flops = 2.0 * R * x.V * K
    gbs = alg_bytes / t_reduce / 1e9
    tfl = flops / t_reduce / 1e12
    bound = "hbm" if gbs / HBM_PEAK_GBS >= tfl / MFMA_BF16_PEAK_TFLOPS else "mfma"
    roof = ({"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
            if bound == "hbm" else
            {"bound": "mfma", "achieved": tfl, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": tfl / MFMA_BF16_PEAK_TFLOPS})
    roof.update({"kernel": "lmhead_reduce_kernel", "traffic": None, "avg_us": t_reduce * 1e6,
                 "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flop_per_launch": flops,
                 "hbm_frac": gbs / HBM_PEAK_GBS, "mfma_frac": tfl / MFMA_BF16_PEAK_TFLOPS})
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ttref_lmhead_commit, ttref_threads
        done, t_total, b = 0, 0.0, 0
        budget = min(args.cpu_budget, 15.0)
        while t_total < budget and b < x.B:
            sub = (np.ascontiguousarray(x.hidden[b:b + 1]), np.ascontiguousarray(x.mask[b:b + 1]))
            t0 = time.perf_counter()
            ttref_lmhead_commit(1, x.S, K, x.V, sub[0], x.weight, sub[1], x.gamma)
            t_total += time.perf_counter() - t0
            done += int(x.mask[b].sum())
            b += 1
        cpu = {"value": done / t_total, "unit": "masked positions/s", "cores": ttref_threads(),
               "kind": "oracle",
               "sample": f"the first {b} sequences of the batch ({done} masked positions), {t_total:.1f} s"}
        log(f"[lmhead] cpu baseline {cpu['value']:.2f} positions/s on {cpu['cores']} threads")
    res = {"metric": "fused LM head + commit: masked positions decided per second", "unit": "positions/s",
           "value": R / t_call, "n_gpus": 1, "steps": reps, "warmup": max(2, args.warmup // 2),
           "ms_per_step": t_call * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic (seeded; N(0,1) hidden states, N(0,3/sqrt(K)) head rows, "
                                    "token peaks)",
           "config": {"workload": f"LM head + commit behind {w3.name}", "B": x.B, "S": x.S, "K": K,
                      "V": x.V, "masked_positions": R, "gamma": x.gamma},
           "lmhead_commit_us_per_call": t_call * 1e6,
           "lmhead_commit_us_per_call_with_timing_events": t_events * 1e6,
           "unfused_library_gemm_all_rows_plus_tt_commit_us": t_unfused * 1e6,
           "library_gemm_masked_rows_us": t_gemm * 1e6,
           "token_agreement_with_unfused_bf16_logits": agree,
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload id; the headline line is 3")
    ap.add_argument("--rotate", type=int, default=4, help="copies of context KV / logits cycled")
    ap.add_argument("--block-size", type=int, default=0,
                    help="block positions S of the workload (0: its own; other sizes are extra lines, "
                         "not the headline)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work sampled")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lmhead", action="store_true",
                    help="the fused LM head + commit line instead (an extra line, not the headline)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the hot path has no collective; sequences and KV heads shard across GPUs with no "
              "exchange, so a multi-GPU figure would be N independent copies of this one.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_diffusion_lm_tt_amd as tt
    from block_diffusion_lm_tt_amd import tensors as TZ
    from block_diffusion_lm_tt_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    tt.lib()
    w = W.WORKLOADS[args.config]
    if args.block_size:
        w = dataclasses.replace(w, S=args.block_size, name=f"{w.name} (block size S={args.block_size})")
    if args.lmhead:
        lmhead_bench(args, torch, tt, TZ, W)
        return
    if w.layers != 1:
        loop_bench(w, args, torch, tt, TZ, W)
        return

    log(f"[bench] generating workload {w.cid}: {w.name}")
    x = w.attn()
    c = w.commit()
    q, kb, vb, kc, vc, ctx = TZ.attn_to_device(x, dev)
    lg, mk = TZ.commit_to_device(c, dev)
    R = max(1, args.rotate)
    kcs = [kc] + [kc.clone() for _ in range(R - 1)]
    vcs = [vc] + [vc.clone() for _ in range(R - 1)]
    lgs = [lg] + [lg.clone() for _ in range(R - 1)]
    out = torch.empty_like(q)
    ws_a = torch.empty(max(1, tt.tt_block_denoise_attn_workspace(x.B, x.S, x.Hq, x.Hkv, x.D, x.Lmax,
                                                                 1 if x.dtype == W.BF16 else 0)),
                       dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, tt.tt_commit_workspace(c.B, c.S, c.V, 1 if c.dtype == W.BF16 else 0)),
                       dtype=torch.uint8, device=dev)
    tok = torch.empty((c.B, c.S), dtype=torch.int32, device=dev)
    com = torch.empty((c.B, c.S), dtype=torch.uint8, device=dev)
    conf = torch.empty((c.B, c.S), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(k: int):
        r = k % R
        tt.tt_block_denoise_attn(q, kb, vb, kcs[r], vcs[r], ctx, out=out, workspace=ws_a)
        tt.tt_commit(lgs[r], mk, c.gamma, token_id=tok, committed=com, conf=conf, workspace=ws_c)

    log(f"[bench] warmup {args.warmup}")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    tt.profile_enable(True)
    tt.profile_reset()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = tt.profile_read()
    tt.profile_enable(False)

    # the attention call alone, as a caller sees it (no library timing events): back-to-back
    # calls over the rotated inputs between two events on the launch stream
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record()
    for k in range(K_PLAIN := max(args.steps, 20)):
        r = k % R
        tt.tt_block_denoise_attn(q, kb, vb, kcs[r], vcs[r], ctx, out=out, workspace=ws_a)
    eb.record()
    torch.cuda.synchronize()
    t_attn_plain = ea.elapsed_time(eb) * 1e-3 / K_PLAIN
    # per-call spread: one event between consecutive calls (>= 50 calls)
    n_dist = max(50, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for k in range(n_dist):
        r = k % R
        tt.tt_block_denoise_attn(q, kb, vb, kcs[r], vcs[r], ctx, out=out, workspace=ws_a)
        evs[k + 1].record()
    torch.cuda.synchronize()
    per_call = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(n_dist)])
    p10, p50, p90 = (float(np.percentile(per_call, p)) for p in (10, 50, 90))
    stream_gbs = stream_read_ceiling(torch, dev)

    copy_probe(args, torch, dev)

    K = args.steps
    t_attn = prof["attn_total_ms"] / max(1, prof["attn_calls"]) * 1e-3
    t_main = prof["attn_main_ms"] / max(1, prof["attn_calls"]) * 1e-3
    t_commit = prof["commit_total_ms"] / max(1, prof["commit_calls"]) * 1e-3
    t_reduce = prof["commit_reduce_ms"] / max(1, prof["commit_calls"]) * 1e-3
    kv_bytes = x.ctx_kv_bytes
    blocks_per_s = x.B / t_attn_plain
    gbs_call = kv_bytes / t_attn_plain / 1e9
    gbs_main = kv_bytes / t_main / 1e9
    tflops = attn_flops(x) / t_main / 1e12
    commit_bytes = c.masked_row_bytes
    log(f"[bench] attn {t_attn_plain*1e6:.1f} us/call back-to-back ({t_attn*1e6:.1f} us with timing "
        f"events; main kernel {t_main*1e6:.1f} us), "
        f"commit {t_commit*1e6:.1f} us/call (reduce {t_reduce*1e6:.1f} us), step {wall/K*1e3:.3f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle), budget {args.cpu_budget} s")
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"[bench] cpu baseline {cpu['value']:.3f} blocks/s on {cpu['cores']} threads")

    res = {
        "metric": METRIC,
        "value": blocks_per_s,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded; N(0,1) Q/K/V, N(0,3) logits with planted peaks)",
        "config": {"workload": w.name, "B": x.B, "S": x.S, "Hq": x.Hq, "Hkv": x.Hkv, "D": x.D,
                   "Lmax": x.Lmax, "sum_ctx_len": int(x.ctx_len.sum()), "V": c.V, "gamma": c.gamma,
                   "masked_positions": int(c.mask.sum()), "rotated_copies": R},
        "context_kv_GBps": gbs_call,
        "context_kv_pct_hbm_peak": 100.0 * gbs_call / HBM_PEAK_GBS,
        "hbm_stream_read_GBps_measured": stream_gbs,
        "context_kv_pct_of_measured_stream_read": 100.0 * gbs_call / stream_gbs,
        "attn_us_per_call": t_attn_plain * 1e6,
        "attn_us_per_call_p10_p50_p90": [p10, p50, p90],
        "attn_us_per_call_with_timing_events": t_attn * 1e6,
        "commit_us_per_call": t_commit * 1e6,
        "commit_GBps": commit_bytes / t_commit / 1e9,
        "mfma_TFLOPs": tflops,
        "mfma_pct_bf16_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
        "roofline": {"kernel": "attn_mfma_kernel", "bound": "hbm", "achieved": gbs_main,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs_main / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("attn_mfma_kernel")
                     if args.config == 3 and not args.block_size else None,
                     "avg_us": t_main * 1e6, "algorithmic_bytes_per_launch": kv_bytes,
                     "profiled_avg_us": profiled_avg_us("attn_mfma_kernel")
                     if args.config == 3 and not args.block_size else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
