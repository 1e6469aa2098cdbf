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


PROFILE_MD = "kernels_b32_s16_ctx8k_bf16.md"
ATTN_SOURCES = ("attn_mfma.hip", "tt_internal.h")
LMHEAD_MD = "kernels_lmhead_b32_s16_k4096_v131072.md"
LMHEAD_SOURCES = ("lmhead.hip", "lmhead_exact.hip", "tt_internal.h")
MAMBA_MD = "kernels_mamba2_b32_s16_h128_p64_n128_bf16.md"
MAMBA_SOURCES = ("mamba.hip", "adaln.hip", "tt_internal.h")


def source_hash(files) -> str:
    """First 16 hex digits of the SHA-256 over the given kernel sources, in order (the hash a
    committed profile summary records for the sources it was taken on)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_diffusion_lm_tt_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attn_source_hash() -> str:
    return source_hash(ATTN_SOURCES)


def _profile_field(md: str, label: str, files, pattern: str):
    """The first group of `pattern` in the committed summary profiles/<md>, when its recorded
    `label` source hash equals the hash of `files` as built here (else None: a summary taken
    on another version of the kernel says nothing about this one)."""
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", md)).read()
    except OSError:
        return None
    m = re.search(label + r" sha256\[:16\][^`]*`([0-9a-f]+)`", text)
    t = re.search(pattern, text)
    if not m or not t or m.group(1) != source_hash(files):
        return None
    return t.group(1)


def profiled_traffic(kernel: str, md: str = PROFILE_MD, label: str = "attention source", files=ATTN_SOURCES):
    """HBM bytes per launch of `kernel` from a committed counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by a plain copy's reading), or None (see _profile_field)."""
    v = _profile_field(md, label, files, kernel + r" traffic_bytes_per_launch: (\d+)")
    return None if v is None else int(v)


def profiled_avg_us(kernel: str, md: str = PROFILE_MD, label: str = "attention source", files=ATTN_SOURCES):
    """The kernel's average duration in a committed rocprofv3 kernel-trace summary, or None.
    (The kernel's name in the trace may carry its template argument, e.g. attn_mfma_kernel<true>.)"""
    v = _profile_field(md, label, files, r"\| " + kernel + r"(?:<[^|]*>)? \| \d+ \| ([0-9.]+) \|")
    return None if v is None else float(v)


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
    """Block loop (the block-loop workload, block_diffusion_lm_tt_amd/blockloop.py): per
    block, T denoising steps; each step runs tt_block_denoise_attn on every layer (its own
    context KV, block Q/K/V drawn per (step, layer)) and then tt_commit on that step's
    logits; the still-masked set shrinks by the committed positions, the last step commits
    whatever is left, and every layer's context cache takes the block's rows
    (tt_ctx_append, the last layer bumping ctx_len). Each block starts from the workload's
    context lengths again. Reported per gamma: blocks/s = B / (time of the T steps and the
    cache update), per-block p10/p50/p90 over the timed blocks, and the positions committed
    at each step. Inputs are generated and copied to HBM before timing."""
    from block_diffusion_lm_tt_amd.blockloop import BlockLoop
    dev = torch.device("cuda:0")
    T, L = w.steps, w.layers
    log(f"[loop] generating workload {w.cid}: {w.name}")
    bl = BlockLoop(w, dev)

    results = []
    reps = max(20, args.steps // 2)
    for gamma in (0.5, 0.8, 0.95):
        for _ in range(max(2, args.warmup // 5)):
            bl.run_block(gamma)
        torch.cuda.synchronize()
        bl.counts.zero_()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record()
        for k in range(reps):
            bl.run_block(gamma)
            evs[k + 1].record()
        torch.cuda.synchronize()
        per = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(reps)])
        ms = evs[0].elapsed_time(evs[reps]) / reps
        p10, p50, p90 = (float(np.percentile(per, p)) for p in (10, 50, 90))
        per_step = (bl.counts.double() / reps / w.B).tolist()
        results.append({"gamma": gamma, "blocks_per_s": w.B / (ms * 1e-3), "ms_per_block": ms,
                        "ms_per_block_p10_p50_p90": [p10, p50, p90],
                        "tokens_per_step_per_sequence": per_step,
                        "threshold_commits_per_sequence": sum(per_step[:-1]),
                        "end_of_block_commits_per_sequence": per_step[-1]})
        log(f"[loop] gamma {gamma}: {ms:.3f} ms per block of {T} steps x {L} layers "
            f"(p10/p50/p90 {p10:.3f}/{p50:.3f}/{p90:.3f}), {w.B / (ms * 1e-3):.1f} blocks/s, "
            f"committed per step per sequence {per_step}")
    # the cache update alone: L layer calls, timed back-to-back
    reps_a = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps_a):
        bl.ctx.copy_(bl.ctx0)
        for l in range(L):
            _, kb, vb = bl.qkv[T - 1][l]
            tt.tt_ctx_append(kb, vb, bl.kcs[l], bl.vcs[l], bl.ctx, bump=(l == L - 1))
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
           "attn_mfma_pct_bf16_peak_gamma_0.8":
               100.0 * attn_flop / (results[1]["ms_per_block"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "ctx_append_us_per_layer": append_us,
           "ctx_append_GBps": append_bytes / append_us / 1e3,
           "sweep": results}
    print(json.dumps(res), flush=True)


def stream_read_ceiling(torch, dev) -> dict:
    """Plain HBM streaming reads measured in the same run: the probe kernels of
    block_diffusion_lm_tt_amd/libttprobe.so over 2 GiB -- 16-byte non-temporal loads into
    registers, and 16-byte LDS-DMA copies -- for several grid sizes, best of four each. GB/s
    is the better of the two; both are reported with their grid."""
    import ctypes
    from block_diffusion_lm_tt_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    for fn in (L.ttprobe_stream_read, L.ttprobe_stream_read_lds):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    nbytes = 1 << 31
    x = torch.ones((nbytes,), dtype=torch.uint8, device=dev)
    sink = torch.empty((1 << 15,), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    out = {"bytes": nbytes}
    for name, fn in (("registers", L.ttprobe_stream_read), ("lds_dma", L.ttprobe_stream_read_lds)):
        best, best_grid = 0.0, 0
        for blocks in (1024, 2048, 4096, 8192, 16384):
            for _ in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                rc = fn(x.data_ptr(), nbytes, sink.data_ptr(), blocks, st.cuda_stream)
                e1.record()
                if rc != 0:
                    raise RuntimeError(f"stream-read probe ({name}) failed: {rc}")
                torch.cuda.synchronize()
                gbs = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if gbs > best:
                    best, best_grid = gbs, blocks
        out[name] = {"GBps": best, "workgroups": best_grid}
    out["GBps"] = max(out["registers"]["GBps"], out["lds_dma"]["GBps"])
    log(f"[bench] streaming read ceiling: registers {out['registers']['GBps']:.0f} GB/s "
        f"({out['registers']['workgroups']} workgroups), LDS-DMA {out['lds_dma']['GBps']:.0f} GB/s "
        f"({out['lds_dma']['workgroups']} workgroups)")
    del x, sink
    return out


def mfma_rate(torch, dev) -> float:
    """The matrix cores' bf16 rate measured in the same run: the probe kernel of libttprobe.so
    (v_mfma_f32_32x32x16_bf16 back to back in four independent chains per wave, two waves per
    SIMD on every CU), best of three, in TFLOP/s."""
    import ctypes
    from block_diffusion_lm_tt_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    L.ttprobe_mfma_rate.restype = ctypes.c_int
    L.ttprobe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 512, 20000
    sink = torch.empty((blocks,), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev)
    flop = blocks * 4 * 4 * iters * 32768.0
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if L.ttprobe_mfma_rate(blocks, iters, sink.data_ptr(), st.cuda_stream) != 0:
            raise RuntimeError("mfma-rate probe failed")
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    log(f"[bench] bf16 matrix-core rate: {best:.0f} TFLOP/s")
    return best


def tile_loop_probe(torch, dev) -> dict:
    """The attention tile loop's resources measured on every CU (probes of libttprobe.so, one
    8-wave workgroup per CU): the LDS read rate of the K operand reads (ds_read_b128) and of
    the V^T operand reads (ds_read_b64_tr_b16), in bytes per shader-clock cycle per CU; and the
    cycles per iteration of the matrix/vector core (16 matrix products and one vector phase per
    wave): matrix only, vector only, both in different waves at once, the two-barrier
    ping-pong, the ping-pong with the next tile's operand reads (128 KB per CU), and one wave
    per SIMD carrying both waves' work (64 rows, the same products and vector work per SIMD),
    without and with its next tile's operand reads (64 KB per CU)."""
    import ctypes
    from block_diffusion_lm_tt_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    for f in (L.ttprobe_lds_read, L.ttprobe_tile_core):
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    blocks, iters = 256, 2000
    sink = torch.zeros((blocks * 8 + 1,), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev)

    def run(fn, arg, waves):
        for _ in range(2):  # the second launch is the one read
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if fn(arg, blocks, iters, sink.data_ptr(), st.cuda_stream) != 0:
                raise RuntimeError("tile-loop probe failed")
            e1.record()
            torch.cuda.synchronize()
        cyc = sink[:blocks * 8].view(blocks, 8)[:, waves].mean().item() / iters
        return cyc, e0.elapsed_time(e1) * 1e3 / iters

    out = {}
    for kind, name in ((0, "k_b128"), (1, "v_tr_b64")):
        cyc, us = run(L.ttprobe_lds_read, kind, slice(0, 8))
        out[f"lds_read_{name}_bytes_per_cycle_per_cu"] = 65536 / cyc
    names = ("matrix_only", "vector_only", "both_at_once", "ping_pong", "ping_pong_with_operand_reads",
             "one_wave_per_simd_64_rows", "one_wave_per_simd_64_rows_with_operand_reads")
    waves = (slice(0, 4), slice(4, 8), slice(0, 8), slice(0, 8), slice(0, 8), slice(0, 4), slice(0, 4))
    for mode, name in enumerate(names):
        cyc, us = run(L.ttprobe_tile_core, mode, waves[mode])
        out[f"core_{name}_cycles_per_iteration"] = cyc
        out[f"core_{name}_us_per_iteration"] = us
    log("[bench] tile-loop probe: " + ", ".join(f"{k} {v:.1f}" for k, v in out.items()))
    return out


def stream_read_same_size(torch, dev, nbytes: int) -> dict:
    """The register-streaming probe over exactly `nbytes` (four rotated buffers, so that the
    last-level cache cannot serve them), best over grid sizes of the median of five
    event-timed launches: the practical ceiling for a kernel that reads that many bytes once."""
    import ctypes
    from block_diffusion_lm_tt_amd.build import PROBE_LIB
    L = ctypes.CDLL(PROBE_LIB)
    L.ttprobe_stream_read.restype = ctypes.c_int
    L.ttprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    nb = (int(nbytes) + 255) // 256 * 256
    R = 4
    bufs = [torch.ones((nb,), dtype=torch.uint8, device=dev) for _ in range(R)]
    sink = torch.empty((1 << 15,), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream(dev)
    best, grid = float("inf"), 0
    for blocks in (256, 512, 1024, 2048, 4096, 8192):
        ts = []
        for k in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if L.ttprobe_stream_read(bufs[k % R].data_ptr(), nb, sink.data_ptr(), blocks, st.cuda_stream) != 0:
                raise RuntimeError("stream-read probe failed")
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(ts[1:]))
        if t < best:
            best, grid = t, blocks
    del bufs, sink
    return {"bytes": nb, "us": best * 1e6, "GBps": nb / best / 1e9, "workgroups": grid}


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
    # exact mode: the head-row norm bound once, then the fused call with its fp64 recheck; the
    # number of recomputed rows is read from the workspace (the counter follows the chunk,
    # runner-up, merged, bound, flag and list arrays, each padded to 256 bytes)
    wb = tt.tt_lmhead_weight_bound(wt)
    ws_x = torch.empty(int(tt.lib().tt_lmhead_commit_exact_workspace(x.B, x.S, K, x.V)), dtype=torch.uint8,
                       device=dev)
    tok3, com3 = torch.empty_like(tok), torch.empty_like(com)

    def exact():
        tt.tt_lmhead_commit(h, wt, mk, x.gamma, token_id=tok3, committed=com3, want_conf=False, workspace=ws_x,
                            w_bound=wb)

    for _ in range(2):
        exact()
    t_exact = timed(exact, reps)
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    rows, nvt = x.B * x.S, (x.V + 255) // 256
    off = al(rows * nvt * 16) + al(rows * nvt * 4) + al(rows * 16) + al(rows * 16) + al(rows * 4) + al(rows * 4)
    n_recomputed = int(ws_x[off:off + 4].view(torch.int32).item())
    same_tok = float((tok3[mk.bool()] == tok[mk.bool()]).double().mean().item()) if R else 1.0
    same_dec = bool(torch.equal(com3, com))
    log(f"[lmhead] exact mode {t_exact*1e6:.1f} us/call, {n_recomputed} rows recomputed in fp64; tokens equal to "
        f"the estimate path at {100 * same_tok:.1f}% of masked positions, decisions equal: {same_dec}")
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
    roof.update({"kernel": "lmhead_reduce_kernel",
                 "traffic": profiled_traffic("lmhead_reduce_kernel", LMHEAD_MD, "LM-head source", LMHEAD_SOURCES),
                 "avg_us": t_reduce * 1e6,
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
           "exact_mode_us_per_call": t_exact * 1e6, "exact_mode_rows_recomputed": n_recomputed,
           "exact_mode_tokens_equal_to_estimates": same_tok, "exact_mode_decisions_equal_to_estimates": same_dec,
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


def mamba_bench(args, torch, tt, TZ, W):
    """The denoiser's Mamba-2 scan from the context tower's seeded state (tt_mamba2_seeded_scan)
    at the batched-serving shape: B=32 sequences, block S=16, d_model 4096 expanded twice to 128
    heads of P=64, state size N=128, 8 B/C groups, bf16 activations and an fp32 state; the
    per-step call of a denoising step (the state after the block is not written). Timed beside
    it: the adaLN-single modulation and gated residual at d=4096 over the same B*S positions.
    The seeded states and inputs rotate over several copies so that the last-level cache cannot
    serve them. Prints one JSON line (an extra line, not the headline)."""
    dev = torch.device("cuda:0")
    B, S, H, P, N, G, d = 32, 16, 128, 64, 128, 8, 4096
    log(f"[mamba] generating B={B} S={S} H={H} P={P} N={N} G={G}")
    m = W.make_mamba(B, S, H, P, N, G, W.BF16, seed=1003)
    base = TZ.mamba_to_device(m, dev)
    R = max(1, args.rotate)
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    y = torch.empty_like(base[0])
    h_out = torch.empty_like(base[7])
    a = W.make_adaln(B, S, d, W.BF16, seed=1003)
    ax, af, atm, atab = TZ.adaln_to_device(a, dev)
    asets = [(ax, af)] + [(ax.clone(), af.clone()) for _ in range(R - 1)]
    ay = torch.empty_like(ax)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(reps):
            fn(k)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    scan = lambda k: tt.tt_mamba2_seeded_scan(*sets[k % R], G=G, y=y)  # noqa: E731
    scan_state = lambda k: tt.tt_mamba2_seeded_scan(*sets[k % R], G=G, y=y, h_out=h_out)  # noqa: E731
    modulate = lambda k: tt.tt_adaln_modulate(asets[k % R][0], atm, atab, y=ay)  # noqa: E731
    gate = lambda k: tt.tt_adaln_gate(asets[k % R][0], asets[k % R][1], atm, atab, out=ay)  # noqa: E731
    reps = max(20, args.steps)
    for fn in (scan, scan_state, modulate, gate):
        timed(fn, max(4, args.warmup))
    t_scan = timed(scan, reps)
    t_state = timed(scan_state, reps)
    t_mod = timed(modulate, reps)
    t_gate = timed(gate, reps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for k in range(reps):
        scan(k)
        evs[k + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(reps)])
    p10, p50, p90 = (float(np.percentile(per, p)) for p in (10, 50, 90))

    state_bytes = B * H * P * N * 4
    act = 2  # bf16
    io_bytes = (2 * B * S * H * P * act + 2 * B * S * G * N * act + B * S * H * 4 + 3 * H * 4)
    alg = state_bytes + io_bytes
    gbs = alg / t_scan / 1e9
    flop = 2.0 * B * H * S * P * N  # the readout of the seeded state, the arithmetic bulk
    ad_mod = 2 * B * S * d * act + (B * 3 * d + 3 * d) * 4
    ad_gate = 3 * B * S * d * act + (B * 3 * d + 3 * d) * 4
    stream = stream_read_ceiling(torch, dev)
    same = stream_read_same_size(torch, dev, alg)
    copy_probe(args, torch, dev)
    log(f"[mamba] scan {t_scan*1e6:.1f} us/call (p10/p50/p90 {p10:.1f}/{p50:.1f}/{p90:.1f}; {gbs:.0f} GB/s), "
        f"with the state written {t_state*1e6:.1f} us; adaLN modulate {t_mod*1e6:.1f} us, gate {t_gate*1e6:.1f} us")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ttref_mamba2_scan, ttref_threads
        done, t_total = 0, 0.0
        budget = min(args.cpu_budget, 15.0)
        while t_total < budget:
            t0 = time.perf_counter()
            ttref_mamba2_scan(B, S, H, P, N, G, m.dtype, m.x, m.dt, m.dt_bias, m.A_log, m.Dskip, m.Bm, m.Cm, m.h0,
                              want_state=False)
            t_total += time.perf_counter() - t0
            done += 1
        cpu = {"value": done * B / t_total, "unit": "sequence-layers/s", "cores": ttref_threads(),
               "kind": "oracle", "sample": f"{done} whole-batch scans of the timed shape, {t_total:.1f} s"}
        log(f"[mamba] cpu baseline {cpu['value']:.1f} sequence-layers/s on {cpu['cores']} threads")
    res = {"metric": "denoiser Mamba-2 block scans from the seeded state: sequence-layers per second",
           "unit": "sequence-layers/s", "value": B / t_scan, "n_gpus": 1, "steps": reps,
           "warmup": max(4, args.warmup), "ms_per_step": t_scan * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; N(0,1) inputs, N(0,1/N) B and C, N(0,0.5^2) seeded state)",
           "config": {"workload": "denoiser Mamba-2 layer, batched serving", "B": B, "S": S, "H": H, "P": P,
                      "N": N, "G": G, "d_model": d, "rotated_copies": R},
           "scan_us_per_call": t_scan * 1e6, "scan_us_p10_p50_p90": [p10, p50, p90],
           "scan_with_state_out_us_per_call": t_state * 1e6,
           "scan_with_state_out_GBps": (alg + state_bytes) / t_state / 1e9,
           "adaln_modulate_us_per_call": t_mod * 1e6, "adaln_modulate_GBps": ad_mod / t_mod / 1e9,
           "adaln_gate_us_per_call": t_gate * 1e6, "adaln_gate_GBps": ad_gate / t_gate / 1e9,
           # (bf16 activations with these P and N take the matrix-core scan)
           "roofline": {"kernel": "mamba2_scan_mfma_kernel", "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": profiled_traffic("mamba2_scan_mfma_kernel", MAMBA_MD, "scan source", MAMBA_SOURCES),
                        "avg_us": t_scan * 1e6,
                        "algorithmic_bytes_per_launch": alg, "readout_flop_per_launch": flop,
                        "frac_of_measured_stream_read": gbs / stream["GBps"],
                        "frac_of_same_size_stream_read": same["us"] / (t_scan * 1e6)},
           "hbm_stream_read_probe": stream, "stream_read_same_bytes": same,
           "cpu_baseline": cpu}
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
    ap.add_argument("--mamba", action="store_true",
                    help="the denoiser's Mamba-2 scan + adaLN line instead (an extra line, not the headline)")
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
    if args.mamba:
        mamba_bench(args, torch, tt, TZ, W)
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
    # the commit call alone, the same way (back-to-back over the rotated logits)
    torch.cuda.synchronize()
    ea.record()
    for k in range(K_PLAIN):
        tt.tt_commit(lgs[k % R], mk, c.gamma, token_id=tok, committed=com, conf=conf, workspace=ws_c)
    eb.record()
    torch.cuda.synchronize()
    t_commit_plain = ea.elapsed_time(eb) * 1e-3 / K_PLAIN
    stream = stream_read_ceiling(torch, dev)
    stream_gbs = stream["GBps"]
    same = stream_read_same_size(torch, dev, x.ctx_kv_bytes)
    same_c = stream_read_same_size(torch, dev, c.masked_row_bytes)
    mfma_meas = mfma_rate(torch, dev)
    core = tile_loop_probe(torch, dev)

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
        f"commit {t_commit_plain*1e6:.1f} us/call back-to-back ({t_commit*1e6:.1f} us with timing events; "
        f"reduce {t_reduce*1e6:.1f} us), step {wall/K*1e3:.3f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle), budget {args.cpu_budget} s")
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"[bench] cpu baseline {cpu['value']:.3f} blocks/s on {cpu['cores']} threads")

    res = {
        # the headline's metric name; other workloads and block sizes name their own S, context, dtype
        "metric": METRIC if args.config == 3 and not args.block_size else
        (f"denoise-attn blocks/sec + context-KV HBM GB/s (% peak), S={x.S} ctx {max(1, x.Lmax // 1024)}K "
         f"{'bf16' if x.dtype == W.BF16 else 'f32'}"),
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
        "hbm_stream_read_probe": stream,
        "stream_read_same_bytes_as_context_kv": same,
        "stream_read_same_bytes_as_commit": same_c,
        "context_kv_pct_of_measured_stream_read": 100.0 * gbs_call / stream_gbs,
        "attn_us_per_call": t_attn_plain * 1e6,
        "attn_us_per_call_p10_p50_p90": [p10, p50, p90],
        "attn_us_per_call_with_timing_events": t_attn * 1e6,
        "commit_us_per_call": t_commit_plain * 1e6,
        "commit_GBps": commit_bytes / t_commit_plain / 1e9,
        "commit_us_per_call_with_timing_events": t_commit * 1e6,
        "commit_reduce_us_with_timing_events": t_reduce * 1e6,
        "mfma_TFLOPs": tflops,
        "mfma_pct_bf16_peak": 100.0 * tflops / MFMA_BF16_PEAK_TFLOPS,
        "mfma_bf16_TFLOPs_measured": mfma_meas,
        "mfma_pct_of_measured_rate": 100.0 * tflops / mfma_meas,
        "tile_loop_probe": core,
        "roofline": {"kernel": "attn_mfma_kernel", "bound": "hbm", "achieved": gbs_main,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs_main / HBM_PEAK_GBS,
                     "traffic": profiled_traffic("attn_mfma_kernel")
                     if args.config == 3 and not args.block_size else None,
                     "avg_us": t_main * 1e6, "algorithmic_bytes_per_launch": kv_bytes,
                     "call_achieved": gbs_call, "call_frac": gbs_call / HBM_PEAK_GBS,
                     "call_us": t_attn_plain * 1e6,
                     "frac_of_measured_stream_read": gbs_main / stream_gbs,
                     "frac_of_same_size_stream_read": same["us"] / (t_main * 1e6),
                     "profiled_avg_us": profiled_avg_us("attn_mfma_kernel")
                     if args.config == 3 and not args.block_size else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
