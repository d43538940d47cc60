#!/usr/bin/env python3
"""Benchmark of the KDA operator on one MI355X.

Timed step (the headline): one kda_chunk_fwd_split call over the long-context
workload, one 1,048,576-token sequence x 32 heads, dk = dv = 128, chunk 64, bf16
q/k/v, fp32 log-decay/beta/o/hT (seeded synthetic inputs already resident in HBM).
`value` is tokens/s of that call.  Before the warm-up the same call runs for
--settle-ms so that clocks have settled; then --warmup untimed calls and exactly
--steps timed calls between two synchronisations.  Its roofline (HBM-bound) and the
fp64 CPU oracle on the workload's two seeded heads (cpu_baseline) go on the line,
with the max-error/RMS of o and hT on those heads.

The other workloads are legs under "legs", each timed with HIP events on the launch
stream, with its own roofline or bandwidth, its error against the oracle on a seeded
slice, and the oracle's own time on the host: the Kimi-Linear-shaped layer (fused,
with 512-token checkpoints, and split), the tiny fp32 case, the varlen packed batch (fused, split and the
shape-chosen path of kda_chunk_fwd_auto), the long-context sequence with 4 heads (the
split path's segment-parallel state pass), the decode / replay state update (1 and 8
tokens) and replay + verify, the backward pass, and the long-context sequence through the
fused kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                       [--legs all|headline] [--no-cpu-baseline] [--copy-calibration]
Prints exactly one JSON line on stdout.  --copy-calibration adds three launches of a
plain elementwise copy of known size (1 GiB read, 1 GiB written) after the timed
region, so that hardware byte counters (FETCH_SIZE / WRITE_SIZE) taken over the
same run can be scaled to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix cores, TFLOP/s
METRIC = "KDA chunked-fwd tokens/s (H=32,d=128) + MFMA util; decode state-update GB/s"
BF16_TOL, F32_TOL = 2e-2, 1e-4

# Algorithmic model of one chunked-forward token-head (dk = dv = d = 128, chunk C = 64):
# bytes: q, k, v bf16 (3 x 256) + log_alpha fp32 (512) + beta fp32 (4) + o fp32 (512)
BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 512
# flops: 6 d^2 for the state products (W S, Qg S, Kd^T U) + C (3 dk + 2 dv) for the
# lower-triangular intra-chunk products (A, M, W, Ut, M U); the UT inverse is not counted.
FLOPS_PER_TOKEN_HEAD = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128)
PROFILES = os.path.join(ROOT, "profiles")
PMC_SUMMARY = os.path.join(PROFILES, "chunk_fwd_kimi_linear_layer_pmc.txt")
SQ_SUMMARY = os.path.join(PROFILES, "chunk_fwd_kimi_linear_layer_sq_counters.txt")
LC_PMC_SUMMARY = os.path.join(PROFILES, "chunk_fwd_split_long_context_pmc.txt")
# the chunk kernels' code is fixed by their source and by the compiler flags the build gives them
CHUNK_BUILD_FILES = [os.path.join(ROOT, "kimi_delta_attention_06_amd", "csrc", "kda_chunk.hip"),
                     os.path.join(ROOT, "kimi_delta_attention_06_amd", "build.py")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_value(path, key):
    """A figure from a rocprofv3 counter summary, if it was taken on the current kernel source and build
    flags, else None."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("kernel_build_sha256_16") != build_hash(CHUNK_BUILD_FILES):
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def chunk_alg_bytes(tokens, heads, n_seqs, d=128, h0=False, qkv_bytes=2):
    """Algorithmic HBM bytes of one chunked-forward call: the token rows read and o written once,
    hT written (and h0 read when present) once per (sequence, head)."""
    per = 3 * d * qkv_bytes + 4 * d + 4 + 4 * d
    return tokens * heads * per + n_seqs * heads * d * d * 4 * (2 if h0 else 1)


def time_launches(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per launch


def settle(fn, ms, stream):
    """Runs fn back to back for at least `ms` of wall time (at least once); returns the launch count."""
    import torch
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        if n % 4 == 0 or ms <= 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                return n


def launch_spread(fn, n, stream):
    """Per-launch times (ms) from an event pair around each of n launches: p10, median, p90."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    pick = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return {"p10_ms": round(pick(0.1), 5), "median_ms": round(pick(0.5), 5), "p90_ms": round(pick(0.9), 5),
            "launches": n}


def copy_bandwidth(dev, stream, nbytes=1 << 30):
    """GB/s of a plain device copy (torch copy_ of nbytes fp32: nbytes read + nbytes written)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    ms = time_launches(lambda: dst.copy_(src), 20, 5, stream)
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def copy_calibration(dev, nbytes=1 << 30):
    """Three launches of a plain elementwise copy (y = -x, fp32) of `nbytes` each way."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("copy calibration: 3 launches of neg over %d bytes (reads %d B, writes %d B each)" % (nbytes, nbytes, nbytes))
    del src, dst
    return {"kernel": "elementwise neg (fp32)", "read_bytes_per_launch": nbytes, "write_bytes_per_launch": nbytes}


def cpu_info():
    threads = len(os.sched_getaffinity(0))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, cpu


def errors(x, ref, tol=None, absolute=False):
    """max|err| / RMS(ref) and RMS(err) / RMS(ref) of x (torch or numpy) against the fp64 reference."""
    import numpy as np
    x = x.detach().double().cpu().numpy() if hasattr(x, "detach") else np.asarray(x, dtype=np.float64)
    x = x.reshape(ref.shape)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    d = x - ref
    emax = float(np.abs(d).max()) if ref.size else 0.0
    out = {"max_err_over_rms": round(emax / rms, 6) if rms else 0.0,
           "rms_err_over_rms": round(float(np.sqrt(np.mean(d ** 2))) / rms, 7) if rms else 0.0}
    if absolute:
        out["max_abs_err"] = float("%.3e" % emax)
    if tol is not None:
        out["within_tolerance"] = bool(emax <= tol if absolute else emax <= tol * rms)
    return out


def timed_oracle(fn, *a, **kw):
    t0 = time.perf_counter()
    r = fn(*a, **kw)
    return r, time.perf_counter() - t0


# ---------------------------------------------------------------------------------------------
# the headline: the long-context sequence through the split path
# ---------------------------------------------------------------------------------------------
def headline(args, dev, stream, copy_gbs):
    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda

    lw = kda_inputs.LONG_CONTEXT
    log("generating %s inputs" % lw.name)
    inp = kda_inputs.make_chunk_inputs(lw, device=dev)
    o = torch.empty(lw.total_tokens, lw.n_heads, lw.dv, dtype=torch.float32, device=dev)
    hT = torch.empty(1, lw.n_heads, lw.dk, lw.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(lw.n_seqs, lw.total_tokens, lw.n_heads, lw.dk, lw.dv,
                                                         lw.chunk_size), dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=None,
                            chunk_size=lw.chunk_size, o=o, hT=hT, workspace=ws)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_settle = settle(step, args.settle_ms, stream)
    settle_ms = (time.perf_counter() - t0) * 1e3
    log("settle: %d calls in %.0f ms; timing %s split: %d warmup + %d steps" % (n_settle, settle_ms, lw.name,
                                                                               args.warmup, args.steps))
    t_wall0 = time.perf_counter()
    ms = time_launches(step, args.steps, args.warmup, stream)
    t_wall = time.perf_counter() - t_wall0
    tok_s = lw.total_tokens / (ms * 1e-3)
    alg_bytes = chunk_alg_bytes(lw.total_tokens, lw.n_heads, 1)
    alg_flops = lw.total_tokens * lw.n_heads * FLOPS_PER_TOKEN_HEAD
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12
    n_chunks = -(-lw.seq_len // lw.chunk_size)
    log("%s split: %.3f ms/call, %.2f M tokens/s, %.0f GB/s algorithmic (%.1f%% of HBM peak)"
        % (lw.name, ms, tok_s / 1e6, gbs, 100 * gbs / HBM_PEAK_GBS))
    spread = launch_spread(step, 3, stream)
    res = {
        "ms": ms, "tok_s": tok_s, "wall": t_wall, "settle_ms": settle_ms, "settle_launches": n_settle,
        "config": {"workload": lw.name, "batch": 1, "seq_len": lw.seq_len, "heads": lw.n_heads, "dk": lw.dk,
                   "dv": lw.dv, "chunk": lw.chunk_size, "tokens": lw.total_tokens, "path": "kda_chunk_fwd_split",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": profile_value(LC_PMC_SUMMARY,
                                                                                     "hbm_bytes_per_call"),
                     "kernel": "split path: chunk_fwd_kernel's in-chunk pass over the first chunk range, then "
                               "one launch per range of its pipelined mode (the state pass over range r beside "
                               "the in-chunk pass over range r + 1; 34 ranges growing by 1.10, 64 to 1,552 chunks): "
                               "one call = one step",
                     "algorithmic_bytes_per_launch": alg_bytes, "copy_GB/s": round(copy_gbs, 1),
                     "frac_of_copy": round(gbs / copy_gbs, 4)},
        "mfma": {"algorithmic_tflops": round(tflops, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops_per_launch": alg_flops},
        "launch_spread": spread,
        "us_per_serial_chunk_step": round(ms * 1e3 / n_chunks, 3),
        "workspace_bytes": ws.numel(),
    }
    # the fused kernel on the same inputs (value tiles of 16 columns)
    fused = lambda: kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=None,
                                  chunk_size=lw.chunk_size, o=o, hT=hT)
    f_ms = time_launches(fused, 3, 1, stream)
    f_gbs = alg_bytes / (f_ms * 1e-3) / 1e9
    res["fused_leg"] = {"ms_per_step": round(f_ms, 3), "tokens_per_s": round(lw.total_tokens / (f_ms * 1e-3), 1),
                        "algorithmic_GB/s": round(f_gbs, 1), "frac_of_hbm_peak": round(f_gbs / HBM_PEAK_GBS, 4),
                        "us_per_serial_chunk_step": round(f_ms * 1e3 / n_chunks, 3)}
    log("%s fused: %.3f ms/call" % (lw.name, f_ms))
    step()  # the split path's outputs for the parity check
    torch.cuda.synchronize()
    del ws
    heads = kda_inputs.long_context_oracle_heads()
    hs = torch.as_tensor(heads, device=dev)
    sub = {k_: inp[k_].index_select(1, hs).cpu() for k_ in ("q", "k", "v", "log_alpha", "beta")}
    o_s, h_s = o.index_select(1, hs).cpu(), hT.index_select(1, hs).cpu()
    del inp, o, hT
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        import oracle
        threads, cpu = cpu_info()
        log("oracle on heads %s of %s (%d tokens) on %d threads" % ([int(x) for x in heads], lw.name, lw.total_tokens, threads))
        (o_ref, h_ref), t_or = timed_oracle(oracle.kda_fwd, sub["q"], sub["k"], sub["v"], sub["log_alpha"],
                                            sub["beta"], None, None, n_threads=threads)
        res["parity"] = {"o": errors(o_s, o_ref, BF16_TOL), "hT": errors(h_s, h_ref, BF16_TOL),
                         "tolerance_max_err_over_rms": BF16_TOL,
                         "sample": "heads %s (seeded), all %d tokens" % ([int(x) for x in heads], lw.total_tokens)}
        scale = lw.n_heads / len(heads)
        res["cpu_baseline"] = {
            "value": round(lw.total_tokens / (t_or * scale), 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": "fp64 token-by-token oracle on %d of %d heads (%d tokens each), %.2f s wall on %d threads (%s); "
                      "value extrapolated to all %d heads (x%.0f time)" % (len(heads), lw.n_heads, lw.total_tokens,
                                                                          t_or, threads, cpu, lw.n_heads, scale),
            "measured_s": round(t_or, 3), "heads_measured": len(heads), "extrapolated": True}
        log("oracle: %.2f s; o max err/rms %.4f, hT %.4f" % (t_or, res["parity"]["o"]["max_err_over_rms"],
                                                             res["parity"]["hT"]["max_err_over_rms"]))
    return res


# ---------------------------------------------------------------------------------------------
# legs
# ---------------------------------------------------------------------------------------------
def leg_kimi_linear(args, dev, stream, copy_gbs, legs):
    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda

    w = kda_inputs.KIMI_LINEAR_LAYER
    inp = kda_inputs.make_chunk_inputs(w, device=dev)
    o = torch.empty(w.total_tokens, w.n_heads, w.dv, dtype=torch.float32, device=dev)
    hT = torch.empty(w.n_seqs, w.n_heads, w.dk, w.dv, dtype=torch.float32, device=dev)
    view = lambda x: x.view(w.n_seqs, -1, *x.shape[1:])
    qb, kb, vb, lab, beb = (view(inp[x]) for x in ("q", "k", "v", "log_alpha", "beta"))

    def step():
        kda.chunk_fwd(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size, o=o, hT=hT)

    ms = time_launches(step, 200, 50, stream)
    alg_bytes = chunk_alg_bytes(w.total_tokens, w.n_heads, w.n_seqs)
    alg_flops = w.total_tokens * w.n_heads * FLOPS_PER_TOKEN_HEAD
    gbs, tflops = alg_bytes / (ms * 1e-3) / 1e9, alg_flops / (ms * 1e-3) / 1e12
    leg = {"path": "kda_chunk_fwd (fused)", "ms_per_step": round(ms, 5),
           "tokens_per_s": round(w.total_tokens / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": profile_value(PMC_SUMMARY,
                                                                                        "hbm_bytes_per_launch"),
                        "kernel": "chunk_fwd_kernel<64,128,64,Mixed,bf16>", "algorithmic_bytes_per_launch": alg_bytes,
                        "frac_of_copy": round(gbs / copy_gbs, 4)},
           "mfma": {"algorithmic_tflops": round(tflops, 2), "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": alg_flops,
                    "counter_busy_frac": profile_value(SQ_SUMMARY, "mfma_busy_frac"),
                    "counter_valu_busy_frac": profile_value(SQ_SUMMARY, "valu_busy_frac")},
           "launch_spread": launch_spread(step, 50, stream)}
    log("%s fused: %.4f ms, %.1f M tokens/s, %.1f%% of HBM peak" % (w.name, ms, w.total_tokens / ms / 1e3,
                                                                    100 * gbs / HBM_PEAK_GBS))
    ck_every = 512
    ck = torch.empty(w.total_tokens // ck_every, w.n_heads, w.dk, w.dv, dtype=torch.float32, device=dev)
    cstep = lambda: kda.chunk_fwd_checkpointed(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size,
                                               ckpt_every=ck_every, o=o, hT=hT, ckpt=ck)
    c_ms = time_launches(cstep, 200, 50, stream)
    legs[w.name + " checkpointed"] = {"ckpt_every": ck_every, "ms_per_step": round(c_ms, 5),
                                      "overhead_vs_plain": round(c_ms / ms - 1.0, 4),
                                      "checkpoint_bytes_per_step": ck.numel() * 4}
    del ck
    ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(w.n_seqs, w.total_tokens, w.n_heads, w.dk, w.dv),
                     dtype=torch.uint8, device=dev)
    sstep = lambda: kda.chunk_fwd_split(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size, o=o, hT=hT,
                                        workspace=ws)
    s_ms = time_launches(sstep, 100, 20, stream)
    astep = lambda: kda.chunk_fwd_auto(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size, o=o, hT=hT,
                                       workspace=ws)
    a_ms = time_launches(astep, 100, 20, stream)
    legs[w.name + " split"] = {"ms_per_step": round(s_ms, 5), "tokens_per_s": round(w.total_tokens / (s_ms * 1e-3), 1),
                               "auto_ms_per_step": round(a_ms, 5),
                               "auto_tokens_per_s": round(w.total_tokens / (a_ms * 1e-3), 1)}
    log("%s split: %.4f ms; kda_chunk_fwd_auto %.4f ms" % (w.name, s_ms, a_ms))
    del ws
    # backward on the same inputs
    b_do = torch.randn(w.total_tokens, w.n_heads, w.dv, generator=torch.Generator(device=dev).manual_seed(77),
                       device=dev)
    b_ws = torch.empty(kda.backward_workspace_bytes(w.n_seqs, w.total_tokens, w.n_heads, w.dk, w.dv),
                       dtype=torch.uint8, device=dev)
    bstep = lambda: kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], b_do,
                                 cu_seqlens=inp["cu_seqlens"], workspace=b_ws)
    b_ms = time_launches(bstep, 5, 1, stream)
    legs[w.name + " backward"] = {"ms_per_step": round(b_ms, 3), "tokens_per_s": round(w.total_tokens / (b_ms * 1e-3), 1),
                                  "workspace_bytes": b_ws.numel(),
                                  "kind": "chunkwise fp32 matrix-core reverse mode (kda_bwd)"}
    log("%s backward: %.3f ms" % (w.name, b_ms))
    del b_do, b_ws
    step()
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        import oracle
        threads, _ = cpu_info()
        (o_ref, h_ref), t_or = timed_oracle(oracle.kda_fwd, inp["q"], inp["k"], inp["v"], inp["log_alpha"],
                                            inp["beta"], None, inp["cu_seqlens"], n_threads=threads)
        leg["parity"] = {"o": errors(o, o_ref, BF16_TOL), "hT": errors(hT, h_ref, BF16_TOL),
                         "sample": "all %d tokens x %d heads" % (w.total_tokens, w.n_heads)}
        leg["cpu_oracle"] = {"seconds": round(t_or, 3), "tokens_per_s": round(w.total_tokens / t_or, 1),
                             "threads": threads, "sample": "whole workload"}
    legs[w.name] = leg


def leg_chunk_other(args, dev, stream, legs):
    """tiny fp32 (256 tokens x 2 heads x 64, chunk 16) and varlen packed (32,768 tokens, 8 sequences)."""
    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda

    for ow in (kda_inputs.TINY_FP32, kda_inputs.VARLEN_PACKED):
        inp = kda_inputs.make_chunk_inputs(ow, device=dev)
        o = torch.empty(ow.total_tokens, ow.n_heads, ow.dv, dtype=torch.float32, device=dev)
        hT = torch.empty(ow.n_seqs, ow.n_heads, ow.dk, ow.dv, dtype=torch.float32, device=dev)
        step = lambda: kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                                     cu_seqlens=inp["cu_seqlens"], chunk_size=ow.chunk_size, o=o, hT=hT)
        ms = time_launches(step, 100, 20, stream)
        qb = inp["q"].element_size()
        alg = chunk_alg_bytes(ow.total_tokens, ow.n_heads, ow.n_seqs, ow.dk, inp["h0"] is not None, qb)
        leg = {"ms_per_step": round(ms, 5), "tokens_per_s": round(ow.total_tokens / (ms * 1e-3), 1),
               "algorithmic_GB/s": round(alg / (ms * 1e-3) / 1e9, 1),
               "frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if ow.dtype == torch.bfloat16:
            ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(ow.n_seqs, ow.total_tokens, ow.n_heads, ow.dk,
                                                                 ow.dv), dtype=torch.uint8, device=dev)
            sstep = lambda: kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                                h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=ow.chunk_size,
                                                o=o, hT=hT, workspace=ws)
            leg["split_ms_per_step"] = round(time_launches(sstep, 100, 20, stream), 5)
            astep = lambda: kda.chunk_fwd_auto(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                               h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=ow.chunk_size,
                                               o=o, hT=hT, workspace=ws)
            a_ms = time_launches(astep, 100, 20, stream)
            leg["auto_ms_per_step"] = round(a_ms, 5)
            leg["auto_tokens_per_s"] = round(ow.total_tokens / (a_ms * 1e-3), 1)
            del ws
        step()
        torch.cuda.synchronize()
        log("%s: %.4f ms" % (ow.name, ms))
        if not args.no_cpu_baseline:
            import oracle
            threads, _ = cpu_info()
            (o_ref, h_ref), t_or = timed_oracle(oracle.kda_fwd, inp["q"], inp["k"], inp["v"], inp["log_alpha"],
                                                inp["beta"], inp["h0"], inp["cu_seqlens"], n_threads=threads)
            fp32 = ow.dtype == torch.float32
            tol = F32_TOL if fp32 else BF16_TOL
            leg["parity"] = {"o": errors(o, o_ref, tol, absolute=fp32), "hT": errors(hT, h_ref, tol, absolute=fp32),
                             "sample": "whole workload"}
            leg["cpu_oracle"] = {"seconds": round(t_or, 4), "tokens_per_s": round(ow.total_tokens / t_or, 1),
                                 "threads": threads, "sample": "whole workload"}
        legs[ow.name] = leg
        del inp, o, hT


def leg_long_context_few_heads(args, dev, stream, legs):
    """The 1M-token sequence with 4 heads through kda_chunk_fwd_split: few chains, so its state pass
    runs over segments in parallel (maps, scan, rerun); head 0 against the oracle."""
    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda
    w = kda_inputs.LONG_CONTEXT_4H
    inp = kda_inputs.make_chunk_inputs(w, device=dev)
    o = torch.empty(w.total_tokens, w.n_heads, w.dv, device=dev)
    hT = torch.empty(w.n_seqs, w.n_heads, w.dk, w.dv, device=dev)
    ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(w.n_seqs, w.total_tokens, w.n_heads, w.dk, w.dv,
                                                         w.chunk_size),
                     dtype=torch.uint8, device=dev)
    step = lambda: kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=None,
                                       chunk_size=w.chunk_size, o=o, hT=hT, workspace=ws)
    ms = time_launches(step, 5, 2, stream)
    leg = {"ms_per_step": round(ms, 3), "tokens_per_s": round(w.total_tokens / (ms * 1e-3), 1),
           "heads": w.n_heads, "path": "kda_chunk_fwd_split (segmented state pass)"}
    log("%s: %.3f ms/call" % (w.name, ms))
    step()
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        import oracle
        threads, _ = cpu_info()
        sub = {k_: inp[k_][:, :1].cpu() for k_ in ("q", "k", "v", "log_alpha", "beta")}
        (o_ref, h_ref), t_or = timed_oracle(oracle.kda_fwd, sub["q"], sub["k"], sub["v"], sub["log_alpha"],
                                            sub["beta"], None, None, n_threads=threads)
        leg["parity"] = {"o": errors(o[:, :1].cpu(), o_ref, BF16_TOL), "hT": errors(hT[:, :1].cpu(), h_ref, BF16_TOL),
                         "sample": "head 0, all %d tokens" % w.total_tokens}
    legs[w.name] = leg
    del inp, o, hT, ws
    torch.cuda.empty_cache()


def leg_decode(args, dev, stream, copy_gbs, legs):
    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda

    dw = kda_inputs.DECODE_256x32
    state_bytes = dw.n_seqs * dw.n_heads * dw.dk * dw.dv * 4
    for n_tok in (1, 8):
        d = kda_inputs.make_decode_inputs(dw, n_tok, device=dev)
        S0 = d["S"].clone()
        d_o = torch.empty(dw.n_seqs, n_tok, dw.n_heads, dw.dv, dtype=torch.float32, device=dev)
        dstep = lambda: kda.recurrent_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S"], o=d_o)
        d_ms = time_launches(dstep, max(args.steps, 100), 50, stream)
        spread = launch_spread(dstep, 50, stream)
        d_bytes = 2 * state_bytes + dw.n_seqs * n_tok * dw.n_heads * BYTES_PER_TOKEN_HEAD
        d_gbs = d_bytes / (d_ms * 1e-3) / 1e9
        leg = {"ms_per_step": round(d_ms, 5), "GB/s": round(d_gbs, 1), "frac_of_hbm_peak": round(d_gbs / HBM_PEAK_GBS, 4),
               "frac_of_copy": round(d_gbs / copy_gbs, 4), "tokens_per_s": round(dw.n_seqs * n_tok / (d_ms * 1e-3), 1),
               "launch_spread": spread, "bytes_per_step": d_bytes}
        log("recurrent_step n=%d: %.4f ms, %.0f GB/s (%.1f%% of peak)" % (n_tok, d_ms, d_gbs, 100 * d_gbs / HBM_PEAK_GBS))
        if not args.no_cpu_baseline:
            import oracle
            threads, _ = cpu_info()
            d["S"].copy_(S0)
            kda.recurrent_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S"], o=d_o)
            torch.cuda.synchronize()
            (o_ref, S_ref), t_or = timed_oracle(oracle.kda_recurrent_step, d["q"], d["k"], d["v"], d["log_alpha"],
                                                d["beta"], S0, n_threads=threads)
            leg["parity"] = {"o": errors(d_o, o_ref, BF16_TOL), "S": errors(d["S"], S_ref, BF16_TOL),
                             "sample": "all %d sequences x %d heads, one step from the seeded state" % (dw.n_seqs,
                                                                                                       dw.n_heads)}
            leg["cpu_oracle"] = {"seconds": round(t_or, 4), "tokens_per_s": round(dw.n_seqs * n_tok / t_or, 1),
                                 "threads": threads, "sample": "one step, all sequences and heads"}
        legs["%s n%d" % (dw.name, n_tok)] = leg
        del d, d_o, S0
    # replay + verify: 8 tokens, per-sequence commit counts drawn uniformly from 0..8 (seeded)
    v = kda_inputs.make_decode_inputs(dw, 8, device=dev)
    gen = torch.Generator().manual_seed(1005 + 7)
    n_commit = torch.randint(0, 9, (dw.n_seqs,), generator=gen, dtype=torch.int32).to(dev)
    v_o = torch.empty(dw.n_seqs, 8, dw.n_heads, dw.dv, dtype=torch.float32, device=dev)
    vstep = lambda: kda.recurrent_verify(v["q"], v["k"], v["v"], v["log_alpha"], v["beta"], v["S"], n_commit, o=v_o)
    v_ms = time_launches(vstep, max(args.steps, 100), 50, stream)
    n_writing = int((n_commit > 0).sum().item())
    v_bytes = (dw.n_seqs + n_writing) * dw.n_heads * dw.dk * dw.dv * 4 + dw.n_seqs * 8 * dw.n_heads * BYTES_PER_TOKEN_HEAD
    v_gbs = v_bytes / (v_ms * 1e-3) / 1e9
    legs[dw.name + " verify n8"] = {"ms_per_step": round(v_ms, 5), "GB/s": round(v_gbs, 1),
                                    "frac_of_hbm_peak": round(v_gbs / HBM_PEAK_GBS, 4),
                                    "frac_of_copy": round(v_gbs / copy_gbs, 4), "sequences_committing": n_writing,
                                    "bytes_per_step": v_bytes}
    log("recurrent_verify n=8 (%d of %d commit): %.4f ms, %.0f GB/s" % (n_writing, dw.n_seqs, v_ms, v_gbs))
    del v, v_o


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=400.0)
    ap.add_argument("--legs", choices=("all", "headline"), default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    copy_gbs = copy_bandwidth(dev, stream)
    log("device copy (1 GiB each way): %.0f GB/s" % copy_gbs)

    h = headline(args, dev, stream, copy_gbs)
    legs = {"long-context-1m-bf16 fused": h.pop("fused_leg")}
    if args.legs == "all":
        leg_kimi_linear(args, dev, stream, copy_gbs, legs)
        leg_chunk_other(args, dev, stream, legs)
        leg_long_context_few_heads(args, dev, stream, legs)
        leg_decode(args, dev, stream, copy_gbs, legs)

    result = {
        "metric": METRIC,
        "value": round(h["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": h["config"],
        "settle_ms": round(h["settle_ms"], 1),
        "settle_launches": h["settle_launches"],
        "roofline": h["roofline"],
        "mfma": h["mfma"],
        "launch_spread": h["launch_spread"],
        "us_per_serial_chunk_step": h["us_per_serial_chunk_step"],
        "workspace_bytes": h["workspace_bytes"],
        "wall_s_timed_region": round(h["wall"], 3),
        "legs": legs,
    }
    for key in ("parity", "cpu_baseline"):
        if key in h:
            result[key] = h[key]
    if args.copy_calibration:
        result["copy_calibration"] = copy_calibration(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
