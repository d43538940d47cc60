#!/usr/bin/env python3
"""Benchmark of the KDA operator on one MI355X.

Timed step: one kda_chunk_fwd pass over the Kimi-Linear-shaped KDA layer
(B=4, T=4096, H=32, dk=dv=128, chunk 64, bf16 q/k/v, fp32 gates and state;
seeded synthetic inputs already resident in HBM).  `value` is tokens/s of that
pass (B*T tokens, all 32 heads).  The same pass with state checkpoints every 512
tokens is timed and reported under "checkpointed".  In the same run the decode/replay state update
(256 sequences x 32 heads, fp32 state, 1 and 8 tokens) and the replay + verify
variant (8 tokens, per-sequence commit counts) are timed and reported under
"decode" (HBM GB/s against the 8 TB/s peak); one chunked pass over a single
1M-token sequence x 32 heads is timed, fused and split (kda_chunk_fwd_split), 1 warm-up + 5 timed
launches each, and reported under "long_context"; and the
fp64 CPU oracle is timed on a bounded sample of the chunk workload ("cpu_baseline").
The backward pass (kda_bwd, chunkwise) on the Kimi-Linear layer is timed under "backward", and
the tiny fp32 and varlen packed chunked workloads under "other_workloads".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-long-context] [--copy-calibration]
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

# Algorithmic model of one chunked-forward token-head (dk = dv = d = 128, chunk C = 64):
# bytes: q, k, v bf16 (3 x 256) + log_alpha fp32 (512) + beta fp32 (4) + o fp32 (512)
BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 512
# flops: 6 d^2 for the state products (W S, Qg S, Kd^T U) + C (3 dk + 2 dv) for the
# lower-triangular intra-chunk products (A, M, W, Ut, M U); the UT inverse is not counted.
FLOPS_PER_TOKEN_HEAD = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "chunk_fwd_kimi_linear_layer_pmc.txt")
SQ_SUMMARY = os.path.join(ROOT, "profiles", "chunk_fwd_kimi_linear_layer_sq_counters.txt")
# the chunk kernel's code is fixed by its source and by the compiler flags the build gives it
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


def traffic_from_profile():
    """HBM bytes per launch measured by rocprofv3 counters for the current kernel build, else None."""
    return profile_value(PMC_SUMMARY, "hbm_bytes_per_launch")


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


def cpu_baseline(inp, n_seqs):
    """fp64 oracle on the first `n_seqs` sequences of the workload, all heads (whole sequences)."""
    import oracle
    T = int(sum(inp["lens"][:n_seqs]))
    sl = slice(0, T)
    args = [inp[x][sl].cpu() for x in ("q", "k", "v", "log_alpha", "beta")]
    cu = inp["cu_seqlens"][: n_seqs + 1].cpu()
    nthreads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.kda_fwd(*args, None, cu, n_threads=nthreads)
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(T / dt, 1), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": "fp64 token-by-token oracle on %d of %d sequences (%d tokens x 32 heads), "
                      "%.2f s wall on %d threads (%s); same token count convention as value"
                      % (n_seqs, len(inp["lens"]), T, dt, nthreads, cpu)}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: ~25 ms of warm-up launches (clocks settle) and ~90 ms timed on the chunk kernel
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-long-context", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=4)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import kda_inputs
    import kimi_delta_attention_06_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- chunked forward, Kimi-Linear-shaped layer ----------------
    w = kda_inputs.KIMI_LINEAR_LAYER
    log("generating %s inputs" % w.name)
    inp = kda_inputs.make_chunk_inputs(w, device=dev)
    o = torch.empty(w.total_tokens, w.n_heads, w.dv, dtype=torch.float32, device=dev)
    hT = torch.empty(w.n_seqs, w.n_heads, w.dk, w.dv, dtype=torch.float32, device=dev)

    # fixed-length batch: pass [B, T, H, d] views (no cu_seqlens)
    qb = inp["q"].view(w.n_seqs, -1, w.n_heads, w.dk)
    kb = inp["k"].view(w.n_seqs, -1, w.n_heads, w.dk)
    vb = inp["v"].view(w.n_seqs, -1, w.n_heads, w.dv)
    lab = inp["log_alpha"].view(w.n_seqs, -1, w.n_heads, w.dk)
    beb = inp["beta"].view(w.n_seqs, -1, w.n_heads)

    def step():
        kda.chunk_fwd(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size, o=o, hT=hT)

    log("timing chunk_fwd: %d warmup + %d steps" % (args.warmup, args.steps))
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ms = time_launches(step, args.steps, args.warmup, stream)
    t_wall = time.perf_counter() - t_wall0
    tokens = w.total_tokens
    tok_s = tokens / (ms * 1e-3)
    alg_bytes = tokens * w.n_heads * BYTES_PER_TOKEN_HEAD + w.n_seqs * w.n_heads * w.dk * w.dv * 4
    alg_flops = tokens * w.n_heads * FLOPS_PER_TOKEN_HEAD
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12
    log("chunk_fwd: %.4f ms/launch, %.1f M tokens/s, %.0f GB/s algorithmic, %.1f TFLOP/s algorithmic"
        % (ms, tok_s / 1e6, gbs, tflops))
    spread = launch_spread(step, 50, stream)
    log("chunk_fwd per-launch spread: p10 %.4f, median %.4f, p90 %.4f ms" % (spread["p10_ms"], spread["median_ms"],
                                                                         spread["p90_ms"]))
    copy_gbs = copy_bandwidth(dev, stream)
    log("device copy (1 GiB each way): %.0f GB/s" % copy_gbs)

    # ---------------- the same pass with 512-token state checkpoints ----------------
    ck_every = 512
    ck = torch.empty(tokens // ck_every, w.n_heads, w.dk, w.dv, dtype=torch.float32, device=dev)

    def cstep():
        kda.chunk_fwd_checkpointed(qb, kb, vb, lab, beb, h0=None, chunk_size=w.chunk_size, ckpt_every=ck_every,
                                   o=o, hT=hT, ckpt=ck)

    c_ms = time_launches(cstep, args.steps, args.warmup, stream)
    ck_bytes = ck.numel() * 4
    checkpointed = {"ckpt_every": ck_every, "ms_per_step": round(c_ms, 5),
                    "overhead_vs_plain": round(c_ms / ms - 1.0, 4), "checkpoint_bytes_per_step": ck_bytes,
                    "algorithmic_GB/s": round((alg_bytes + ck_bytes) / (c_ms * 1e-3) / 1e9, 1)}
    log("chunk_fwd_checkpointed (every %d tokens): %.4f ms/launch (%+.1f%%)" % (ck_every, c_ms, 100 * (c_ms / ms - 1)))
    del ck

    # ---------------- decode / replay ----------------
    dw = kda_inputs.DECODE_256x32
    decode = {}
    for n_tok in (1, 8):
        d_inp = kda_inputs.make_decode_inputs(dw, n_tok, device=dev)
        d_o = torch.empty(dw.n_seqs, n_tok, dw.n_heads, dw.dv, dtype=torch.float32, device=dev)

        def dstep(d_inp=d_inp, d_o=d_o):
            kda.recurrent_step(d_inp["q"], d_inp["k"], d_inp["v"], d_inp["log_alpha"], d_inp["beta"], d_inp["S"],
                               o=d_o)

        d_ms = time_launches(dstep, max(args.steps, 20), args.warmup, stream)
        d_spread = launch_spread(dstep, 50, stream)
        d_bytes = 2 * dw.n_seqs * dw.n_heads * dw.dk * dw.dv * 4 + dw.n_seqs * n_tok * dw.n_heads * BYTES_PER_TOKEN_HEAD
        d_gbs = d_bytes / (d_ms * 1e-3) / 1e9
        decode["n%d" % n_tok] = {"ms_per_step": round(d_ms, 5), "GB/s": round(d_gbs, 1),
                                 "frac_of_hbm_peak": round(d_gbs / HBM_PEAK_GBS, 4),
                                 "frac_of_copy": round(d_gbs / copy_gbs, 4),
                                 "tokens_per_s": round(dw.n_seqs * n_tok / (d_ms * 1e-3), 1), "launch_spread": d_spread,
                                 "bytes_per_step": d_bytes}
        log("recurrent_step n=%d: %.4f ms, %.0f GB/s (%.1f%% of peak)" % (n_tok, d_ms, d_gbs, 100 * d_gbs / HBM_PEAK_GBS))
        del d_inp, d_o

    # replay + verify: 8 tokens, per-sequence commit counts drawn uniformly from 0..8 (seeded)
    v_inp = kda_inputs.make_decode_inputs(dw, 8, device=dev)
    gen = torch.Generator().manual_seed(1005 + 7)
    n_commit = torch.randint(0, 9, (dw.n_seqs,), generator=gen, dtype=torch.int32).to(dev)
    v_o = torch.empty(dw.n_seqs, 8, dw.n_heads, dw.dv, dtype=torch.float32, device=dev)

    def vstep():
        kda.recurrent_verify(v_inp["q"], v_inp["k"], v_inp["v"], v_inp["log_alpha"], v_inp["beta"], v_inp["S"],
                             n_commit, o=v_o)

    v_ms = time_launches(vstep, max(args.steps, 20), args.warmup, stream)
    n_writing = int((n_commit > 0).sum().item())
    state_bytes = dw.n_heads * dw.dk * dw.dv * 4
    v_bytes = (dw.n_seqs + n_writing) * state_bytes + dw.n_seqs * 8 * dw.n_heads * BYTES_PER_TOKEN_HEAD
    v_gbs = v_bytes / (v_ms * 1e-3) / 1e9
    decode["verify_n8"] = {"ms_per_step": round(v_ms, 5), "GB/s": round(v_gbs, 1),
                           "frac_of_hbm_peak": round(v_gbs / HBM_PEAK_GBS, 4), "frac_of_copy": round(v_gbs / copy_gbs, 4),
                           "sequences_committing": n_writing, "bytes_per_step": v_bytes}
    log("recurrent_verify n=8 (%d of %d sequences commit): %.4f ms, %.0f GB/s (%.1f%% of peak)"
        % (n_writing, dw.n_seqs, v_ms, v_gbs, 100 * v_gbs / HBM_PEAK_GBS))
    del v_inp, v_o

    # ---------------- backward pass on the Kimi-Linear layer ----------------
    b_do = torch.randn(w.total_tokens, w.n_heads, w.dv, generator=torch.Generator(device=dev).manual_seed(77),
                       device=dev)
    b_ws = torch.empty(kda.backward_workspace_bytes(w.n_seqs, w.total_tokens, w.n_heads, w.dk, w.dv),
                       dtype=torch.uint8, device=dev)

    def bstep():
        kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], b_do, cu_seqlens=inp["cu_seqlens"],
                     workspace=b_ws)

    b_ms = time_launches(bstep, 5, 1, stream)
    backward = {"workload": w.name, "ms_per_step": round(b_ms, 3), "tokens_per_s": round(tokens / (b_ms * 1e-3), 1),
                "workspace_bytes": b_ws.numel(), "kind": "chunkwise fp32 matrix-core reverse mode (kda_bwd)"}
    log("backward (kda_bwd) on %s: %.3f ms/call, %.2f M tokens/s" % (w.name, b_ms, tokens / (b_ms * 1e-3) / 1e6))
    del b_do, b_ws

    # ---------------- the other chunked workloads, timed as well ----------------
    # tiny fp32 (256 tokens x 2 heads x 64 dims, chunk 16: launch-bound) and varlen packed
    # (32,768 tokens in 8 sequences x 32 heads, nonzero h0)
    other = {}
    for ow in (kda_inputs.TINY_FP32, kda_inputs.VARLEN_PACKED):
        o_inp = kda_inputs.make_chunk_inputs(ow, device=dev)
        o_o = torch.empty(ow.total_tokens, ow.n_heads, ow.dv, dtype=torch.float32, device=dev)
        o_h = torch.empty(ow.n_seqs, ow.n_heads, ow.dk, ow.dv, dtype=torch.float32, device=dev)

        def ostep(o_inp=o_inp, o_o=o_o, o_h=o_h, ow=ow):
            kda.chunk_fwd(o_inp["q"], o_inp["k"], o_inp["v"], o_inp["log_alpha"], o_inp["beta"], h0=o_inp["h0"],
                          cu_seqlens=o_inp["cu_seqlens"], chunk_size=ow.chunk_size, o=o_o, hT=o_h)

        o_ms = time_launches(ostep, 100, 20, stream)
        o_bytes = ow.total_tokens * ow.n_heads * (3 * ow.dk * o_inp["q"].element_size() + 4 * ow.dk + 4 + 4 * ow.dv)
        other[ow.name] = {"ms_per_step": round(o_ms, 5), "tokens_per_s": round(ow.total_tokens / (o_ms * 1e-3), 1),
                          "algorithmic_GB/s": round(o_bytes / (o_ms * 1e-3) / 1e9, 1)}
        log("%s: %.4f ms/launch, %.2f M tokens/s" % (ow.name, o_ms, ow.total_tokens / (o_ms * 1e-3) / 1e6))
        del o_inp, o_o, o_h

    # ---------------- long context: one 1M-token sequence x 32 heads (32 chains) ----------------
    long_context = None
    if not args.no_long_context:
        lw = kda_inputs.LONG_CONTEXT
        log("generating %s inputs" % lw.name)
        l_inp = kda_inputs.make_chunk_inputs(lw, device=dev)
        l_o = torch.empty(lw.total_tokens, lw.n_heads, lw.dv, dtype=torch.float32, device=dev)
        l_hT = torch.empty(1, lw.n_heads, lw.dk, lw.dv, dtype=torch.float32, device=dev)

        def lstep():
            kda.chunk_fwd(l_inp["q"], l_inp["k"], l_inp["v"], l_inp["log_alpha"], l_inp["beta"], h0=None,
                          chunk_size=lw.chunk_size, o=l_o, hT=l_hT)

        l_ws = None

        def lstep_split():
            kda.chunk_fwd_split(l_inp["q"], l_inp["k"], l_inp["v"], l_inp["log_alpha"], l_inp["beta"], h0=None,
                                chunk_size=lw.chunk_size, o=l_o, hT=l_hT, workspace=l_ws)

        l_bytes = lw.total_tokens * lw.n_heads * BYTES_PER_TOKEN_HEAD + lw.n_heads * lw.dk * lw.dv * 4
        long_context = {"workload": lw.name, "tokens": lw.total_tokens, "heads": lw.n_heads}
        for leg, fn in (("fused", lstep), ("split", lstep_split)):
            if leg == "split":
                l_ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(lw.n_seqs, lw.total_tokens, lw.n_heads, lw.dk,
                                                                       lw.dv, lw.chunk_size),
                                   dtype=torch.uint8, device=dev)
            l_ms = time_launches(fn, 5, 1, stream)
            l_tok = lw.total_tokens / (l_ms * 1e-3)
            n_chunks = -(-lw.seq_len // lw.chunk_size)
            long_context[leg] = {"ms_per_step": round(l_ms, 3), "tokens_per_s": round(l_tok, 1),
                                 "algorithmic_GB/s": round(l_bytes / (l_ms * 1e-3) / 1e9, 1),
                                 "us_per_serial_chunk_step": round(l_ms * 1e3 / n_chunks, 3)}
            log("long context, %s (%d tokens x %d heads): %.2f ms/launch, %.2f M tokens/s"
                % (leg, lw.total_tokens, lw.n_heads, l_ms, l_tok / 1e6))
        if l_ws is not None:
            long_context["split"]["workspace_bytes"] = l_ws.numel()
        del l_inp, l_o, l_hT, l_ws

    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.n_seqs, "seq_len": w.seq_len, "heads": w.n_heads,
                   "dk": w.dk, "dv": w.dv, "chunk": w.chunk_size, "tokens": tokens,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(),
                     "kernel": "chunk_fwd_kernel", "algorithmic_bytes_per_launch": alg_bytes,
                     "copy_GB/s": round(copy_gbs, 1), "frac_of_copy": round(gbs / copy_gbs, 4)},
        "launch_spread": spread,
        "mfma": {"algorithmic_tflops": round(tflops, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops_per_launch": alg_flops,
                 # rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / (cycles x SIMDs) and VALU busy of the same kernel
                 "counter_busy_frac": profile_value(SQ_SUMMARY, "mfma_busy_frac"),
                 "counter_valu_busy_frac": profile_value(SQ_SUMMARY, "valu_busy_frac")},
        "checkpointed": checkpointed,
        "decode": decode,
        "long_context": long_context,
        "backward": backward,
        "other_workloads": other,
        "wall_s_timed_region": round(t_wall, 3),
    }
    if args.copy_calibration:
        result["copy_calibration"] = copy_calibration(dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
