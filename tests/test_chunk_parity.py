"""kda_chunk_fwd (HIP) against the fp64 oracle.

Tolerances: fp32 inputs, max |err| <= 1e-4; bf16 inputs, max |err| <= 2e-2 * RMS(ref),
for o and hT separately (the norm-wise error RMS(err)/RMS(ref) is printed too).
Inputs are seeded synthetic draws of the Kimi-Linear-shaped KDA layer (32 heads of
128 dims, chunk 64) and of the tiny fp32 case (2 heads of 64 dims, chunk 16).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-4


def to64(x):
    return x.detach().cpu().double().numpy()


def report(name, x, ref):
    x = to64(x) if isinstance(x, torch.Tensor) else x
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.abs(x - ref).max()) if ref.size else 0.0
    nerr = float(np.sqrt(np.mean((x - ref) ** 2))) / rms if rms > 0 else 0.0
    print("  %-3s max|err| %.3e  rms(ref) %.3e  max/rms %.2e  rms-err/rms %.2e" % (
        name, err, rms, err / rms if rms else 0.0, nerr), flush=True)
    return err, rms


def check_bf16(o, hT, o_ref, h_ref):
    eo, ro = report("o", o, o_ref)
    eh, rh = report("hT", hT, h_ref)
    assert np.isfinite(to64(o)).all() and np.isfinite(to64(hT)).all()
    assert eo <= BF16_TOL * ro, (eo, ro)
    assert eh <= BF16_TOL * rh, (eh, rh)


def run(inp, chunk_size=None, h0="inp"):
    import kimi_delta_attention_06_amd as kda
    h0 = inp["h0"] if h0 == "inp" else h0
    o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=h0,
                          cu_seqlens=inp["cu_seqlens"], chunk_size=chunk_size or inp["chunk_size"])
    torch.cuda.synchronize()
    return o, hT


def ref(inp, h0="inp"):
    h0 = inp["h0"] if h0 == "inp" else h0
    return oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0, inp["cu_seqlens"])


def test_tiny_fp32_workload():
    """B=1, T=256, H=2, dk=dv=64, chunk 16, fp32 everything, h0 = 0."""
    print("tiny fp32: T=256 H=2 d=64 C=16", flush=True)
    inp = kda_inputs.make_chunk_inputs(kda_inputs.TINY_FP32, device="cuda")
    o_ref, h_ref = ref(inp)
    for h0 in (None, torch.zeros(1, 2, 64, 64, device="cuda")):
        o, hT = run(inp, h0=h0)
        eo, _ = report("o", o, o_ref)
        eh, _ = report("hT", hT, h_ref)
        assert eo <= F32_TOL and eh <= F32_TOL


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_small_varlen_bf16(C, dk, dv):
    """Several chunks with ragged tails, empty and 1-token sequences, nonzero h0."""
    lens = [150, 0, 1, 64, 97, 33]
    print("small varlen bf16 C=%d dk=%d dv=%d lens=%s" % (C, dk, dv, lens), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 3, dk, dv, torch.bfloat16, h0_std=0.02, seed=11 + C + dk,
                                              device="cuda")
    o, hT = run(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_small_varlen_bf16_narrow_decay(C, dk, dv):
    """Gate law x0.1 (blocks decay by < 8 nats: the fp16 path for the diagonal sub-blocks)."""
    lens = [150, 0, 1, 64, 97, 33]
    print("small varlen bf16, narrow decay, C=%d dk=%d dv=%d" % (C, dk, dv), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 3, dk, dv, torch.bfloat16, gate_scale=0.1, h0_std=0.02,
                                              seed=31 + C + dk, device="cuda")
    o, hT = run(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)


def test_mixed_narrow_and_wide_decay_channels():
    """One channel half decays by < 8 nats per block and the other by more, so the two waves
    of a row block take different paths for the diagonal sub-blocks."""
    inp = kda_inputs.make_custom_chunk_inputs([200, 77], 4, 128, 128, torch.bfloat16, gate_scale=0.1,
                                              h0_std=0.02, seed=41, device="cuda")
    inp["log_alpha"][:, :, 64:96] = -0.6  # 9.6 nats per 16-token block on these channels
    o, hT = run(inp, chunk_size=64)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)


@pytest.mark.parametrize("C,dk,dv", [(64, 64, 64), (64, 64, 128), (32, 128, 64), (16, 64, 128)])
def test_small_varlen_fp32_more_shapes(C, dk, dv):
    """fp32 inputs at the remaining supported (chunk, dk, dv) combinations (C = 64 needs dk = 64)."""
    lens = [140, 0, 1, 64, 29]
    print("small varlen fp32 C=%d dk=%d dv=%d" % (C, dk, dv), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 2, dk, dv, torch.float32, h0_std=0.02, seed=17 + C + dv,
                                              device="cuda")
    o, hT = run(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    eo, _ = report("o", o, o_ref)
    eh, _ = report("hT", hT, h_ref)
    assert eo <= F32_TOL and eh <= F32_TOL


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("dk", [64, 128])
def test_small_varlen_fp32(C, dk):
    lens = [70, 0, 1, 33, 16]
    print("small varlen fp32 C=%d dk=%d" % (C, dk), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 2, dk, dk, torch.float32, h0_std=0.02, seed=5 + C,
                                              device="cuda")
    o, hT = run(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    eo, _ = report("o", o, o_ref)
    eh, _ = report("hT", hT, h_ref)
    assert eo <= F32_TOL and eh <= F32_TOL


def test_kimi_linear_layer_workload():
    """B=4, T=4096, H=32, dk=dv=128, chunk 64, bf16 q/k/v, log_alpha = -0.1 softplus, h0 = 0."""
    print("kimi-linear layer: B=4 T=4096 H=32 d=128 C=64", flush=True)
    inp = kda_inputs.make_chunk_inputs(kda_inputs.KIMI_LINEAR_LAYER, device="cuda")
    o, hT = run(inp)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)


def test_varlen_packed_workload():
    """32768 tokens in 8 seeded sequences (min 256), H=32, d=128, chunk 64, h0 ~ N(0, 0.02^2)."""
    inp = kda_inputs.make_chunk_inputs(kda_inputs.VARLEN_PACKED, device="cuda")
    print("varlen packed: lens=%s" % list(inp["lens"]), flush=True)
    o, hT = run(inp)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)


@pytest.mark.slow
def test_long_context_workload_two_heads():
    """B=1, T=1,048,576, H=32, d=128, chunk 64: o and hT checked on 2 seeded heads."""
    heads = kda_inputs.long_context_oracle_heads()
    print("long context: T=1048576 H=32 d=128 C=64, oracle heads %s" % list(heads), flush=True)
    inp = kda_inputs.make_chunk_inputs(kda_inputs.LONG_CONTEXT, device="cuda")
    o, hT = run(inp)
    hs = torch.as_tensor(heads, device="cuda")
    sub = {k: inp[k].index_select(1, hs).cpu() for k in ("q", "k", "v", "log_alpha", "beta")}
    o_s = o.index_select(1, hs).cpu()
    h_s = hT.index_select(1, hs).cpu()
    del inp, o, hT
    torch.cuda.empty_cache()
    print("  running the oracle on 2 heads x 1M tokens", flush=True)
    o_ref, h_ref = oracle.kda_fwd(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], None, None)
    check_bf16(o_s, h_s, o_ref, h_ref)
