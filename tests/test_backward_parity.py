"""kda_bwd (HIP, token-recurrent fp32 backward) against the fp64 oracle's reverse mode.

The kernel evaluates the adjoint recurrence in fp32 from inputs that are exact in fp32
(bf16 inputs widen exactly), so its error is fp32 rounding accumulated over a sequence:
tolerance max |err| <= 1e-3 * RMS(ref) for every gradient (dq, dk, dv, dlog_alpha, dbeta,
dh0) separately, for fp32 and bf16 inputs alike.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-3


def to64(x):
    return x.detach().cpu().double().numpy()


def check(g, ref):
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"):
        x, r = to64(g[key]).reshape(ref[key].shape), ref[key]
        rms = float(np.sqrt(np.mean(r ** 2))) if r.size else 0.0
        err = float(np.abs(x - r).max()) if r.size else 0.0
        print("  %-10s max|err| %.3e  rms(ref) %.3e  max/rms %.2e" % (key, err, rms, err / rms if rms else 0.0),
              flush=True)
        assert np.isfinite(x).all(), key
        assert err <= TOL * rms, (key, err, rms)


def run(inp, do, dhT):
    import kimi_delta_attention_06_amd as kda
    g = kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, h0=inp["h0"],
                     cu_seqlens=inp["cu_seqlens"], dhT=dhT)
    torch.cuda.synchronize()
    return g


def ref(inp, do, dhT):
    return oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"], inp["cu_seqlens"],
                          do, dhT)


def cotangents(inp, seed, with_dhT=True):
    g = torch.Generator(device="cpu").manual_seed(seed)
    T, H, dv = inp["v"].shape
    N = inp["cu_seqlens"].numel() - 1
    dk = inp["q"].shape[2]
    do = torch.randn(T, H, dv, generator=g).cuda()
    dhT = torch.randn(N, H, dk, dv, generator=g).cuda() * 0.1 if with_dhT else None
    return do, dhT


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_backward_small_varlen(dtype, dk, dv):
    """Sequences across several 64-token segments with ragged tails, an empty and a 1-token one,
    nonzero h0 and dhT."""
    lens = [150, 0, 1, 64, 97, 33]
    print("backward: %s dk=%d dv=%d lens=%s" % (dtype, dk, dv, lens), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 3, dk, dv, dtype, h0_std=0.02, seed=21 + dk + dv, device="cuda")
    do, dhT = cotangents(inp, 5 + dk)
    check(run(inp, do, dhT), ref(inp, do, dhT))


def test_backward_without_initial_or_final_state():
    inp = kda_inputs.make_custom_chunk_inputs([130, 7], 2, 128, 128, torch.bfloat16, seed=8, device="cuda")
    do, _ = cotangents(inp, 9, with_dhT=False)
    check(run(inp, do, None), ref(inp, do, None))


def test_backward_kimi_linear_layer_two_heads():
    """The Kimi-Linear-shaped layer (B=4, T=4096, d=128) on 2 of its 32 heads, gate law x0.1."""
    w = kda_inputs.KIMI_LINEAR_LAYER
    inp = kda_inputs.make_chunk_inputs(w, device="cuda")
    hs = torch.tensor([3, 17], device="cuda")
    sub = {k_: inp[k_].index_select(1, hs).contiguous() for k_ in ("q", "k", "v", "log_alpha", "beta")}
    sub["h0"] = None
    sub["cu_seqlens"] = inp["cu_seqlens"]
    del inp
    do, dhT = cotangents(sub, 11)
    print("backward: Kimi-Linear layer, heads 3 and 17, B=4 T=4096", flush=True)
    check(run(sub, do, dhT), ref(sub, do, dhT))
