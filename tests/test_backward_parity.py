"""kda_bwd (HIP, chunkwise fp32 matrix-core backward) and kda_bwd_recurrent (HIP, token by
token, fp32) against the fp64 oracle's reverse mode.

Both evaluate the adjoint in fp32 from inputs that are exact in fp32 (bf16 inputs widen
exactly), so their error is fp32 rounding accumulated over a sequence: tolerance
max |err| <= 1e-3 * RMS(ref) for every gradient (dq, dk, dv, dlog_alpha, dbeta, dh0)
separately, for fp32 and bf16 inputs alike.
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


def run(inp, do, dhT, method="chunk"):
    import kimi_delta_attention_06_amd as kda
    g = kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, h0=inp["h0"],
                     cu_seqlens=inp["cu_seqlens"], dhT=dhT, method=method)
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


METHODS = ["chunk", "recurrent"]


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_backward_small_varlen(method, dtype, dk, dv):
    """Sequences across several chunks and 64-token segments with ragged tails and unaligned
    starts, an empty and a 1-token one, nonzero h0 and dhT."""
    lens = [150, 0, 1, 64, 97, 33]
    print("backward %s: %s dk=%d dv=%d lens=%s" % (method, dtype, dk, dv, lens), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 3, dk, dv, dtype, h0_std=0.02, seed=21 + dk + dv, device="cuda")
    do, dhT = cotangents(inp, 5 + dk)
    check(run(inp, do, dhT, method), ref(inp, do, dhT))


@pytest.mark.parametrize("method", METHODS)
def test_backward_without_initial_or_final_state(method):
    inp = kda_inputs.make_custom_chunk_inputs([130, 7], 2, 128, 128, torch.bfloat16, seed=8, device="cuda")
    do, _ = cotangents(inp, 9, with_dhT=False)
    check(run(inp, do, None, method), ref(inp, do, None))


@pytest.mark.parametrize("lens", [[16], [15], [17, 16, 48, 3]])
def test_backward_chunk_boundaries(lens):
    """Lengths at, below and past the 16-token chunk: full, ragged and single-row chunks."""
    print("backward chunk: lens=%s" % (lens,), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=len(lens),
                                              device="cuda")
    do, dhT = cotangents(inp, 3)
    check(run(inp, do, dhT), ref(inp, do, dhT))


def test_backward_chunk_strong_decay():
    """Gate law x5: about 4 nats per token and channel on average, ~65 per 16-token chunk and
    ~105 at most, so chunks fall on both sides of the 64-nat switch between decay factors
    balanced around the chunk's middle and the exact elementwise ones."""
    inp = kda_inputs.make_custom_chunk_inputs([200, 45], 2, 128, 128, torch.bfloat16, gate_scale=5.0, h0_std=0.02,
                                              seed=77, device="cuda")
    la = inp["log_alpha"].double()
    print("backward chunk strong decay: mean log a %.2f, min over 16 tokens %.1f" %
          (float(la.mean()), float(la[:16].sum(0).min())), flush=True)
    do, dhT = cotangents(inp, 4)
    check(run(inp, do, dhT), ref(inp, do, dhT))


@pytest.mark.parametrize("method", METHODS)
def test_backward_kimi_linear_layer_two_heads(method):
    """The Kimi-Linear-shaped layer (B=4, T=4096, d=128) on 2 of its 32 heads, gate law x0.1."""
    w = kda_inputs.KIMI_LINEAR_LAYER
    inp = kda_inputs.make_chunk_inputs(w, device="cuda")
    hs = torch.tensor([3, 17], device="cuda")
    sub = {k_: inp[k_].index_select(1, hs).contiguous() for k_ in ("q", "k", "v", "log_alpha", "beta")}
    sub["h0"] = None
    sub["cu_seqlens"] = inp["cu_seqlens"]
    del inp
    do, dhT = cotangents(sub, 11)
    print("backward %s: Kimi-Linear layer, heads 3 and 17, B=4 T=4096" % method, flush=True)
    check(run(sub, do, dhT, method), ref(sub, do, dhT))
