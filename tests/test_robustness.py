"""Parity on adversarial inputs: every chunked path against the fp64 oracle where the chunk
algebra is hardest to evaluate in finite precision.

* wide_decay: log a = -30 on a third of the key channels (480 nats per 16 tokens, far past the
  range where decay factors balanced around a block's middle stay finite) and exactly 0 on
  another third;
* large_values / small_values: bf16 v near 1e4 or 1e-5 and h0 near 1e3 or 1e-7, outside the
  range of the fp16 matrix-core operands either way;
* parallel_keys: beta = 1 with keys that repeat exactly or differ by 1e-3 inside a chunk (the
  largest key-Gram entries, the UT inverse furthest from the identity).

Each at chunk 16 and 64 through the fused, split, pipelined-split and checkpointed forwards
(bf16: max |err| <= 2e-2 * RMS(ref) for o and hT separately; fp32: max |err| <= 1e-4) and
through both backward methods (max |err| <= 1e-3 * RMS(ref) per gradient).
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from test_backward_parity import check as check_grads
from test_backward_parity import cotangents
from test_chunk_parity import check_bf16, report, to64

pytestmark = pytest.mark.gpu

KINDS = kda_inputs.ADVERSARIAL_KINDS
LENS = [150, 0, 1, 64, 97, 33]


def kda():
    import kimi_delta_attention_06_amd as m
    return m


def adv(kind, lens=LENS, H=3, d=128, dtype=torch.bfloat16, seed=0):
    return kda_inputs.make_adversarial_chunk_inputs(kind, lens, H, d, d, dtype=dtype, seed=seed + KINDS.index(kind),
                                                    device="cuda")


def ref(inp):
    return oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"], inp["cu_seqlens"])


def fwd(path, inp, C, **kw):
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    if path == "fused":
        out = kda().chunk_fwd(*args, h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=C, **kw)
    elif path == "split":
        out = kda().chunk_fwd_split(*args, h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=C, **kw)
    else:
        out = kda().chunk_fwd_checkpointed(*args, h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=C,
                                           ckpt_every=2 * C, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("path", ["fused", "split", "checkpointed"])
def test_forward_adversarial(kind, C, path):
    print("adversarial forward: %s, %s, chunk %d, lens %s" % (kind, path, C, LENS), flush=True)
    inp = adv(kind, seed=10 * C)
    out = fwd(path, inp, C)
    o, hT = out[0], out[1]
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    if path == "checkpointed":
        # the state after 2C tokens of the first sequence (slot 1 with spacing 2C): the oracle's
        # final state over that prefix
        ck = out[2]
        p = 2 * C
        sub = {k_: inp[k_][:p] for k_ in ("q", "k", "v", "log_alpha", "beta")}
        _, h_p = oracle.kda_fwd(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], inp["h0"][:1],
                                torch.tensor([0, p], dtype=torch.int32))
        e, r = report("ckpt", ck[0:1], h_p)
        assert e <= 2e-2 * r


@pytest.mark.parametrize("kind", KINDS)
def test_split_pipelined_adversarial(kind):
    """Few chains and 150+ chunks: the state pass runs over ranges beside the in-chunk pass."""
    lens = [9000, 700]
    print("adversarial pipelined split: %s, lens %s" % (kind, lens), flush=True)
    inp = adv(kind, lens=lens, H=2, seed=99)
    o, hT = fwd("split", inp, 64)
    check_bf16(o, hT, *ref(inp))


@pytest.mark.parametrize("kind", KINDS)
def test_split_segmented_adversarial(kind):
    """One chain of 521 chunks: the state pass runs over 8 segments (maps, scan, rerun)."""
    lens = [33300]
    print("adversarial segmented split: %s, lens %s" % (kind, lens), flush=True)
    inp = adv(kind, lens=lens, H=1, seed=131)
    o, hT = fwd("split", inp, 64)
    check_bf16(o, hT, *ref(inp))


@pytest.mark.parametrize("C", [16, 32, 64])
def test_forward_fp32_wide_decay(C):
    """fp32 inputs (every product on the fp32 matrix core), dk = dv = 128."""
    inp = adv("wide_decay", lens=[150, 1, 77], H=2, dtype=torch.float32, seed=5)
    o, hT = fwd("fused", inp, C)
    o_ref, h_ref = ref(inp)
    eo, _ = report("o", o, o_ref)
    eh, _ = report("hT", hT, h_ref)
    assert eo <= 1e-4 and eh <= 1e-4


def test_forward_extreme_finite_log_alpha():
    """log a of -1e30 (alpha 0 to any precision) on some tokens and channels, -1e4 on others:
    finite, so taken; the results are those of a gate of exactly 0 there."""
    inp = kda_inputs.make_custom_chunk_inputs([150, 40], 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=4,
                                              device="cuda")
    la = inp["log_alpha"]
    la[5:60:7, :, :50] = -1e30
    la[70:90, :, 60:64] = -1e4
    for path, C in (("fused", 64), ("fused", 16), ("split", 64)):
        o, hT = fwd(path, inp, C)[:2]
        check_bf16(o, hT, *ref(inp))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("method", ["chunk", "recurrent"])
def test_backward_adversarial(kind, method):
    print("adversarial backward: %s, %s" % (kind, method), flush=True)
    inp = adv(kind, lens=[150, 0, 1, 64, 33], H=2, seed=50)
    do, dhT = cotangents(inp, 12)
    if kind == "large_values":
        do = do * 100.0
    g = kda().backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, h0=inp["h0"],
                       cu_seqlens=inp["cu_seqlens"], dhT=dhT, method=method)
    torch.cuda.synchronize()
    check_grads(g, oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"],
                                  inp["cu_seqlens"], do, dhT))


@pytest.mark.parametrize("kind", ["wide_decay", "large_values"])
def test_decode_adversarial(kind):
    """The decode / replay step (fp32 throughout) on the same laws, 8 tokens per sequence."""
    inp = adv(kind, lens=[8] * 6, H=4, seed=71)
    N, H = 6, 4
    tok = lambda x: x.view(N, 8, H, -1).contiguous() if x.dim() == 3 else x.view(N, 8, H).contiguous()
    S = inp["h0"].clone()
    o = kda().recurrent_step(tok(inp["q"]), tok(inp["k"]), tok(inp["v"]), tok(inp["log_alpha"]), tok(inp["beta"]), S)
    torch.cuda.synchronize()
    o_ref, h_ref = ref(inp)
    check_bf16(o.view(N * 8, H, -1), S, o_ref, h_ref)
