"""kda_chunk_fwd_split (HIP, two passes: in-chunk work to a workspace, then the state pass)
against the fp64 oracle, and against the fused kda_chunk_fwd on the same inputs.

Tolerance against the oracle: bf16 inputs, max |err| <= 2e-2 * RMS(ref) for o and hT
separately.  Against the fused kernel: max |diff| <= 1e-4 * RMS(ref): both paths round the
same operands at the same points (v in fp32 in the chunk's power-of-two units, Y to fp32 and
then fp16, U, S and the in-chunk operands to fp16), so only the order of fp32 accumulation
may differ.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle
from test_chunk_parity import check_bf16, report, to64

pytestmark = pytest.mark.gpu

SAME_TOL = 1e-4


def run_split(inp, chunk_size=None, h0="inp", workspace=None):
    import kimi_delta_attention_06_amd as kda
    h0 = inp["h0"] if h0 == "inp" else h0
    o, hT = kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=h0,
                                cu_seqlens=inp["cu_seqlens"], chunk_size=chunk_size or inp["chunk_size"],
                                workspace=workspace)
    torch.cuda.synchronize()
    return o, hT


def run_fused(inp, chunk_size=None):
    import kimi_delta_attention_06_amd as kda
    o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], chunk_size=chunk_size or inp["chunk_size"])
    torch.cuda.synchronize()
    return o, hT


def ref(inp):
    return oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"], inp["cu_seqlens"])


def check_same(a, b, ref_arr, name):
    d = float(np.abs(to64(a) - to64(b)).max()) if ref_arr.size else 0.0
    rms = float(np.sqrt(np.mean(ref_arr ** 2))) if ref_arr.size else 0.0
    print("  %-3s split vs fused max|diff| %.3e (rms(ref) %.3e)" % (name, d, rms), flush=True)
    assert d <= SAME_TOL * rms, (d, rms)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_split_small_varlen_bf16(C, dk, dv):
    """Several chunks with ragged tails, empty and 1-token sequences, nonzero h0."""
    lens = [150, 0, 1, 64, 97, 33]
    print("split: small varlen bf16 C=%d dk=%d dv=%d lens=%s" % (C, dk, dv, lens), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, 3, dk, dv, torch.bfloat16, h0_std=0.02, seed=11 + C + dk,
                                              device="cuda")
    o, hT = run_split(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    of, hf = run_fused(inp, chunk_size=C)
    check_same(o, of, o_ref, "o")
    check_same(hT, hf, h_ref, "hT")


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("dk", [64, 128])
def test_split_many_chains_one_tile_per_chain(C, dk):
    """At least 256 (sequence, head) chains with dv = 128: the state pass takes the whole value
    width in one workgroup per chain (ragged lengths, empty and 1-token sequences)."""
    lens = [(37 * i) % 150 for i in range(40)]  # includes 0, 1-token and multi-chunk sequences
    lens[3] = 1
    H = 7  # 280 chains
    print("split: many chains C=%d dk=%d H=%d lens %s" % (C, dk, H, lens[:8]), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, H, dk, 128, torch.bfloat16, h0_std=0.02, seed=200 + C + dk,
                                              device="cuda")
    o, hT = run_split(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    of, hf = run_fused(inp, chunk_size=C)
    check_same(o, of, o_ref, "o")
    check_same(hT, hf, h_ref, "hT")


@pytest.mark.parametrize("C", [16, 64])
def test_split_narrow_decay(C):
    """Gate law x0.1: the fp16 path for every diagonal sub-block."""
    inp = kda_inputs.make_custom_chunk_inputs([150, 0, 1, 64, 97, 33], 3, 128, 128, torch.bfloat16,
                                              gate_scale=0.1, h0_std=0.02, seed=31 + C, device="cuda")
    o, hT = run_split(inp, chunk_size=C)
    check_bf16(o, hT, *ref(inp))


def test_split_mixed_narrow_and_wide_decay_channels():
    inp = kda_inputs.make_custom_chunk_inputs([200, 77], 4, 128, 128, torch.bfloat16, gate_scale=0.1,
                                              h0_std=0.02, seed=41, device="cuda")
    inp["log_alpha"][:, :, 64:96] = -0.6  # 9.6 nats per 16-token block on these channels
    o, hT = run_split(inp, chunk_size=64)
    check_bf16(o, hT, *ref(inp))


def test_split_final_state_in_place():
    """hT may be h0 itself: every chain reads its h0 before it writes hT."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_custom_chunk_inputs([130, 65], 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=3,
                                              device="cuda")
    o_ref, h_ref = ref(inp)
    h = inp["h0"].clone()
    o, hT = kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=h,
                                cu_seqlens=inp["cu_seqlens"], chunk_size=64, hT=h)
    torch.cuda.synchronize()
    check_bf16(o, h, o_ref, h_ref)


def test_split_workspace_reused_with_smaller_input():
    """One caller-held workspace serves a large call and then a smaller one."""
    import kimi_delta_attention_06_amd as kda
    a = kda_inputs.make_custom_chunk_inputs([300, 17, 129], 3, 128, 128, torch.bfloat16, h0_std=0.02, seed=5,
                                            device="cuda")
    b = kda_inputs.make_custom_chunk_inputs([70, 1], 2, 128, 128, torch.bfloat16, seed=6, device="cuda")
    ws = torch.empty(8 << 20, dtype=torch.uint8, device="cuda")
    for inp in (a, b):
        o, hT = run_split(inp, chunk_size=64, workspace=ws)
        check_bf16(o, hT, *ref(inp))


def test_split_kimi_linear_layer_workload():
    """B=4, T=4096, H=32, dk=dv=128, chunk 64: against the oracle and the fused kernel."""
    print("split: kimi-linear layer: B=4 T=4096 H=32 d=128 C=64", flush=True)
    inp = kda_inputs.make_chunk_inputs(kda_inputs.KIMI_LINEAR_LAYER, device="cuda")
    o, hT = run_split(inp)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    of, hf = run_fused(inp)
    check_same(o, of, o_ref, "o")
    check_same(hT, hf, h_ref, "hT")


def test_split_varlen_packed_workload():
    inp = kda_inputs.make_chunk_inputs(kda_inputs.VARLEN_PACKED, device="cuda")
    print("split: varlen packed: lens=%s" % list(inp["lens"]), flush=True)
    o, hT = run_split(inp)
    check_bf16(o, hT, *ref(inp))


@pytest.mark.slow
def test_split_long_context_workload_two_heads():
    """B=1, T=1,048,576, H=32, d=128, chunk 64 through the split path: o and hT on 2 seeded heads."""
    heads = kda_inputs.long_context_oracle_heads()
    print("split: long context T=1048576 H=32, oracle heads %s" % list(heads), flush=True)
    inp = kda_inputs.make_chunk_inputs(kda_inputs.LONG_CONTEXT, device="cuda")
    o, hT = run_split(inp)
    hs = torch.as_tensor(heads, device="cuda")
    sub = {k: inp[k].index_select(1, hs).cpu() for k in ("q", "k", "v", "log_alpha", "beta")}
    o_s = o.index_select(1, hs).cpu()
    h_s = hT.index_select(1, hs).cpu()
    del inp, o, hT
    torch.cuda.empty_cache()
    o_ref, h_ref = oracle.kda_fwd(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], None, None)
    check_bf16(o_s, h_s, o_ref, h_ref)


@pytest.mark.parametrize("lens,H,dv,path", [
    ([2600, 17, 1400, 1260], 2, 128, "split"),   # 8 chains: the fused kernel would use 16-column tiles
    ([600, 17, 400, 260], 2, 128, "fused"),      # the same chains, 5 chunks per sequence on average
    ([256] * 64, 2, 128, "fused"),               # 128 chains of 4 chunks: one round of 64-column fused tiles
    ([1100] * 64, 2, 128, "split"),              # one round of fused tiles, 17 chunks per sequence
    ([256] * 40 + [300, 212] * 12, 4, 128, "split"),  # 256 chains: two rounds of fused tiles
    ([256] * 128, 2, 64, "fused"),               # 256 chains at dv = 64: one fused tile per chain
])
def test_auto_takes_the_path_its_rule_names(lens, H, dv, path):
    """kda_chunk_fwd_auto: the same bits as the path the shape rule picks, against the oracle; the fused
    choice runs without a workspace."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_custom_chunk_inputs(lens, H, 128, dv, torch.bfloat16, h0_std=0.02, seed=len(lens) + H,
                                              device="cuda")
    args = (inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"])
    kw = dict(h0=inp["h0"], cu_seqlens=inp["cu_seqlens"], chunk_size=64)
    if path == "fused":
        o_a, h_a = kda.chunk_fwd_auto(*args, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"), **kw)
        o_p, h_p = kda.chunk_fwd(*args, **kw)
    else:
        o_a, h_a = kda.chunk_fwd_auto(*args, **kw)
        o_p, h_p = kda.chunk_fwd_split(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_p) and torch.equal(h_a, h_p)
    check_bf16(o_a, h_a, *ref(inp))
