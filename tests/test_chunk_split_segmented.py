"""kda_chunk_fwd_split on few (sequence, head) chains with long sequences, where the state pass
runs in parallel over segments of each chain: per-segment affine maps, their composition by a
scan from h0, and a rerun of every segment from its entering state.

Shapes are chosen so that chains x dv/32 <= 64 and the longest sequence has at least 512
chunks (the segmented form), with sequences that end in different segments, empty and
one-token sequences, nonzero h0, and dk, dv, chunk size varied.  Against the fp64 oracle at
the bf16 bound (max |err| <= 2e-2 * RMS(ref) for o and hT separately); the difference from
the fused kda_chunk_fwd (the same operand precisions, plus the rounding of each segment's map)
is printed.
"""
import pytest
import torch

import kda_inputs
from test_chunk_parity import check_bf16, report
from test_chunk_split import ref, run_fused, run_split

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lens,H,dk,dv,C", [
    ([44800], 1, 128, 128, 64),                 # one chain, 700 chunks: 10 segments
    ([40000, 9000, 33, 0], 2, 128, 128, 64),    # 8 segments; sequences ending in segments 7, 1 and 0, one empty
    ([20500, 1], 2, 64, 64, 32),                # dk = dv = 64, chunk 32: 641 chunks
    ([8200], 8, 128, 64, 16),                   # dv = 64, chunk 16: 513 chunks, eight heads
])
def test_split_segmented_against_oracle(lens, H, dk, dv, C):
    print("split segmented: lens=%s H=%d dk=%d dv=%d C=%d" % (lens, H, dk, dv, C), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, H, dk, dv, torch.bfloat16, h0_std=0.02, seed=sum(lens) + 7 * H,
                                              device="cuda")
    o, hT = run_split(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    of, hf = run_fused(inp, chunk_size=C)
    report("segmented vs fused o", o.cpu(), of.cpu().double().numpy())
    report("segmented vs fused hT", hT.cpu(), hf.cpu().double().numpy())


def test_split_segmented_final_state_in_place_and_absent():
    """hT aliasing h0: every segment runs in one launch, and the chain's last segment writes hT
    while its first starts from h0 (read from the workspace copy the scan made); hT not
    requested."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_custom_chunk_inputs([36000, 2000], 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=43,
                                              device="cuda")
    o_ref, h_ref = ref(inp)
    h = inp["h0"].clone()
    o, _ = kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=h,
                               cu_seqlens=inp["cu_seqlens"], chunk_size=64, hT=h)
    torch.cuda.synchronize()
    check_bf16(o, h, o_ref, h_ref)
    o2, _ = kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                                cu_seqlens=inp["cu_seqlens"], chunk_size=64, output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o2, o)


@pytest.mark.parametrize("C,T,gate,bscale,h0_std", [(16, 8320, 3e-4, 0.05, 1.0), (64, 33280, 5e-5, 0.01, 3.0)])
def test_split_segmented_long_memory(C, T, gate, bscale, h0_std):
    """One chain of 520 chunks (8 segments of 65) with weak decay and small beta, so that the
    state entering a segment still matters at its end: every segment's map M is far from zero
    and the scan's composition decides the result.  The oracle's final state with h0 and with
    zeros differ by far more than the tolerance, which makes sure of that."""
    import numpy as np
    import oracle
    inp = kda_inputs.make_custom_chunk_inputs([T], 1, 128, 128, torch.bfloat16, gate_scale=gate, h0_std=h0_std,
                                              seed=T + C, device="cuda")
    inp["beta"] = (inp["beta"] * bscale).contiguous()
    print("split segmented, long memory: T=%d C=%d" % (T, C), flush=True)
    o, hT = run_split(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    _, h_zero = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], None, inp["cu_seqlens"])
    carried = float(np.abs(h_ref - h_zero).max()) / float(np.sqrt(np.mean(h_ref ** 2)))
    print("  h0's share of hT: max|hT(h0) - hT(0)| / rms(hT) = %.3f" % carried, flush=True)
    assert carried > 0.1
