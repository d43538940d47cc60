"""kda_chunk_fwd_split on inputs with few (sequence, head) chains and long sequences, where
the state pass runs over ranges of chunks beside the next range's in-chunk pass, against
the fp64 oracle and against the fused kda_chunk_fwd.

Shapes are chosen so that the state pass needs at most 128 workgroups (chains x dv/32)
and the longest sequence has 128 to 511 chunks (two or more ranges; from 512 chunks, few
enough chains take the segmented form of test_chunk_split_segmented).  Against the oracle:
bf16 inputs, max |err| <= 2e-2 * RMS(ref), as in test_chunk_split.

Against the fused kernel: the state pass of this form runs one wave per 16 value columns,
which feeds each product's accumulators to the next product as its B operand; the 32 terms
of a k-step are then summed in another order than in the fused kernel, so an fp32 sum can
differ in its last bit, and the fp16 rounding of Y or U that follows can then land one fp16
ulp (2^-11 relative) away.  Such a flip moves the o rows of its chunk by about one fp16 ulp
of U times |q.k| or an entry of M (both at most 1 for unit keys and queries), and the state by
far less after the decay and the key product, while most elements are unaffected.  So the
comparison bounds the largest difference by 1e-2 * RMS(ref) (half the oracle bound, several
fp16 ulps of the largest U) and the RMS of the differences by 1e-4 * RMS(ref), which a
systematic error (a wrong term, index or scale) would exceed by orders of magnitude.
"""
import numpy as np
import pytest
import torch

import kda_inputs
from test_chunk_parity import check_bf16, to64
from test_chunk_split import check_same, ref, run_fused, run_split

pytestmark = pytest.mark.gpu

ORDER_MAX_TOL = 1e-2
ORDER_RMS_TOL = 1e-4


def check_close_order(a, b, ref_arr, name):
    """a and b agree up to the fp16 rounding flips of a different fp32 summation order."""
    if not ref_arr.size:
        return
    d = np.abs(to64(a) - to64(b))
    rms = float(np.sqrt(np.mean(ref_arr ** 2)))
    dmax, drms = float(d.max()), float(np.sqrt(np.mean(d ** 2)))
    print("  %-3s pipelined vs fused max|diff|/rms %.3e  rms-diff/rms %.3e" % (name, dmax / rms, drms / rms),
          flush=True)
    assert dmax <= ORDER_MAX_TOL * rms, (dmax, rms)
    assert drms <= ORDER_RMS_TOL * rms, (drms, rms)


@pytest.mark.parametrize("lens,H,dk,dv,C", [
    ([16384], 4, 128, 128, 64),          # 256 chunks: ranges of 80, 80 and 96
    ([9000, 3000, 70, 0], 2, 128, 128, 64),  # sequences ending in different ranges, one empty
    ([5000, 4097], 3, 64, 64, 32),       # dk = dv = 64, chunk 32
    ([8100], 8, 128, 64, 16),            # dv = 64, chunk 16: 507 chunks, six ranges
])
def test_split_pipelined_against_oracle_and_fused(lens, H, dk, dv, C):
    print("split pipelined: lens=%s H=%d dk=%d dv=%d C=%d" % (lens, H, dk, dv, C), flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(lens, H, dk, dv, torch.bfloat16, h0_std=0.02, seed=sum(lens) + H,
                                              device="cuda")
    o, hT = run_split(inp, chunk_size=C)
    o_ref, h_ref = ref(inp)
    check_bf16(o, hT, o_ref, h_ref)
    of, hf = run_fused(inp, chunk_size=C)
    check_close_order(o, of, o_ref, "o")
    check_close_order(hT, hf, h_ref, "hT")


def test_split_pipelined_final_state_in_place_and_absent():
    """hT aliasing h0 (each chain reads h0 in the first range and writes hT in the range where it
    ends), and hT not requested (the hand-over between ranges goes through the workspace)."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_custom_chunk_inputs([12000, 600], 2, 128, 128, torch.bfloat16, h0_std=0.02, seed=41,
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
    check_same(o2, o, o_ref, "o")
