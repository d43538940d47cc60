"""kda_chunk_fwd_split_noalloc (the split forward on the library's own per-GPU workspace, for
callers that cannot allocate) against kda_chunk_fwd_split with a caller workspace, through the
C ABI: two calls in a row, the second with a smaller input, each bit-identical to the split path
with its own workspace (the same kernels on the same operands) and within the bf16 tolerance of
the fp64 oracle (max |err| <= 2e-2 * RMS(ref) for o and hT)."""
import ctypes

import pytest
import torch

import kda_inputs
import oracle
from test_chunk_parity import check_bf16

pytestmark = pytest.mark.gpu


def c_call(fn, inp, C, o, hT, ws=None):
    from kimi_delta_attention_06_amd import _lib
    lib = _lib.load()
    P = lambda t: None if t is None else t.data_ptr()
    T, H, dk = inp["q"].shape
    dv = inp["v"].shape[2]
    N = inp["cu_seqlens"].numel() - 1
    args = [P(inp["q"]), P(inp["k"]), P(inp["v"]), P(inp["log_alpha"]), P(inp["beta"]), P(inp["h0"]),
            P(inp["cu_seqlens"]), N, T, H, dk, dv, C, _lib.KDA_DTYPE_BF16, P(o), P(hT)]
    if ws is not None:
        args += [P(ws), ws.numel()]
    rc = getattr(lib, fn)(*args, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _lib.status_string(rc)
    torch.cuda.synchronize()


def test_noalloc_matches_split_on_two_calls():
    from kimi_delta_attention_06_amd import _lib
    big = kda_inputs.make_custom_chunk_inputs([1500, 900, 77, 0, 1], 8, 128, 128, torch.bfloat16, h0_std=0.02,
                                              seed=61, device="cuda")
    small = kda_inputs.make_custom_chunk_inputs([200, 33], 2, 128, 128, torch.bfloat16, seed=62, device="cuda")
    for name, inp, C in (("big", big, 64), ("small", small, 32)):
        T, H, _ = inp["q"].shape
        N = inp["cu_seqlens"].numel() - 1
        need = ctypes.c_size_t(0)
        assert _lib.load().kda_chunk_fwd_split_workspace_size(N, T, H, 128, 128, C, _lib.KDA_DTYPE_BF16,
                                                             ctypes.byref(need)) == 0
        assert need.value <= _lib.NOALLOC_SCRATCH_BYTES
        print("noalloc %s: lens %s, %d heads, chunk %d, workspace %d B" % (name, list(inp["lens"]), H, C, need.value),
              flush=True)
        ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
        o1, h1 = (torch.full((T, H, 128), float("nan"), device="cuda"),
                  torch.full((N, H, 128, 128), float("nan"), device="cuda"))
        o2, h2 = torch.full_like(o1, float("nan")), torch.full_like(h1, float("nan"))
        c_call("kda_chunk_fwd_split", inp, C, o1, h1, ws)
        c_call("kda_chunk_fwd_split_noalloc", inp, C, o2, h2)
        assert torch.equal(o1, o2) and torch.equal(h1, h2)
        check_bf16(o2, h2, *oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"],
                                           inp["cu_seqlens"]))
