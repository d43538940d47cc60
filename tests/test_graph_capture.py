"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on the capture stream).

The library launches kernels only (no allocation, memset or synchronisation on the call
path), so a captured call must replay to the same bits as the eager call.  Each graph is
replayed three times, with the program's own eager launches and a device synchronisation
between the replays, and every replay is compared with the eager result bit for bit; the
outputs are filled with NaN before each replay so that a replay that writes nothing fails.
"""
import pytest
import torch

import kda_inputs

pytestmark = pytest.mark.gpu


def capture(body):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()  # first launches outside the capture (per-device kernel attributes are set here)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    return g


def eager_noise(inp):
    """Unrelated eager work between replays: another launch of the same library on other buffers."""
    import kimi_delta_attention_06_amd as kda
    o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], chunk_size=64)
    torch.randn(1 << 16, device="cuda").sum()
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("split", [False, True])
def test_chunk_fwd_graph_replays_match_eager(split):
    import kimi_delta_attention_06_amd as kda
    print("graph chunk_fwd split=%s" % split, flush=True)
    inp = kda_inputs.make_custom_chunk_inputs([300, 64, 1, 0, 129], 4, 128, 128, torch.bfloat16, h0_std=0.02,
                                              seed=91, device="cuda")
    T, H = inp["v"].shape[0], inp["v"].shape[1]
    o = torch.empty(T, H, 128, dtype=torch.float32, device="cuda")
    hT = torch.empty(5, H, 128, 128, dtype=torch.float32, device="cuda")
    ws = None
    if split:
        ws = torch.empty(kda.chunk_fwd_split_workspace_bytes(5, T, H, 128, 128, 64), dtype=torch.uint8,
                         device="cuda")

    def body():
        if split:
            kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                                cu_seqlens=inp["cu_seqlens"], chunk_size=64, o=o, hT=hT, workspace=ws)
        else:
            kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], chunk_size=64, o=o, hT=hT)

    body()
    torch.cuda.synchronize()
    o_e, h_e = o.clone(), hT.clone()
    g = capture(body)
    for rep in range(3):
        o.fill_(float("nan"))
        hT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_e), rep
        assert torch.equal(hT, h_e), rep
        eager_noise(inp)


def test_decode_loop_graph_replays_match_eager():
    """Four decode steps (one token each, state updated in place) and one replay + verify step,
    captured as one graph; the state is reset eagerly before each replay."""
    import kimi_delta_attention_06_amd as kda
    print("graph decode loop", flush=True)
    w = kda_inputs.DecodeWorkload("graph", 6, 4, 128, 128, 0.02, torch.bfloat16, 5)
    steps = [kda_inputs.make_decode_inputs(w, 1, device="cuda", seed=500 + i) for i in range(4)]
    ver = kda_inputs.make_decode_inputs(w, 5, device="cuda", seed=600)
    commit = torch.tensor([0, 1, 5, 3, 2, 4], dtype=torch.int32, device="cuda")
    S0 = steps[0]["S"].clone()
    S = S0.clone()
    outs = [torch.empty(6, 1, 4, 128, dtype=torch.float32, device="cuda") for _ in steps]
    o_ver = torch.empty(6, 5, 4, 128, dtype=torch.float32, device="cuda")

    def body():
        for d, o in zip(steps, outs):
            kda.recurrent_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S, o=o)
        kda.recurrent_verify(ver["q"], ver["k"], ver["v"], ver["log_alpha"], ver["beta"], S, commit, o=o_ver)

    body()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [o_ver.clone(), S.clone()]
    S.copy_(S0)
    g = capture(body)
    noise = kda_inputs.make_custom_chunk_inputs([200], 2, 128, 128, torch.bfloat16, seed=3, device="cuda")
    for rep in range(3):
        S.copy_(S0)
        for o in outs + [o_ver]:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(outs + [o_ver, S], ref)):
            assert torch.equal(x, r), (rep, i)
        eager_noise(noise)


def test_backward_graph_replays_match_eager():
    """kda_bwd captured as one graph: its four launches, with the reverse pass forked to a second
    stream beside the forward-states pass and joined back through events (one workgroup of each
    per CU when chains x dv/64 <= 256, as here)."""
    import kimi_delta_attention_06_amd as kda
    print("graph backward", flush=True)
    inp = kda_inputs.make_custom_chunk_inputs([300, 64, 1, 0, 129], 4, 128, 128, torch.bfloat16, h0_std=0.02,
                                              seed=93, device="cuda")
    T, H = inp["v"].shape[0], inp["v"].shape[1]
    g0 = torch.Generator(device="cpu").manual_seed(94)
    do = torch.randn(T, H, 128, generator=g0).cuda()
    dhT = (0.1 * torch.randn(5, H, 128, 128, generator=g0)).cuda()
    ws = torch.empty(kda.backward_workspace_bytes(5, T, H, 128, 128), dtype=torch.uint8, device="cuda")
    keys = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0")

    def body():
        return kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, h0=inp["h0"],
                            cu_seqlens=inp["cu_seqlens"], dhT=dhT, workspace=ws)

    ref = body()
    torch.cuda.synchronize()
    ref = {key: ref[key].clone() for key in keys}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = body()
    torch.cuda.synchronize()
    for rep in range(3):
        for key in keys:
            out[key].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in keys:
            assert torch.equal(out[key], ref[key]), (rep, key)
        eager_noise(inp)
