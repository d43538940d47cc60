"""Seeded random configurations of every entry point against the fp64 oracle.

Each case draws its own shape from a fixed numpy seed: number of sequences, their
lengths (empty, single-token, ragged and multi-chunk), heads, dk and dv, chunk size,
input dtype, gate law (x1 or x0.1), initial state present or absent, and for the
decode entry points the token count and per-sequence commit counts.  Inputs are the
same laws as the workloads (kda_inputs).  Tolerances are the ones of the other parity
tests: bf16 inputs max |err| <= 2e-2 * RMS(ref) per output tensor, fp32 inputs
max |err| <= 1e-4 for the forward and the decode paths; gradients max |err| <=
1e-3 * RMS(ref) per gradient.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle

pytestmark = pytest.mark.gpu


def to64(x):
    return x.detach().cpu().double().numpy()


def check(name, x, ref, dtype, tol_rel=2e-2, tol_abs=1e-4):
    x = to64(x).reshape(ref.shape)
    assert np.isfinite(x).all(), name
    if ref.size == 0:
        return
    err = float(np.abs(x - ref).max())
    rms = float(np.sqrt(np.mean(ref ** 2)))
    print("  %-10s max|err| %.3e rms %.3e" % (name, err, rms), flush=True)
    if dtype == torch.float32:
        assert err <= tol_abs, (name, err)
    else:
        assert err <= tol_rel * rms, (name, err, rms)


def chunk_case(seed):
    r = np.random.default_rng(seed)
    dtype = torch.bfloat16 if r.random() < 0.6 else torch.float32
    dk, dv = int(r.choice([64, 128])), int(r.choice([64, 128]))
    if dtype == torch.float32 and dk == 128:
        C = int(r.choice([16, 32]))
    else:
        C = int(r.choice([16, 32, 64]))
    n = int(r.integers(1, 6))
    lens = [int(x) for x in r.choice([0, 1, 5, 16, 63, 64, 65, 130, 257, 300], size=n)]
    if sum(lens) == 0:
        lens[0] = 77
    return dict(lens=lens, H=int(r.integers(1, 5)), dk=dk, dv=dv, C=C, dtype=dtype,
                gate=float(r.choice([1.0, 0.1])), h0_std=float(r.choice([0.0, 0.02])), seed=seed)


@pytest.mark.parametrize("seed", range(2000, 2016))
def test_chunk_fwd_random_configs(seed):
    import kimi_delta_attention_06_amd as kda
    c = chunk_case(seed)
    print("chunk fuzz %s" % c, flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(c["lens"], c["H"], c["dk"], c["dv"], c["dtype"], gate_scale=c["gate"],
                                              h0_std=c["h0_std"], seed=seed, device="cuda")
    o_ref, h_ref = oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"],
                                  inp["cu_seqlens"])
    o, hT = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], chunk_size=c["C"])
    torch.cuda.synchronize()
    check("o", o, o_ref, c["dtype"])
    check("hT", hT, h_ref, c["dtype"])
    if c["dtype"] == torch.bfloat16:  # the two-pass path takes bf16 inputs
        o2, h2 = kda.chunk_fwd_split(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], h0=inp["h0"],
                                     cu_seqlens=inp["cu_seqlens"], chunk_size=c["C"])
        torch.cuda.synchronize()
        check("o split", o2, o_ref, c["dtype"])
        check("hT split", h2, h_ref, c["dtype"])


@pytest.mark.parametrize("seed", range(3000, 3012))
def test_decode_and_verify_random_configs(seed):
    import kimi_delta_attention_06_amd as kda
    r = np.random.default_rng(seed)
    dtype = torch.bfloat16 if r.random() < 0.5 else torch.float32
    dk, dv = int(r.choice([64, 128])), int(r.choice([64, 128]))
    n_tok, n_seqs, H = int(r.integers(1, 9)), int(r.integers(1, 7)), int(r.integers(1, 5))
    print("decode fuzz: %s dk=%d dv=%d n_tokens=%d seqs=%d heads=%d" % (dtype, dk, dv, n_tok, n_seqs, H), flush=True)
    w = kda_inputs.DecodeWorkload("fuzz", n_seqs, H, dk, dv, 0.02, dtype, seed)
    inp = kda_inputs.make_decode_inputs(w, n_tok, device="cuda", seed=seed)
    S0 = inp["S"].cpu()
    # the plain step
    S = inp["S"].clone()
    o = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S0)
    check("o", o, o_ref, torch.float32)
    check("S", S, S_ref, torch.float32)
    # replay + verify with random commit counts (including 0 and n_tokens)
    commit = r.integers(0, n_tok + 1, size=n_seqs).astype(np.int32)
    S = inp["S"].clone()
    ov = kda.recurrent_verify(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S,
                              torch.from_numpy(commit).cuda())
    torch.cuda.synchronize()
    ov_ref, Sv_ref = oracle.kda_recurrent_verify(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S0,
                                                 commit)
    check("o verify", ov, ov_ref, torch.float32)
    check("S verify", S, Sv_ref, torch.float32)


@pytest.mark.parametrize("seed", range(4000, 4006))
def test_backward_random_configs(seed):
    import kimi_delta_attention_06_amd as kda
    c = chunk_case(seed)
    print("backward fuzz %s" % c, flush=True)
    inp = kda_inputs.make_custom_chunk_inputs(c["lens"], c["H"], c["dk"], c["dv"], c["dtype"], gate_scale=c["gate"],
                                              h0_std=c["h0_std"], seed=seed, device="cuda")
    g = torch.Generator(device="cpu").manual_seed(seed)
    T, H = inp["v"].shape[0], inp["v"].shape[1]
    do = torch.randn(T, H, c["dv"], generator=g).cuda()
    dhT = (0.1 * torch.randn(len(c["lens"]), H, c["dk"], c["dv"], generator=g)).cuda()
    ref = oracle.kda_bwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["h0"], inp["cu_seqlens"],
                         do, dhT)
    for method in ("chunk", "recurrent"):
        gb = kda.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], do, h0=inp["h0"],
                          cu_seqlens=inp["cu_seqlens"], dhT=dhT, method=method)
        torch.cuda.synchronize()
        for name in ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dh0"):
            if name == "dh0" and inp["h0"] is None:
                continue
            check("%s %s" % (method, name), gb[name], ref[name], torch.bfloat16, tol_rel=1e-3)
