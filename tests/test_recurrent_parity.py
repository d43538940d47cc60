"""kda_recurrent_step (HIP) against the fp64 oracle.

Workload: 256 sequences x 32 heads, dk = dv = 128, fp32 state ~ N(0, 0.02^2),
one decode token or a replay of 8 draft tokens, bf16 q/k/v (q, k unit-norm),
per-channel log_alpha = -softplus(N(0,1)), beta = sigmoid(N(0,1)).
Tolerance (bf16 inputs): max |err| <= 2e-2 * RMS(reference), for o and for the
updated state separately; fp32 inputs: max |err| <= 1e-4.  Token counts 1, 3, 5, 6 and
8 are covered on every (dk, dv) shape.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import oracle

pytestmark = pytest.mark.gpu


def errs(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else x
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.abs(x - ref).max()), rms


def run_case(n_tokens, n_seqs=None, dk=128, dv=128, dtype=torch.bfloat16, seed=None):
    import kimi_delta_attention_06_amd as kda
    w = kda_inputs.DecodeWorkload("t", kda_inputs.DECODE_256x32.n_seqs, 32, dk, dv, 0.02, dtype, 1005)
    inp = kda_inputs.make_decode_inputs(w, n_tokens, device="cuda", n_seqs=n_seqs, seed=seed)
    S_host = inp["S"].cpu()
    o = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S_host)
    return o, inp["S"], o_ref, S_ref


@pytest.mark.parametrize("n_tokens", [1, 6, 8])
def test_decode_workload_matches_oracle(n_tokens):
    print("decode 256x32 d128 n_tokens=%d" % n_tokens, flush=True)
    o, S, o_ref, S_ref = run_case(n_tokens)
    eo, ro = errs(o, o_ref)
    es, rs = errs(S, S_ref)
    print("o max err %.3e rms %.3e | S max err %.3e rms %.3e" % (eo, ro, es, rs))
    assert eo <= 2e-2 * ro and es <= 2e-2 * rs
    # the decode path is fp32 end to end: far inside the bound
    assert eo <= 1e-5 and es <= 1e-5


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("n_tokens", [1, 3, 5, 6, 8])
def test_decode_shapes_fp32_inputs(dk, dv, n_tokens):
    o, S, o_ref, S_ref = run_case(n_tokens, n_seqs=5, dk=dk, dv=dv, dtype=torch.float32, seed=77 + n_tokens)
    eo, _ = errs(o, o_ref)
    es, _ = errs(S, S_ref)
    assert eo <= 1e-4 and es <= 1e-4


def test_decode_is_deterministic():
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_decode_inputs(kda_inputs.DECODE_256x32, 8, device="cuda", n_seqs=16)
    S1 = inp["S"].clone()
    S2 = inp["S"].clone()
    o1 = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S1)
    o2 = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_successive_steps_equal_one_replay():
    """Eight 1-token steps == one 8-token replay (same state, same outputs up to rounding)."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_decode_inputs(kda_inputs.DECODE_256x32, 8, device="cuda", n_seqs=8)
    S_a = inp["S"].clone()
    o_a = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S_a)
    S_b = inp["S"].clone()
    outs = []
    for t in range(8):
        sl = lambda x: x[:, t:t + 1].contiguous()
        outs.append(kda.recurrent_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_alpha"]),
                                       sl(inp["beta"]), S_b))
    torch.cuda.synchronize()
    o_b = torch.cat(outs, dim=1)
    assert (o_a - o_b).abs().max().item() <= 1e-5
    assert (S_a - S_b).abs().max().item() <= 1e-5


def run_verify(n_tokens, commit, dk=128, dv=128, dtype=torch.bfloat16, seed=None):
    import kimi_delta_attention_06_amd as kda
    w = kda_inputs.DecodeWorkload("t", kda_inputs.DECODE_256x32.n_seqs, 32, dk, dv, 0.02, dtype, 1005)
    inp = kda_inputs.make_decode_inputs(w, n_tokens, device="cuda", n_seqs=len(commit), seed=seed)
    S_host = inp["S"].cpu()
    nc = torch.tensor(commit, dtype=torch.int32, device="cuda")
    o = kda.recurrent_verify(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S"], nc)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_recurrent_verify(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S_host,
                                               np.asarray(commit))
    return o, inp["S"], o_ref, S_ref, S_host


def test_verify_commits_per_sequence_prefix():
    """Replay + verify, 8 tokens: per-sequence commit counts 0..8 (and out-of-range values, clamped)."""
    commit = [0, 1, 2, 3, 4, 5, 6, 7, 8, -3, 11, 8, 0, 5, 2, 7]
    print("verify n_tokens=8 commit=%s" % commit, flush=True)
    o, S, o_ref, S_ref, S0 = run_verify(8, commit, seed=91)
    eo, ro = errs(o, o_ref)
    es, rs = errs(S, S_ref)
    print("o max err %.3e rms %.3e | S max err %.3e rms %.3e" % (eo, ro, es, rs))
    assert eo <= 1e-5 and es <= 1e-5
    # nothing committed: the state is not written at all (bit-identical)
    for i, c in enumerate(commit):
        if c <= 0:
            assert torch.equal(S[i].cpu(), S0[i])


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("n_tokens", [1, 5, 6, 8])
def test_verify_shapes_fp32_inputs(dk, dv, n_tokens):
    commit = [n_tokens, 0, 1, n_tokens - 1, 3]
    o, S, o_ref, S_ref, _ = run_verify(n_tokens, commit, dk=dk, dv=dv, dtype=torch.float32, seed=5 + n_tokens)
    eo, _ = errs(o, o_ref)
    es, _ = errs(S, S_ref)
    assert eo <= 1e-4 and es <= 1e-4


def test_verify_with_full_commit_equals_step():
    """n_commit = n_tokens everywhere is kda_recurrent_step, bit for bit."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_decode_inputs(kda_inputs.DECODE_256x32, 8, device="cuda", n_seqs=12, seed=93)
    S1 = inp["S"].clone()
    o1 = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S1)
    S2 = inp["S"].clone()
    o2 = kda.recurrent_verify(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S2,
                              torch.full((12,), 8, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_steep_decay_rows():
    """Rows decaying by 60-80 nats over the call (state rows driven to ~0) beside ordinary ones."""
    import kimi_delta_attention_06_amd as kda
    inp = kda_inputs.make_decode_inputs(kda_inputs.DECODE_256x32, 8, device="cuda", n_seqs=6, seed=95)
    inp["log_alpha"][1, :, 3, :16] = -10.0   # sequence 1, head 3: 80 nats over 8 tokens
    inp["log_alpha"][4, :, :, 100:] = -7.6   # sequence 4, all heads: 60.8 nats
    S0 = inp["S"].cpu()
    o = kda.recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_recurrent_step(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S0)
    eo, _ = errs(o, o_ref)
    es, _ = errs(inp["S"], S_ref)
    print("steep decay: o max err %.3e | S max err %.3e" % (eo, es))
    assert eo <= 1e-5 and es <= 1e-5
