"""The chunkwise algebra (fp64 NumPy model) equals the token-by-token oracle.

Chunked and recurrent evaluations must agree for every chunk size, including
chunk sizes that do not divide the sequence length (padded partial chunks) and
packed sequences (state reset at every boundary).  This validates, before any
kernel exists, the algebra the HIP chunk kernel implements.
"""
import numpy as np
import pytest

import oracle
from kda_chunk_model import chunk_fwd
from test_oracle_pins import f32, rand_inputs


def rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


@pytest.mark.parametrize("sub", [None, 4])
def test_every_chunk_size_matches_oracle(sub):
    rng = np.random.default_rng(21)
    T, H, dk, dv = 23, 2, 8, 6
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    h0 = f32(0.5 * rng.standard_normal((1, H, dk, dv)))
    o_ref, h_ref = oracle.kda_fwd(q, k, v, la, be, h0)
    for C in range(1, T + 3):
        if sub is not None and C % sub:
            continue
        o, hT = chunk_fwd(q, k, v, la, be, h0, chunk_size=C, sub=sub)
        assert rel(o, o_ref) < 1e-11, C
        assert rel(hT, h_ref) < 1e-11, C


def test_varlen_chunked_matches_oracle():
    rng = np.random.default_rng(22)
    lens = [7, 0, 16, 1, 33, 9]
    T, H, dk, dv = sum(lens), 2, 8, 8
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    h0 = f32(0.3 * rng.standard_normal((len(lens), H, dk, dv)))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_ref, h_ref = oracle.kda_fwd(q, k, v, la, be, h0, cu)
    for C, sub in [(4, None), (8, 4), (16, 4), (16, 16)]:
        o, hT = chunk_fwd(q, k, v, la, be, h0, cu, chunk_size=C, sub=sub)
        assert rel(o, o_ref) < 1e-11
        assert rel(hT, h_ref) < 1e-11


def test_blocked_factorisation_survives_strong_decay():
    """Strong per-channel decay (log a = -5 on some channels, 0 on others).

    The plain factorisation exp(g_r) * exp(-g_i) overflows once the chunk's
    cumulative decay passes ~-709 in fp64; the sub-block form stays finite as
    long as one sub-block's decay stays above that, and matches the oracle.
    """
    rng = np.random.default_rng(23)
    T, H, dk, dv = 256, 1, 8, 4
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    la[:, :, :3] = -5.0
    la[:, :, 3:5] = 0.0
    o_ref, h_ref = oracle.kda_fwd(q, k, v, la, be)
    with np.errstate(over="ignore", invalid="ignore"):
        o_plain, _ = chunk_fwd(q, k, v, la, be, chunk_size=256)
    assert not np.isfinite(o_plain).all()
    o, hT = chunk_fwd(q, k, v, la, be, chunk_size=256, sub=16)
    assert rel(o, o_ref) < 1e-11 and rel(hT, h_ref) < 1e-11


def _gram_ref(X, K, LA):
    # the decay between rows i and r as the sum of the steps in between (not a difference of
    # running sums, which a step of -1e30 would swamp)
    LA = np.asarray(LA, np.float64)
    C = X.shape[0]
    out = np.zeros((C, C))
    for r in range(C):
        for i in range(r + 1):
            out[r, i] = np.sum(X[r] * K[i] * np.exp(LA[i + 1:r + 1].sum(0)))
    return out


@pytest.mark.parametrize("law", ["wide", "mixed", "extreme"])
def test_kernel_factorisation_stays_finite_for_any_decay(law):
    """The chunk kernel's fp32 factorisation of the decay-scaled Gram (balanced sub-blocks up to
    160 nats of decay, block-start references with per-element diagonal factors beyond) keeps
    every operand finite and matches the fp64 Gram, where the balanced form alone overflows."""
    from kda_chunk_model import gram_factored_f32
    rng = np.random.default_rng({"wide": 31, "mixed": 32, "extreme": 33}[law])
    C, D = 64, 48
    X = rng.standard_normal((C, D)) / np.sqrt(D)
    K = rng.standard_normal((C, D)) / np.sqrt(D)
    LA = -np.log1p(np.exp(rng.standard_normal((C, D))))
    if law == "wide":
        LA[:, :16] = -30.0
        LA[:, 16:32] = 0.0
    elif law == "mixed":
        LA[16:32, :8] = -12.5    # one 16-token block decaying by 200 nats (exact path)
        LA[32:48, 8:16] = -9.0   # one by 144 nats (balanced, wide)
        LA[:, 40:] = -1e-3
    else:
        LA[5:60:7, :10] = -1e30
        LA[:, 10:12] = -3e3
    ref = _gram_ref(X, K, LA)
    out, finite = gram_factored_f32(X, K, LA)
    assert finite
    assert np.abs(out - ref).max() <= 2e-6 * max(1.0, np.abs(ref).max())
    # the balanced form alone overflows once a block decays by more than ~177 nats
    assert (LA.reshape(C // 16, 16, D).sum(1) < -177).any()
    _, finite_bal = gram_factored_f32(X, K, LA, limit_nats=np.inf)
    assert not finite_bal
