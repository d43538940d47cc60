"""Pins of the oracle's backward (reverse mode of the recurrence), independent of its code:

* central finite differences of the (separately pinned) forward oracle, for every input
  that has a gradient (q, k, v, log_alpha, beta, h0) on a small packed batch with a
  nonzero initial state and nonzero output / final-state cotangents;
* the chain rule across a split: one sequence run as two halves, the second half's dh0
  fed to the first half as its dhT, gives the gradients of the whole;
* beta = 0 (pure decay): dv and dbeta's write-side terms vanish exactly as the algebra
  says (dv = 0), and dlog_alpha sums to the decay's sensitivity read off finite differences.
"""
import numpy as np
import pytest

import oracle


def make(lens, H=2, dk=3, dv=4, seed=0, beta_zero=False):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk)).astype(np.float32) * 0.7
    k = rng.standard_normal((T, H, dk)).astype(np.float32) * 0.7
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    la = (-0.4 * np.log1p(np.exp(rng.standard_normal((T, H, dk))))).astype(np.float32)
    be = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    if beta_zero:
        be[:] = 0.0
    h0 = (0.3 * rng.standard_normal((len(lens), H, dk, dv))).astype(np.float32)
    do = rng.standard_normal((T, H, dv)).astype(np.float32)
    dhT = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(q=q, k=k, v=v, la=la, be=be, h0=h0, do=do, dhT=dhT, cu=cu)


def loss(d):
    o, hT = oracle.kda_fwd(d["q"], d["k"], d["v"], d["la"], d["be"], d["h0"], d["cu"])
    return float((o * d["do"]).sum() + (hT * d["dhT"]).sum())


def grads(d):
    return oracle.kda_bwd(d["q"], d["k"], d["v"], d["la"], d["be"], d["h0"], d["cu"], d["do"], d["dhT"])


NAME = {"q": "dq", "k": "dk", "v": "dv", "la": "dlog_alpha", "be": "dbeta", "h0": "dh0"}


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    d = make([5, 3, 1], seed=seed)
    g = grads(d)
    eps = 1e-2  # inputs are fp32: the central difference's rounding error stays ~1e-5 relative
    for key, gname in NAME.items():
        x = d[key]
        fd = np.zeros(x.shape)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + eps
            lp = loss(d)
            x[idx] = x0 - eps
            lm = loss(d)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * eps)
        err = np.abs(fd - g[gname]).max()
        scale = max(np.abs(fd).max(), 1e-3)
        assert err <= 2e-3 * scale, (gname, err, scale)


def test_chain_rule_across_a_split():
    """The second half's dh0 is the first half's dhT: two half runs give the whole run's gradients."""
    whole = make([8], seed=3)
    g = grads(whole)
    a = {kk: (vv[:4] if kk in ("q", "k", "v", "la", "be", "do") else vv) for kk, vv in whole.items()}
    b = {kk: (vv[4:] if kk in ("q", "k", "v", "la", "be", "do") else vv) for kk, vv in whole.items()}
    a["cu"] = np.array([0, 4], dtype=np.int64)
    b["cu"] = np.array([0, 4], dtype=np.int64)
    _, hT_a = oracle.kda_fwd(a["q"], a["k"], a["v"], a["la"], a["be"], a["h0"], a["cu"])
    b["h0"] = hT_a.astype(np.float32)
    gb = grads(b)
    a["dhT"] = gb["dh0"].astype(np.float32)
    ga = grads(a)
    for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
        both = np.concatenate([ga[key], gb[key]], axis=0)
        assert np.allclose(both, g[key], rtol=1e-5, atol=1e-6), key
    assert np.allclose(ga["dh0"], g["dh0"], rtol=1e-5, atol=1e-6)


def test_beta_zero_has_no_write_gradient():
    """With beta = 0 nothing is written: v has no influence, so dv = 0 exactly."""
    d = make([6], seed=5, beta_zero=True)
    g = grads(d)
    assert np.all(g["dv"] == 0.0)
    assert np.abs(g["dbeta"]).max() > 0  # beta still matters at first order
