"""Pins for the fp64 oracle: closed forms, exact arithmetic, brute force, calculus.

None of these re-types the oracle's loop.  Each targets a mistake the oracle
could plausibly make: decaying columns instead of key rows, erasing before the
decay, a wrong sign on the delta term, reading out before the write, a
transposed state, a wrong stride between heads or sequences, a state that leaks
across a packed boundary.

The recurrence being pinned (KDA: delta rule with a channel-wise forget gate,
"Kimi K3 technical report summary", section 1, pre-training table, KDA row):
  S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f32(x):
    """Round to fp32 (the oracle reads fp32-representable inputs) and return fp64."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def rand_inputs(rng, T, H, dk, dv, gate=1.0, unit=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -gate * np.log1p(np.exp(rng.standard_normal((T, H, dk))))
    be = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return tuple(f32(x) for x in (q, k, v, la, be))


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- closed forms


def test_beta_zero_is_pure_channel_decay():
    """beta = 0: S_t = Diag(exp(sum_{i<=t} log a_i)) S_0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(1)
    T, H, dk, dv = 37, 3, 16, 12
    q, k, v, la, _ = rand_inputs(rng, T, H, dk, dv)
    be = np.zeros((T, H))
    h0 = f32(rng.standard_normal((1, H, dk, dv)))
    o, hT = oracle.kda_fwd(q, k, v, la, be, h0)
    g = np.cumsum(la, axis=0)  # [T, H, dk]
    for h in range(H):
        for t in (0, 5, T - 1):
            St = np.exp(g[t, h])[:, None] * h0[0, h]
            assert rel(o[t, h], St.T @ q[t, h]) < 1e-13
        assert rel(hT[0, h], np.exp(g[T - 1, h])[:, None] * h0[0, h]) < 1e-13


def hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def test_orthonormal_keys_exact_overwrite():
    """alpha = 1, beta = 1, orthonormal keys: a write replaces the value stored under k.

    Keys are Hadamard rows / 4 (d = 16), exactly orthonormal in binary.
    With h0 = 0 and distinct keys, o_t = sum_{i<=t} (k_i . q_t) v_i; after a
    repeated key, S^T k returns the most recent value written under it.
    """
    rng = np.random.default_rng(2)
    d, dv = 16, 8
    K = hadamard(d) / 4.0
    T = 24
    order = list(range(d)) + [3, 7, 3, 0, 15, 7, 9, 3]
    k = K[order][:, None, :]
    q = f32(rng.standard_normal((T, 1, d)))
    v = f32(rng.standard_normal((T, 1, dv)))
    la = np.zeros((T, 1, d))
    be = np.ones((T, 1))
    o, hT = oracle.kda_fwd(q, k, v, la, be)
    # first d tokens: distinct keys
    for t in range(d):
        expect = sum((k[i, 0] @ q[t, 0]) * v[i, 0] for i in range(t + 1))
        assert np.abs(o[t, 0] - expect).max() < 1e-13
    # final state: each key returns its last written value
    last = {}
    for t, key in enumerate(order):
        last[key] = t
    S = hT[0, 0]
    for key, t in last.items():
        assert np.abs(S.T @ K[key] - v[t, 0]).max() < 1e-13


def test_single_token_closed_form_order_of_decay_and_erase():
    """T = 1: S_1 = D h0 + b k (v - (D h0)^T k)^T with D = Diag(alpha); o = S_1^T q.

    Distinguishes decay-then-erase from erase-then-decay and catches a sign error.
    """
    rng = np.random.default_rng(3)
    H, dk, dv = 2, 8, 6
    q, k, v, la, be = rand_inputs(rng, 1, H, dk, dv)
    h0 = f32(rng.standard_normal((1, H, dk, dv)))
    o, hT = oracle.kda_fwd(q, k, v, la, be, h0)
    for h in range(H):
        Dh0 = np.exp(la[0, h])[:, None] * h0[0, h]
        S1 = Dh0 + be[0, h] * np.outer(k[0, h], v[0, h] - Dh0.T @ k[0, h])
        assert rel(hT[0, 0 + h], S1) < 1e-14
        assert rel(o[0, h], S1.T @ q[0, h]) < 1e-14
        # with h0 = 0 the state is the outer product b k v^T and o = b (q.k) v
    o0, hT0 = oracle.kda_fwd(q, k, v, la, be)
    for h in range(H):
        assert rel(hT0[0, h], be[0, h] * np.outer(k[0, h], v[0, h])) < 1e-15
        assert rel(o0[0, h], be[0, h] * (q[0, h] @ k[0, h]) * v[0, h]) < 1e-14


def test_partial_beta_moves_readout_toward_value():
    """Unit k, 0<b<1: S_t^T k_t = (1-b) S'^T k_t + b v_t with S' = Diag(a_t) S_{t-1}."""
    rng = np.random.default_rng(4)
    T, dk, dv = 6, 8, 5
    q, k, v, la, be = rand_inputs(rng, T, 1, dk, dv)
    h0 = f32(rng.standard_normal((1, 1, dk, dv)))
    S_prev = h0[0, 0]
    for t in range(T):
        _, hT = oracle.kda_fwd(q[: t + 1], k[: t + 1], v[: t + 1], la[: t + 1], be[: t + 1], h0)
        Sp = np.exp(la[t, 0])[:, None] * S_prev
        kt = k[t, 0]
        nk = kt @ kt  # = 1 up to fp32 rounding of k
        lhs = hT[0, 0].T @ kt
        rhs = (1 - be[t, 0] * nk) * (Sp.T @ kt) + be[t, 0] * nk * v[t, 0]
        assert np.abs(lhs - rhs).max() < 1e-13
        S_prev = hT[0, 0]


def test_delta_write_is_a_gradient_step_on_the_regression_loss():
    """S_t = S' - b grad L(S'), L(S) = 1/2 |S^T k - v|^2 (finite differences, no formula reuse)."""
    rng = np.random.default_rng(5)
    dk, dv = 4, 3
    q, k, v, la, be = rand_inputs(rng, 1, 1, dk, dv)
    h0 = f32(rng.standard_normal((1, 1, dk, dv)))
    _, hT = oracle.kda_fwd(q, k, v, la, be, h0)
    Sp = np.exp(la[0, 0])[:, None] * h0[0, 0]

    def loss(S):
        r = S.T @ k[0, 0] - v[0, 0]
        return 0.5 * r @ r

    grad = np.zeros_like(Sp)
    eps = 1e-5
    for c in range(dk):
        for j in range(dv):
            E = np.zeros_like(Sp)
            E[c, j] = eps
            grad[c, j] = (loss(Sp + E) - loss(Sp - E)) / (2 * eps)
    assert np.abs(hT[0, 0] - (Sp - be[0, 0] * grad)).max() < 1e-9


def test_exact_rational_example():
    """A 3-token, 2-channel example evaluated in exact rational arithmetic.

    q, k, v, beta and h0 are dyadic (exact in fp32).  The gate enters as fp32 log(alpha);
    the exact computation uses alpha = exp(fp32 log(alpha)) as a rational, so the only
    differences left are the oracle's fp64 roundings (~1e-15).
    """
    F = Fraction
    la32 = np.log(np.array([[0.5, 0.75], [1.0, 0.5], [0.75, 1.0]])).astype(np.float32)
    alpha = [[F(float(np.exp(np.float64(x)))) for x in row] for row in la32]
    beta = [F(1, 2), F(1), F(1, 4)]
    k = [[F(1, 2), F(-3, 4)], [F(1), F(0)], [F(0), F(-1)]]
    q = [[F(1), F(0)], [F(3, 8), F(-5, 8)], [F(1, 2), F(1, 2)]]
    v = [[F(2), F(-1)], [F(1, 2), F(3)], [F(-1), F(1)]]
    S = [[F(1), F(0)], [F(0), F(2)]]
    outs = []
    for t in range(3):
        S = [[alpha[t][c] * S[c][j] for j in range(2)] for c in range(2)]  # decay key rows
        y = [sum(k[t][c] * S[c][j] for c in range(2)) for j in range(2)]  # k^T S
        S = [[S[c][j] - beta[t] * k[t][c] * y[j] + beta[t] * k[t][c] * v[t][j] for j in range(2)]
             for c in range(2)]
        outs.append([sum(S[c][j] * q[t][c] for c in range(2)) for j in range(2)])
    tofl = lambda a: np.array([[float(x) for x in r] for r in a])
    o, hT = oracle.kda_fwd(tofl(q)[:, None], tofl(k)[:, None], tofl(v)[:, None],
                           la32.astype(np.float64)[:, None], tofl([[b] for b in beta]),
                           tofl([[1, 0], [0, 2]])[None, None])
    assert np.abs(o[:, 0] - tofl(outs)).max() < 1e-14
    assert np.abs(hT[0, 0] - tofl(S)).max() < 1e-14


# ---------------------------------------------------------------- brute force


def test_dense_unrolling_bruteforce():
    """S_t = P_{t,0} S_0 + sum_{i<=t} P_{t,i} b_i k_i v_i^T with explicit dk x dk transitions.

    M_j = (I - b_j k_j k_j^T) Diag(a_j) and P_{t,i} = M_t ... M_{i+1} are built as dense
    matrices; o_t = S_t^T q_t.  Tiny T and d, random h0.
    """
    rng = np.random.default_rng(6)
    for T, dk, dv in [(1, 3, 2), (5, 4, 3), (8, 8, 5)]:
        q, k, v, la, be = rand_inputs(rng, T, 1, dk, dv, unit=False)
        h0 = f32(rng.standard_normal((1, 1, dk, dv)))
        o, hT = oracle.kda_fwd(q, k, v, la, be, h0)
        M = [(np.eye(dk) - be[j, 0] * np.outer(k[j, 0], k[j, 0])) @ np.diag(np.exp(la[j, 0])) for j in range(T)]

        def P(t, i):  # M_t ... M_{i+1} (identity when i == t)
            R = np.eye(dk)
            for j in range(i + 1, t + 1):
                R = M[j] @ R
            return R

        for t in range(T):
            St = P(t, -1) @ h0[0, 0] + sum(P(t, i) @ (be[i, 0] * np.outer(k[i, 0], v[i, 0])) for i in range(t + 1))
            assert rel(o[t, 0], St.T @ q[t, 0]) < 1e-12
        assert rel(hT[0, 0], St) < 1e-12


# ---------------------------------------------------------------- invariants


def test_heads_and_sequences_are_independent_and_reset():
    """Packed varlen run == separate single-head, single-sequence runs (strides and resets)."""
    rng = np.random.default_rng(7)
    lens = [5, 0, 9, 1, 13]
    T, H, dk, dv = sum(lens), 3, 6, 4
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    h0 = f32(rng.standard_normal((len(lens), H, dk, dv)))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, hT = oracle.kda_fwd(q, k, v, la, be, h0, cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        for h in range(H):
            sl = slice(h, h + 1)
            o1, h1 = oracle.kda_fwd(q[a:b, sl], k[a:b, sl], v[a:b, sl], la[a:b, sl], be[a:b, sl], h0[n:n + 1, sl])
            assert np.array_equal(o[a:b, h:h + 1], o1)
            assert np.array_equal(hT[n, h], h1[0, 0])
    # an empty sequence returns its initial state
    assert np.array_equal(hT[1], h0[1])


def test_split_and_resume():
    """run(T) == run(first m) then run(rest) with h0 = hT (the state is the whole carry).

    h0 enters as fp32, so the carried state is rounded once: agreement is to ~1e-7.
    """
    rng = np.random.default_rng(8)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    o, hT = oracle.kda_fwd(q, k, v, la, be)
    for m in (1, 17, 39):
        oa, ha = oracle.kda_fwd(q[:m], k[:m], v[:m], la[:m], be[:m])
        ob, hb = oracle.kda_fwd(q[m:], k[m:], v[m:], la[m:], be[m:], ha)
        assert rel(np.concatenate([oa, ob]), o) < 1e-6
        assert rel(hb, hT) < 1e-6


def test_linearity_in_values_and_state_and_queries():
    rng = np.random.default_rng(9)
    T, H, dk, dv = 20, 2, 8, 6
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    v2 = f32(rng.standard_normal(v.shape))
    h0 = f32(rng.standard_normal((1, H, dk, dv)))
    h02 = f32(rng.standard_normal((1, H, dk, dv)))
    q2 = f32(rng.standard_normal(q.shape))
    o1, s1 = oracle.kda_fwd(q, k, v, la, be, h0)
    o2, s2 = oracle.kda_fwd(q, k, v2, la, be, h02)
    o3, s3 = oracle.kda_fwd(q, k, v + v2, la, be, h0 + h02)  # sums are exact in fp32? use fp64 tolerance
    assert rel(o3, o1 + o2) < 1e-6 and rel(s3, s1 + s2) < 1e-6
    oq, _ = oracle.kda_fwd(q2, k, v, la, be, h0)
    oqq, _ = oracle.kda_fwd(f32(q + q2), k, v, la, be, h0)
    assert rel(oqq, o1 + oq) < 1e-6


def test_key_channel_permutation_equivariance_and_scalar_gate_case():
    """Permuting key channels of q, k, alpha jointly leaves o unchanged and permutes rows of hT.

    With the gate equal across channels (the scalar-gate delta rule), permuting
    channels of q and k alone is also an equivariance.
    """
    rng = np.random.default_rng(10)
    T, H, dk, dv = 25, 2, 8, 5
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    h0 = f32(rng.standard_normal((1, H, dk, dv)))
    perm = rng.permutation(dk)
    o, hT = oracle.kda_fwd(q, k, v, la, be, h0)
    op, hTp = oracle.kda_fwd(q[..., perm], k[..., perm], v, la[..., perm], be, h0[:, :, perm, :])
    assert rel(op, o) < 1e-13 and rel(hTp, hT[:, :, perm, :]) < 1e-13
    la_s = np.repeat(la[..., :1], dk, axis=-1)
    o_s, hT_s = oracle.kda_fwd(q, k, v, la_s, be, h0)
    o_sp, hT_sp = oracle.kda_fwd(q[..., perm], k[..., perm], v, la_s, be, h0[:, :, perm, :])
    assert rel(o_sp, o_s) < 1e-13 and rel(hT_sp, hT_s[:, :, perm, :]) < 1e-13


def test_value_channels_evolve_independently_and_threads_are_bitwise():
    """Columns of S never mix: a run on value columns [a, b) equals that slice of the full run.

    Also the OpenMP split over columns gives bit-identical results for any thread count.
    """
    rng = np.random.default_rng(11)
    T, H, dk, dv = 30, 1, 8, 32
    q, k, v, la, be = rand_inputs(rng, T, H, dk, dv)
    h0 = f32(rng.standard_normal((1, H, dk, dv)))
    o, hT = oracle.kda_fwd(q, k, v, la, be, h0, n_threads=1)
    o8, hT8 = oracle.kda_fwd(q, k, v, la, be, h0, n_threads=8)
    assert np.array_equal(o, o8) and np.array_equal(hT, hT8)
    os_, hs = oracle.kda_fwd(q, k, v[..., 8:13], la, be, h0[..., 8:13])
    assert np.array_equal(os_, o[..., 8:13]) and np.array_equal(hs, hT[..., 8:13])


def test_recurrent_step_wrapper_is_packed_forward():
    rng = np.random.default_rng(12)
    N, n, H, dk, dv = 3, 4, 2, 8, 8
    q, k, v, la, be = rand_inputs(rng, N * n, H, dk, dv)
    S = f32(rng.standard_normal((N, H, dk, dv)))
    o, S1 = oracle.kda_recurrent_step(q.reshape(N, n, H, dk), k.reshape(N, n, H, dk), v.reshape(N, n, H, dv),
                                      la.reshape(N, n, H, dk), be.reshape(N, n, H), S)
    for i in range(N):
        sl = slice(i * n, (i + 1) * n)
        o1, h1 = oracle.kda_fwd(q[sl], k[sl], v[sl], la[sl], be[sl], S[i:i + 1])
        assert np.array_equal(o[i], o1) and np.array_equal(S1[i], h1[0])


def test_replay_verify_commits_a_prefix_and_outputs_continue_from_it():
    """Replay + verify ("Kimi K3 model structure (7)", section "KDA state rollback"): the kept
    state is the one after the committed prefix, and the draft outputs are what stepping the
    drafts from that kept state gives (so o and the kept state agree at the commit point)."""
    rng = np.random.default_rng(21)
    N, n, H, dk, dv = 4, 6, 2, 8, 8
    q, k, v, la, be = (x.reshape(N, n, *x.shape[1:]) for x in rand_inputs(rng, N * n, H, dk, dv))
    S = f32(rng.standard_normal((N, H, dk, dv)))
    commit = np.array([0, 2, 6, 9])  # 9 is clamped to n
    o, Sk = oracle.kda_recurrent_verify(q, k, v, la, be, S, commit)
    o_all, S_all = oracle.kda_recurrent_step(q, k, v, la, be, S)
    assert np.array_equal(o, o_all)
    assert np.array_equal(Sk[0], S[0])                      # nothing committed: state untouched
    assert np.array_equal(Sk[2], S_all[2]) and np.array_equal(Sk[3], S_all[3])  # everything committed
    c = 2
    o_pre, S_pre = oracle.kda_recurrent_step(q[1:2, :c], k[1:2, :c], v[1:2, :c], la[1:2, :c], be[1:2, :c], S[1:2])
    assert np.array_equal(Sk[1], S_pre[0])
    o_draft, _ = oracle.kda_recurrent_step(q[1:2, c:], k[1:2, c:], v[1:2, c:], la[1:2, c:], be[1:2, c:],
                                           f32(Sk[1:2]))
    # the draft outputs continue from the kept state (to fp32 rounding of that state)
    assert rel(o[1, c:], o_draft[0]) < 1e-6
    assert np.array_equal(o[1, :c], o_pre[0])


def test_rejects_bad_cu_seqlens():
    rng = np.random.default_rng(13)
    q, k, v, la, be = rand_inputs(rng, 10, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, la, be, cu_seqlens=[0, 6, 4, 10])
    with pytest.raises(ValueError):
        oracle.kda_fwd(q, k, v, la, be, cu_seqlens=[0, 9])
