"""fp64 NumPy model of the chunkwise-parallel KDA form (test infrastructure).

KDA is computed chunk-wise: parallel inside a chunk, recurrent across chunks
("Kimi K3 technical report summary", section 1, pre-training table, KDA row);
the transition of one token, (I - b k k^T) Diag(a), is diagonal plus rank one,
hence the "DPLR chunk kernel" named in "Kimi K3 NPU Training", section "NPU
operator support".  The pages state no chunk formulas; the algebra below is
derived from the token recurrence and is checked here against the oracle for
every chunk size.  It is the algebra the HIP kernel implements; this model
shares no code with that kernel.

For one chunk with rows r = 0..C-1, entering state S0 and per-channel
cumulative log-decay g_r = sum_{i<=r} log a_i:
  A[r, i]  = b_r sum_c k_rc k_ic exp(g_rc - g_ic)       (i < r, strictly lower)
  M[r, i]  =     sum_c q_rc k_ic exp(g_rc - g_ic)       (i <= r)
  T        = (I + A)^-1
  W        = T Diag(b) (K * exp(G)),   Ut = T Diag(b) V
  U        = Ut - W S0
  O        = (Q * exp(G)) S0 + M U
  S_next   = Diag(exp(g_last)) S0 + (K * exp(g_last - G))^T U
Partial chunks are padded with q = k = v = 0, log a = 0, b = 0, which leaves the
result exact (padded rows give zero rows of U and identity rows of T).

`sub` selects the overflow-safe evaluation of A and M used by the kernel: the
chunk is cut into sub-blocks of `sub` rows; a pair of sub-blocks (R > I) uses
the last row of block I as the reference (both factors <= 1), and a diagonal
sub-block uses the in-block cumulative decay (left factor <= 1, right factor
>= 1, bounded by the decay across one sub-block).
"""
import numpy as np


def _gram_plain(X, K, G):
    return (X * np.exp(G)) @ (K * np.exp(-G)).T


def _gram_blocked(X, K, G, sub):
    C = X.shape[0]
    out = np.zeros((C, C))
    nb = (C + sub - 1) // sub
    for R in range(nb):
        r0, r1 = R * sub, min(C, (R + 1) * sub)
        ref_in = G[r0 - 1] if r0 > 0 else np.zeros(G.shape[1])
        c = G[r0:r1] - ref_in  # in-block cumulative decay (<= 0)
        # diagonal sub-block
        out[r0:r1, r0:r1] = (X[r0:r1] * np.exp(c)) @ (K[r0:r1] * np.exp(-c)).T
        for I in range(R):
            i0, i1 = I * sub, (I + 1) * sub
            rho = G[i1 - 1]
            left = X[r0:r1] * np.exp(G[r0:r1] - rho)
            right = K[i0:i1] * np.exp(rho - G[i0:i1])
            out[r0:r1, i0:i1] = left @ right.T
    return out


def chunk_step(Q, K, V, LA, B, S0, sub=None):
    """One chunk (rows already padded to the chunk size). Returns (O, S_next)."""
    C = Q.shape[0]
    G = np.cumsum(LA, axis=0)
    gram = _gram_plain if sub is None else (lambda X, Kk, Gg: _gram_blocked(X, Kk, Gg, sub))
    lower_strict = np.tril(np.ones((C, C)), -1).astype(bool)
    lower = np.tril(np.ones((C, C))).astype(bool)
    A = np.where(lower_strict, B[:, None] * gram(K, K, G), 0.0)
    M = np.where(lower, gram(Q, K, G), 0.0)
    T = np.linalg.inv(np.eye(C) + A)
    W = T @ (B[:, None] * K * np.exp(G))
    Ut = T @ (B[:, None] * V)
    U = Ut - W @ S0
    O = (Q * np.exp(G)) @ S0 + M @ U
    S = np.exp(G[-1])[:, None] * S0 + (K * np.exp(G[-1] - G)).T @ U
    return O, S


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size=64, sub=None):
    """Chunked forward over packed sequences; same shapes and outputs as the oracle."""
    q, k, v, la, be = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    C = chunk_size
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.asarray(h0[n, h], dtype=np.float64).copy()
            for s in range(a, b, C):
                e = min(b, s + C)
                L = e - s
                pad = lambda x, w: np.concatenate([x[s:e, h], np.zeros((C - L,) + x.shape[2:])]) if w else x[s:e, h]
                Q, K, V, LA = (pad(x, True) for x in (q, k, v, la))
                Bv = np.concatenate([be[s:e, h], np.zeros(C - L)])
                O, S = chunk_step(Q, K, V, LA, Bv, S, sub)
                o[s:e, h] = O[:L]
            hT[n, h] = S
    return o, hT


def gram_factored_f32(X, K, LA, sub=16, limit_nats=160.0):
    """The decay-scaled Gram G[r, i] = sum_c X_rc K_ic exp(g_rc - g_ic) (i <= r) of one chunk,
    evaluated in fp32 with the factorisation the chunk kernel uses (a model of its arithmetic,
    for checking exponent ranges on the CPU).

    g is the running sum of LA over the chunk's rows.  Rows are cut into sub-blocks of `sub`;
    c is the in-sub-block cumulative decay and s its total per channel:
      * a channel whose sub-block decays by at most `limit_nats` is balanced around the block's
        middle: left X e^{c - s/2}, right K e^{s/2 - c}, both at most e^{|s|/2};
      * a wider channel is referenced to the block start: left X e^{c} (<= 1) with the
        diagonal sub-block formed element by element from e^{c_r - c_i} (<= 1);
      * sub-block pairs R > I: left X_r e^{c_r} e^{G_{R-1} - G_I} (built from the stored
        block factors), right K_i e^{s_I - c_i}, all <= 1.
    Each step's decay is floored at 2^-160 (about -111 nats), as in the kernel.  Returns the
    fp32 Gram (lower triangle incl. the diagonal; the upper part zero) and whether every
    operand stayed finite.
    """
    f = np.float32
    X, K = X.astype(f), K.astype(f)
    l2 = f(1.4426950408889634)
    cx_step = np.maximum(LA.astype(f) * l2, f(-160.0))
    C, D = X.shape
    nb = (C + sub - 1) // sub
    lim = f(limit_nats) * l2
    out = np.zeros((C, C), f)
    finite = True
    c_all, s_all, own, b2 = [], [], [], []
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        for R in range(nb):
            r0, r1 = R * sub, min(C, (R + 1) * sub)
            c = np.cumsum(cx_step[r0:r1], axis=0, dtype=f)
            s = c[-1]
            exact = s < -lim
            c_all.append(c)
            s_all.append(s)
            own.append(np.where(exact, f(1.0), np.exp2(s / 2)).astype(f))
            b2.append(np.where(exact, np.exp2(s), np.exp2(s / 2) ** 2).astype(f))
            # diagonal sub-block
            left = np.where(exact, X[r0:r1] * np.exp2(c), X[r0:r1] * np.exp2(c - s / 2))
            right = np.where(exact, f(0.0), K[r0:r1] * np.exp2(s / 2 - c))
            finite &= bool(np.isfinite(left).all() and np.isfinite(right).all())
            bal = np.where(exact, f(0.0), left) @ right.T
            L = r1 - r0
            ex = np.zeros((L, L), f)
            for r in range(L):
                for i in range(r + 1):
                    e = np.exp2(np.minimum(c[r] - c[i], f(0.0)))
                    ex[r, i] = np.sum(np.where(exact, X[r0 + r] * K[r0 + i] * e, f(0.0)), dtype=f)
            out[r0:r1, r0:r1] = np.tril(bal + ex)
        for R in range(nb):
            r0, r1 = R * sub, min(C, (R + 1) * sub)
            c, s = c_all[R], s_all[R]
            exact = s < -lim
            qL = np.where(exact, X[r0:r1] * np.exp2(c), X[r0:r1] * np.exp2(c - s / 2))
            for I in range(R):
                i0, i1 = I * sub, (I + 1) * sub
                fac = own[R].copy()
                for J in range(I + 1, R):
                    fac = fac * b2[J]
                left = qL * fac
                right = K[i0:i1] * np.exp2(s_all[I] - c_all[I])
                finite &= bool(np.isfinite(left).all() and np.isfinite(right).all())
                out[r0:r1, i0:i1] = left @ right.T
    return out, finite
