"""KDA oracle (test infrastructure only).

A plain fp64 CPU evaluation of the Kimi Delta Attention recurrence, token by
token, written in C (``kda_oracle.c``) and loaded with ctypes.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library never does, and this package never imports the HIP path.

Pins: the oracle is checked against closed forms, exact rational arithmetic,
finite-difference gradients and brute-force dense unrolling in
``tests/test_oracle_*.py``; the backward (`kda_bwd`) against central finite
differences of the pinned forward and the chain rule across a sequence split;
no function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None

# IEEE fp64 without contraction or reassociation: the oracle's rounding follows the source order.
GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile the oracle library with gcc (a second or so)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc"] + GCC_FLAGS + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            lib.kda_oracle_fwd.restype = ctypes.c_int
            lib.kda_oracle_fwd.argtypes = [ctypes.c_void_p] * 7 + [
                ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            lib.kda_oracle_bwd.restype = ctypes.c_int
            lib.kda_oracle_bwd.argtypes = [ctypes.c_void_p] * 7 + [
                ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 8 + [
                ctypes.c_int]
            lib.kda_oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 / fp32 widen exactly to fp32)
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def kda_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, n_threads: int = 0):
    """Oracle forward over packed sequences.

    q, k: [T, H, dk]; v: [T, H, dv]; log_alpha: [T, H, dk]; beta: [T, H];
    h0: [N, H, dk, dv] or None; cu_seqlens: [N+1] (None = one sequence of length T).
    Returns (o [T, H, dv] float64, hT [N, H, dk, dv] float64).
    """
    q, k, v, la, be, h0 = (_f32(x) for x in (q, k, v, log_alpha, beta, h0))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and la.shape == (T, H, dk) and v.shape == (T, H, dv) and be.shape == (T, H)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    if h0 is not None:
        assert h0.shape == (N, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(h0), _ptr(cu),
                                N, T, H, dk, dv, _ptr(o), _ptr(hT), int(n_threads))
    if rc != 0:
        raise ValueError("kda oracle rejected its arguments (rc=%d)" % rc)
    return o, hT


def kda_recurrent_step(q, k, v, log_alpha, beta, S, n_threads: int = 0):
    """Oracle decode / replay: n tokens per sequence applied to state S.

    q, k: [N, n, H, dk]; v: [N, n, H, dv]; log_alpha: [N, n, H, dk]; beta: [N, n, H];
    S: [N, H, dk, dv].  Returns (o [N, n, H, dv], S_new [N, H, dk, dv]) in float64.
    The same recurrence as `kda_fwd`, with each sequence's n tokens packed and h0 = S.
    """
    q, k, v, la, be, S = (_f32(x) for x in (q, k, v, log_alpha, beta, S))
    N, n, H, dk = q.shape
    dv = v.shape[3]
    cu = np.arange(N + 1, dtype=np.int64) * n
    o, hT = kda_fwd(q.reshape(N * n, H, dk), k.reshape(N * n, H, dk), v.reshape(N * n, H, dv),
                    la.reshape(N * n, H, dk), be.reshape(N * n, H), S, cu, n_threads)
    return o.reshape(N, n, H, dv), hT


def kda_recurrent_verify(q, k, v, log_alpha, beta, S, n_commit, n_threads: int = 0):
    """Oracle replay + verify ("Kimi K3 model structure (7)", section "KDA state rollback").

    Every token of a sequence is applied in order and writes its output (the later,
    uncommitted draft tokens see the continued state); the returned state of sequence i
    is the state after its first n_commit[i] tokens (S itself for 0).  Both parts are the
    recurrence of `kda_fwd`: the outputs on all n tokens, the state on the committed
    prefix packed as its own sequences.  Returns (o [N, n, H, dv], S_new [N, H, dk, dv]).
    """
    q, k, v, la, be, S = (_f32(x) for x in (q, k, v, log_alpha, beta, S))
    n_commit = np.asarray(n_commit.cpu() if hasattr(n_commit, "cpu") else n_commit, dtype=np.int64)
    N, n, H, dk = q.shape
    dv = v.shape[3]
    o, _ = kda_recurrent_step(q, k, v, la, be, S, n_threads)
    c = np.clip(n_commit, 0, n)
    if c.sum() == 0:
        return o, S.astype(np.float64)
    cu = np.concatenate([[0], np.cumsum(c)]).astype(np.int64)
    take = lambda x: np.concatenate([x[i, :c[i]] for i in range(N)], axis=0)
    _, S_new = kda_fwd(take(q), take(k), take(v), take(la), take(be), S, cu, n_threads)
    return o, S_new


def kda_bwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, do=None, dhT=None, n_threads: int = 0):
    """Oracle backward (reverse mode of `kda_fwd`, written out in ``kda_oracle.c``).

    Gradients of  sum_t o_t . do_t + sum hT . dhT  with respect to q, k, v, log_alpha, beta and h0.
    Shapes as `kda_fwd`; do: [T, H, dv]; dhT: [N, H, dk, dv] or None (zeros).
    Returns a dict of float64 arrays: dq, dk, dlog_alpha [T, H, dk]; dv [T, H, dv]; dbeta [T, H];
    dh0 [N, H, dk, dv].
    """
    q, k, v, la, be, h0, do, dhT = (_f32(x) for x in (q, k, v, log_alpha, beta, h0, do, dhT))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert do is not None and do.shape == (T, H, dv)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = len(cu) - 1
    if dhT is not None:
        assert dhT.shape == (N, H, dk, dv)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dlog_alpha=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)), dh0=np.zeros((N, H, dk, dv)))
    rc = _load().kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(h0), _ptr(cu), N, T, H, dk, dv,
                                _ptr(do), _ptr(dhT), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), int(n_threads))
    if rc != 0:
        raise ValueError("kda oracle (backward) rejected its arguments (rc=%d)" % rc)
    return out
