"""KDA (Kimi Delta Attention) operator for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in include/kda.h (libkda.so).  This module
only checks and marshals arguments; every step of the computation runs in the
HIP kernels.  PyTorch provides device memory and the current stream.

    o, hT = chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size=64)
    o, hT, ckpt = chunk_fwd_checkpointed(..., ckpt_every=512)  # + states every 512 tokens
    o, hT = chunk_fwd_split(...)                          # two passes, for few (sequence, head) chains
    o, hT = chunk_fwd_split_noalloc(...)                  # the same with the library's own workspace
    g = backward(q, k, v, log_alpha, beta, do, h0=None, cu_seqlens=None, dhT=None)  # dq, dk, dv, ...
    g = backward(..., method="recurrent")                # token by token, no decay bound
    o = recurrent_step(q, k, v, log_alpha, beta, S)      # updates S in place
    o = recurrent_verify(q, k, v, log_alpha, beta, S, n_commit)  # commits a prefix per sequence

Shapes: q, k [T, H, dk]; v [T, H, dv]; log_alpha [T, H, dk] fp32; beta [T, H]
fp32; h0/hT [N, H, dk, dv] fp32; cu_seqlens [N+1] int32.  A leading batch
dimension [B, T, ...] is accepted for fixed-length input.  recurrent_step and
recurrent_verify take tokens as [N, n, H, d] and S as [N, H, dk, dv];
recurrent_verify also takes n_commit [N] int32 (tokens whose updates are kept).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

__all__ = ["chunk_fwd", "chunk_fwd_checkpointed", "chunk_fwd_split", "chunk_fwd_split_noalloc", "chunk_fwd_auto",
           "chunk_fwd_split_workspace_bytes",
           "backward", "backward_workspace_bytes", "recurrent_step", "recurrent_verify", "KDAError"]


class KDAError(RuntimeError):
    pass


def _check(code: int, what: str):
    if code == _lib.KDA_OK:
        return
    msg = "%s failed: %s" % (what, _lib.status_string(code))
    if code in (_lib.KDA_ERR_INVALID_ARGUMENT, _lib.KDA_ERR_UNSUPPORTED):
        raise ValueError(msg)
    raise KDAError(msg)


def _dtype_code(*ts):
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt:
            raise ValueError("q, k, v must share one dtype, got %s" % [x.dtype for x in ts])
    if dt == torch.bfloat16:
        return _lib.KDA_DTYPE_BF16
    if dt == torch.float32:
        return _lib.KDA_DTYPE_F32
    raise ValueError("q, k, v must be bfloat16 or float32, got %s" % dt)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def chunk_fwd(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size: int = 64,
              output_final_state: bool = True, o: Optional[torch.Tensor] = None,
              hT: Optional[torch.Tensor] = None):
    """Chunkwise KDA forward; returns (o fp32 [T, H, dv], hT fp32 [N, H, dk, dv] or None)."""
    o, hT, _ = _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT, 0, None)
    return o, hT


def chunk_fwd_split(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size: int = 64,
                    output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                    hT: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """`chunk_fwd` as two passes (bf16 inputs): the in-chunk work of every chunk in parallel, then the
    state pass; for inputs with few (sequence, head) chains.  `workspace` (uint8, at least the size the
    library reports) is allocated when not given.  Returns (o, hT)."""
    o, hT, _ = _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT, 0, None,
                      split=True, workspace=workspace)
    return o, hT


def chunk_fwd_auto(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size: int = 64,
                   output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                   hT: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """The chunked forward on whichever of `chunk_fwd_split` and `chunk_fwd` is faster for the input's shape
    (kda_chunk_fwd_auto; the rule is in kda.h).  `workspace` as for `chunk_fwd_split` (allocated when not
    given and the input is bf16).  Returns (o, hT)."""
    o, hT, _ = _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT, 0, None,
                      split="auto", workspace=workspace)
    return o, hT


def chunk_fwd_split_noalloc(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size: int = 64,
                            output_final_state: bool = True, o: Optional[torch.Tensor] = None,
                            hT: Optional[torch.Tensor] = None):
    """`chunk_fwd_split` with the library's own per-GPU workspace (kda_chunk_fwd_split_noalloc): the C call
    allocates nothing.  Pass preallocated `o` (and `hT`) to keep the whole call free of allocation, e.g. under
    HIP graph capture.  Calls on one GPU share the workspace and must not overlap in time."""
    o, hT, _ = _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT, 0, None,
                      split="noalloc")
    return o, hT


def chunk_fwd_split_workspace_bytes(n_seqs: int, total_tokens: int, n_heads: int, dk: int, dv: int,
                                    chunk_size: int = 64) -> int:
    """Bytes of workspace `chunk_fwd_split` needs for bf16 inputs of these sizes."""
    need = ctypes.c_size_t(0)
    rc = _lib.load().kda_chunk_fwd_split_workspace_size(int(n_seqs), int(total_tokens), int(n_heads), int(dk),
                                                        int(dv), int(chunk_size), _lib.KDA_DTYPE_BF16,
                                                        ctypes.byref(need))
    _check(rc, "kda_chunk_fwd_split_workspace_size")
    return int(need.value)


def chunk_fwd_checkpointed(q, k, v, log_alpha, beta, h0=None, cu_seqlens=None, chunk_size: int = 64,
                           ckpt_every: int = 512, output_final_state: bool = True,
                           o: Optional[torch.Tensor] = None, hT: Optional[torch.Tensor] = None,
                           ckpt: Optional[torch.Tensor] = None):
    """chunk_fwd that also returns ckpt fp32 [T // ckpt_every, H, dk, dv]: the state of sequence n after
    p tokens (p a positive multiple of ckpt_every) is in slot (start_n + p) // ckpt_every - 1."""
    return _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT,
                  int(ckpt_every), ckpt)


def _chunk(q, k, v, log_alpha, beta, h0, cu_seqlens, chunk_size, output_final_state, o, hT, ckpt_every, ckpt,
           split=False, workspace=None):
    lib = _lib.load()
    batched = q.dim() == 4
    if batched:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires packed [T, H, d] inputs")
        B, T = q.shape[0], q.shape[1]
        q, k, v = q.reshape(B * T, *q.shape[2:]), k.reshape(B * T, *k.shape[2:]), v.reshape(B * T, *v.shape[2:])
        log_alpha = log_alpha.reshape(B * T, *log_alpha.shape[2:])
        beta = beta.reshape(B * T, *beta.shape[2:])
        n_seqs = B
    dev = q.device
    q, k, v = _dev(q, "q", device=dev), _dev(k, "k", device=dev), _dev(v, "v", device=dev)
    code = _dtype_code(q, k, v)
    log_alpha = _dev(log_alpha, "log_alpha", torch.float32, dev)
    beta = _dev(beta, "beta", torch.float32, dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [T, H, dk] and v [T, H, dv]")
    T_total, H, dk = q.shape
    dv = v.shape[2]
    if log_alpha.shape != q.shape or beta.shape != (T_total, H):
        raise ValueError("expected log_alpha [T, H, dk] and beta [T, H]")
    if cu_seqlens is not None:
        cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
    elif not batched:
        n_seqs = 1 if T_total > 0 else 0
    h0 = _dev(h0, "h0", torch.float32, dev)
    if h0 is not None and tuple(h0.shape) != (n_seqs, H, dk, dv):
        raise ValueError("h0 must be [N, H, dk, dv] = %s" % ((n_seqs, H, dk, dv),))
    if o is None:
        o = torch.empty(T_total, H, dv, dtype=torch.float32, device=dev)
    else:
        o = _dev(o, "o", torch.float32, dev)
        if tuple(o.shape) != (T_total, H, dv):
            raise ValueError("o must be [T, H, dv]")
    if output_final_state:
        if hT is None:
            hT = torch.empty(n_seqs, H, dk, dv, dtype=torch.float32, device=dev)
        else:
            hT = _dev(hT, "hT", torch.float32, dev)
            if tuple(hT.shape) != (n_seqs, H, dk, dv):
                raise ValueError("hT must be [N, H, dk, dv]")
    else:
        hT = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    if split == "noalloc":
        rc = lib.kda_chunk_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                             _ptr(cu_seqlens), n_seqs, T_total, H, dk, dv, int(chunk_size), code,
                                             _ptr(o), _ptr(hT), stream)
        _check(rc, "kda_chunk_fwd_split_noalloc")
    elif split == "auto" and code != _lib.KDA_DTYPE_BF16:
        # (fp32 inputs: the fused kernel, no workspace)
        rc = lib.kda_chunk_fwd_auto(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                    _ptr(cu_seqlens), n_seqs, T_total, H, dk, dv, int(chunk_size), code, _ptr(o),
                                    _ptr(hT), None, 0, stream)
        _check(rc, "kda_chunk_fwd_auto")
    elif split:
        need = ctypes.c_size_t(0)
        rc = lib.kda_chunk_fwd_split_workspace_size(n_seqs, T_total, H, dk, dv, int(chunk_size), code,
                                                    ctypes.byref(need))
        _check(rc, "kda_chunk_fwd_split_workspace_size")
        if workspace is None:
            workspace = torch.empty(max(int(need.value), 16), dtype=torch.uint8, device=dev)
        else:
            workspace = _dev(workspace, "workspace", torch.uint8, dev)
        fn, name = ((lib.kda_chunk_fwd_auto, "kda_chunk_fwd_auto") if split == "auto"
                    else (lib.kda_chunk_fwd_split, "kda_chunk_fwd_split"))
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens), n_seqs,
                T_total, H, dk, dv, int(chunk_size), code, _ptr(o), _ptr(hT), _ptr(workspace), workspace.numel(),
                stream)
        _check(rc, name)
    elif ckpt_every == 0:
        rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                               _ptr(cu_seqlens), n_seqs, T_total, H, dk, dv, int(chunk_size), code, _ptr(o),
                               _ptr(hT), stream)
        _check(rc, "kda_chunk_fwd")
    else:
        if ckpt_every < 0:
            raise ValueError("ckpt_every must be positive")
        n_slots = T_total // ckpt_every
        if ckpt is None:
            ckpt = torch.empty(n_slots, H, dk, dv, dtype=torch.float32, device=dev)
        else:
            ckpt = _dev(ckpt, "ckpt", torch.float32, dev)
            if tuple(ckpt.shape) != (n_slots, H, dk, dv):
                raise ValueError("ckpt must be [T // ckpt_every, H, dk, dv] = %s" % ((n_slots, H, dk, dv),))
        rc = lib.kda_chunk_fwd_checkpointed(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0),
                                            _ptr(cu_seqlens), n_seqs, T_total, H, dk, dv, int(chunk_size), code,
                                            _ptr(o), _ptr(hT), int(ckpt_every), _ptr(ckpt), stream)
        _check(rc, "kda_chunk_fwd_checkpointed")
    if batched:
        o = o.view(B, T, H, dv)
    return o, hT, ckpt


def backward(q, k, v, log_alpha, beta, do, h0=None, cu_seqlens=None, dhT=None,
             workspace: Optional[torch.Tensor] = None, method: str = "chunk"):
    """Gradients of sum(o * do) + sum(hT * dhT) for the forward of `chunk_fwd` on the same inputs.

    q, k, v, log_alpha, beta, h0, cu_seqlens as `chunk_fwd` (packed [T, H, d] or batched [B, T, H, d]);
    do like o; dhT like hT (None: zeros).  `workspace` (uint8, at least `backward_workspace_bytes`) is
    allocated when not given.  method "chunk" (kda_bwd, 16-token chunks on the fp32 matrix core) or
    "recurrent" (kda_bwd_recurrent, token by token, no decay bound).  Returns a dict: dq, dk, dv,
    dlog_alpha (shapes of their inputs), dbeta, dh0 [N, H, dk, dv].
    """
    if method not in ("chunk", "recurrent"):
        raise ValueError("method must be 'chunk' or 'recurrent'")
    lib = _lib.load()
    batched = q.dim() == 4
    if batched:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens requires packed [T, H, d] inputs")
        B, Tb = q.shape[0], q.shape[1]
        flat = lambda x: x.reshape(B * Tb, *x.shape[2:]) if x is not None else None
        q, k, v, log_alpha, beta, do = (flat(x) for x in (q, k, v, log_alpha, beta, do))
        n_seqs = B
    dev = q.device
    q, k, v = _dev(q, "q", device=dev), _dev(k, "k", device=dev), _dev(v, "v", device=dev)
    code = _dtype_code(q, k, v)
    log_alpha = _dev(log_alpha, "log_alpha", torch.float32, dev)
    beta = _dev(beta, "beta", torch.float32, dev)
    do = _dev(do, "do", torch.float32, dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q, k [T, H, dk] and v [T, H, dv]")
    T_total, H, dk = q.shape
    dv = v.shape[2]
    if log_alpha.shape != q.shape or beta.shape != (T_total, H) or do.shape != v.shape:
        raise ValueError("expected log_alpha [T, H, dk], beta [T, H] and do [T, H, dv]")
    if cu_seqlens is not None:
        cu_seqlens = _dev(cu_seqlens, "cu_seqlens", torch.int32, dev)
        n_seqs = cu_seqlens.numel() - 1
    elif not batched:
        n_seqs = 1 if T_total > 0 else 0
    h0 = _dev(h0, "h0", torch.float32, dev)
    dhT = _dev(dhT, "dhT", torch.float32, dev)
    for name, x in (("h0", h0), ("dhT", dhT)):
        if x is not None and tuple(x.shape) != (n_seqs, H, dk, dv):
            raise ValueError("%s must be [N, H, dk, dv] = %s" % (name, (n_seqs, H, dk, dv)))
    out = dict(dq=torch.empty(T_total, H, dk, dtype=torch.float32, device=dev),
               dk=torch.empty(T_total, H, dk, dtype=torch.float32, device=dev),
               dv=torch.empty(T_total, H, dv, dtype=torch.float32, device=dev),
               dlog_alpha=torch.empty(T_total, H, dk, dtype=torch.float32, device=dev),
               dbeta=torch.empty(T_total, H, dtype=torch.float32, device=dev),
               dh0=torch.empty(n_seqs, H, dk, dv, dtype=torch.float32, device=dev))
    need = backward_workspace_bytes(n_seqs, T_total, H, dk, dv, method)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    else:
        workspace = _dev(workspace, "workspace", torch.uint8, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    name = "kda_bwd" if method == "chunk" else "kda_bwd_recurrent"
    rc = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(h0), _ptr(cu_seqlens),
                            n_seqs, T_total, H, dk, dv, code, _ptr(do), _ptr(dhT), _ptr(out["dq"]), _ptr(out["dk"]),
                            _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dh0"]),
                            _ptr(workspace), workspace.numel(), stream)
    _check(rc, name)
    if batched:
        for key in ("dq", "dk", "dv", "dlog_alpha", "dbeta"):
            out[key] = out[key].view(B, Tb, *out[key].shape[1:])
    return out


def backward_workspace_bytes(n_seqs: int, total_tokens: int, n_heads: int, dk: int, dv: int,
                             method: str = "chunk") -> int:
    """Bytes of workspace `backward` needs with this method."""
    need = ctypes.c_size_t(0)
    name = "kda_bwd_workspace_size" if method == "chunk" else "kda_bwd_recurrent_workspace_size"
    rc = getattr(_lib.load(), name)(int(n_seqs), int(total_tokens), int(n_heads), int(dk), int(dv),
                                    ctypes.byref(need))
    _check(rc, name)
    return int(need.value)


def _recurrent(fn_name, q, k, v, log_alpha, beta, S, n_commit, o):
    lib = _lib.load()
    dev = S.device
    q, k, v = _dev(q, "q", device=dev), _dev(k, "k", device=dev), _dev(v, "v", device=dev)
    code = _dtype_code(q, k, v)
    log_alpha = _dev(log_alpha, "log_alpha", torch.float32, dev)
    beta = _dev(beta, "beta", torch.float32, dev)
    S = _dev(S, "S", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q, k [N, n, H, dk] and v [N, n, H, dv]")
    N, n, H, dk = q.shape
    dv = v.shape[3]
    if log_alpha.shape != q.shape or beta.shape != (N, n, H) or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("expected log_alpha [N, n, H, dk], beta [N, n, H], S [N, H, dk, dv]")
    if o is None:
        o = torch.empty(N, n, H, dv, dtype=torch.float32, device=dev)
    else:
        o = _dev(o, "o", torch.float32, dev)
        if tuple(o.shape) != (N, n, H, dv):
            raise ValueError("o must be [N, n, H, dv]")
    stream = torch.cuda.current_stream(dev).cuda_stream
    if fn_name == "kda_recurrent_step":
        rc = lib.kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                    N, n, H, dk, dv, code, _ptr(o), stream)
    else:
        n_commit = _dev(n_commit, "n_commit", torch.int32, dev)
        if tuple(n_commit.shape) != (N,):
            raise ValueError("n_commit must be [N] int32")
        rc = lib.kda_recurrent_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                      _ptr(n_commit), N, n, H, dk, dv, code, _ptr(o), stream)
    _check(rc, fn_name)
    return o


def recurrent_step(q, k, v, log_alpha, beta, S, o: Optional[torch.Tensor] = None):
    """Decode / replay of n tokens per sequence: updates S [N, H, dk, dv] in place, returns o [N, n, H, dv]."""
    return _recurrent("kda_recurrent_step", q, k, v, log_alpha, beta, S, None, o)


def recurrent_verify(q, k, v, log_alpha, beta, S, n_commit, o: Optional[torch.Tensor] = None):
    """Replay + verify: every token writes o [N, n, H, dv]; S [N, H, dk, dv] keeps the state after the
    first n_commit[i] tokens of sequence i (unchanged for 0); the later (draft) updates are dropped."""
    return _recurrent("kda_recurrent_verify", q, k, v, log_alpha, beta, S, n_commit, o)
