"""Seeded synthetic inputs for the KDA operator (shared by tests, bench and smoke).

This module draws inputs only; it contains none of the operator's arithmetic.
It is the single piece of code that both the HIP path and the oracle see.

Input laws (the workload description of a Kimi-Linear-shaped KDA layer: 32 heads
of 128 dims, "Kimi K3 NPU Training", section "Kimi Linear is not the K3 config"):

* q, k, v ~ N(0, 1); q and k are L2-normalised over the head dimension per
  (token, head) in fp32 and then cast (round-to-nearest-even) to the storage
  dtype.  The kernel never re-normalises: the values as stored are the inputs.
* log_alpha = -gate_scale * softplus(z), z ~ N(0, 1), one value per
  (token, head, key channel): the channel-wise forget gate in log space.
* beta = sigmoid(z'), z' ~ N(0, 1), one value per (token, head).
* h0 (when present) ~ N(0, h0_std^2), fp32 [n_seqs, H, dk, dv].

Draw order inside one generator: q, k, v, log_alpha, beta, then h0 / S.  Long
inputs are drawn in token slices (each slice draws q, k, v, log_alpha, beta in
that order), which keeps the temporary fp32 buffers small.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ChunkWorkload:
    name: str
    n_seqs: int
    seq_len: Optional[int]  # None -> seeded random lengths (varlen)
    total_tokens: int
    n_heads: int
    dk: int
    dv: int
    chunk_size: int
    dtype: torch.dtype  # storage dtype of q, k, v
    gate_scale: float
    h0_std: float  # 0 -> no initial state
    seed: int
    min_len: int = 0


TINY_FP32 = ChunkWorkload("tiny-fp32", 1, 256, 256, 2, 64, 64, 16, torch.float32, 1.0, 0.0, 1001)
KIMI_LINEAR_LAYER = ChunkWorkload("kimi-linear-layer-bf16", 4, 4096, 16384, 32, 128, 128, 64,
                                  torch.bfloat16, 0.1, 0.0, 1002)
VARLEN_PACKED = ChunkWorkload("varlen-packed-bf16", 8, None, 32768, 32, 128, 128, 64,
                              torch.bfloat16, 1.0, 0.02, 1003, min_len=256)
LONG_CONTEXT = ChunkWorkload("long-context-1m-bf16", 1, 1048576, 1048576, 32, 128, 128, 64,
                             torch.bfloat16, 1.0, 0.0, 1004)

# the 1M-token sequence with 4 heads (32 heads spread over 8 GPUs): few chains, so the split
# path's state pass runs over segments in parallel
LONG_CONTEXT_4H = ChunkWorkload("long-context-1m-4heads-bf16", 1, 1048576, 1048576, 4, 128, 128, 64,
                                torch.bfloat16, 1.0, 0.0, 1006)

CHUNK_WORKLOADS = {w.name: w for w in (TINY_FP32, KIMI_LINEAR_LAYER, VARLEN_PACKED, LONG_CONTEXT, LONG_CONTEXT_4H)}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    n_seqs: int
    n_heads: int
    dk: int
    dv: int
    state_std: float
    dtype: torch.dtype
    seed: int


DECODE_256x32 = DecodeWorkload("decode-256seq-h32-d128", 256, 32, 128, 128, 0.02, torch.bfloat16, 1005)


# ---------------------------------------------------------------------------
# Helpers
# ---------------------------------------------------------------------------


def varlen_lengths(total: int, n_seqs: int, min_len: int, seed: int) -> np.ndarray:
    """Sequence lengths summing to `total`, each >= min_len, seeded (numpy PCG64)."""
    rng = np.random.default_rng(seed)
    extra = rng.multinomial(total - n_seqs * min_len, [1.0 / n_seqs] * n_seqs)
    return (min_len + extra).astype(np.int64)


def cu_seqlens_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu.astype(np.int32)


def long_context_oracle_heads(seed: int = 1004, n_heads: int = 32, count: int = 2) -> np.ndarray:
    """The seeded heads on which the 1M-token workload is checked against the oracle."""
    return np.sort(np.random.default_rng(seed).choice(n_heads, count, replace=False))


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    # L2 normalisation of the last dim in fp32 (input construction, not operator math)
    return x / torch.sqrt((x * x).sum(dim=-1, keepdim=True))


def _draw_tokens(gen, shape_tok, n_heads, dk, dv, dtype, gate_scale, device):
    """Draw q, k, v, log_alpha, beta for `shape_tok` token positions (a tuple)."""
    f32 = torch.float32
    q = torch.randn(*shape_tok, n_heads, dk, generator=gen, device=device, dtype=f32)
    q = _unit_rows(q).to(dtype)
    k = torch.randn(*shape_tok, n_heads, dk, generator=gen, device=device, dtype=f32)
    k = _unit_rows(k).to(dtype)
    v = torch.randn(*shape_tok, n_heads, dv, generator=gen, device=device, dtype=f32).to(dtype)
    z = torch.randn(*shape_tok, n_heads, dk, generator=gen, device=device, dtype=f32)
    log_alpha = -gate_scale * torch.nn.functional.softplus(z)
    zb = torch.randn(*shape_tok, n_heads, generator=gen, device=device, dtype=f32)
    beta = torch.sigmoid(zb)
    return q, k, v, log_alpha.contiguous(), beta.contiguous()


def make_chunk_inputs(w: ChunkWorkload, device="cpu", total_tokens: Optional[int] = None,
                      slice_tokens: int = 65536, seed: Optional[int] = None) -> dict:
    """Inputs for `kda_chunk_fwd` on workload `w` (token-major [T_total, H, d]).

    `total_tokens` overrides the workload's length (fixed-length workloads keep
    n_seqs and scale seq_len; varlen keeps n_seqs and redraws lengths).
    """
    seed = w.seed if seed is None else seed
    T_total = w.total_tokens if total_tokens is None else int(total_tokens)
    if w.seq_len is None:
        min_len = min(w.min_len, T_total // w.n_seqs)
        lens = varlen_lengths(T_total, w.n_seqs, min_len, seed)
    else:
        assert T_total % w.n_seqs == 0
        lens = np.full(w.n_seqs, T_total // w.n_seqs, dtype=np.int64)
    cu = cu_seqlens_from_lengths(lens)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    H, dk, dv = w.n_heads, w.dk, w.dv
    q = torch.empty(T_total, H, dk, dtype=w.dtype, device=device)
    k = torch.empty_like(q)
    v = torch.empty(T_total, H, dv, dtype=w.dtype, device=device)
    la = torch.empty(T_total, H, dk, dtype=torch.float32, device=device)
    be = torch.empty(T_total, H, dtype=torch.float32, device=device)
    for t0 in range(0, T_total, slice_tokens):
        t1 = min(T_total, t0 + slice_tokens)
        qs, ks, vs, las, bes = _draw_tokens(gen, (t1 - t0,), H, dk, dv, w.dtype, w.gate_scale, device)
        q[t0:t1], k[t0:t1], v[t0:t1], la[t0:t1], be[t0:t1] = qs, ks, vs, las, bes
        del qs, ks, vs, las, bes
    h0 = None
    if w.h0_std > 0:
        h0 = w.h0_std * torch.randn(w.n_seqs, H, dk, dv, generator=gen, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=be, h0=h0,
                cu_seqlens=torch.from_numpy(cu).to(device), chunk_size=w.chunk_size,
                lens=lens, seed=seed, workload=w.name)


def make_decode_inputs(w: DecodeWorkload, n_tokens: int, device="cpu", n_seqs: Optional[int] = None,
                       seed: Optional[int] = None, gate_scale: float = 1.0) -> dict:
    """Inputs for `kda_recurrent_step`: tokens [N, n_tokens, H, d] and state S [N, H, dk, dv]."""
    seed = (w.seed + 100 * n_tokens) if seed is None else seed
    N = w.n_seqs if n_seqs is None else int(n_seqs)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q, k, v, la, be = _draw_tokens(gen, (N, n_tokens), w.n_heads, w.dk, w.dv, w.dtype, gate_scale, device)
    S = w.state_std * torch.randn(N, w.n_heads, w.dk, w.dv, generator=gen, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=be, S=S, seed=seed, workload=w.name)


def make_custom_chunk_inputs(lens, n_heads, dk, dv, dtype=torch.bfloat16, gate_scale=1.0, h0_std=0.0,
                             seed=0, device="cpu") -> dict:
    """Free-form varlen inputs for edge-case tests (lengths may be 0)."""
    lens = np.asarray(lens, dtype=np.int64)
    cu = cu_seqlens_from_lengths(lens)
    T_total = int(cu[-1])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q, k, v, la, be = _draw_tokens(gen, (T_total,), n_heads, dk, dv, dtype, gate_scale, device)
    h0 = None
    if h0_std > 0:
        h0 = h0_std * torch.randn(len(lens), n_heads, dk, dv, generator=gen, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=be, h0=h0,
                cu_seqlens=torch.from_numpy(cu).to(device), lens=lens, seed=seed)


# ---------------------------------------------------------------------------
# Adversarial inputs for edge-case tests (input construction only)
# ---------------------------------------------------------------------------

ADVERSARIAL_KINDS = ("wide_decay", "large_values", "small_values", "parallel_keys")


def make_adversarial_chunk_inputs(kind: str, lens, n_heads, dk, dv, dtype=torch.bfloat16, seed=0,
                                  device="cpu") -> dict:
    """Draws as make_custom_chunk_inputs (h0 ~ N(0, 0.02^2)), then changes one aspect:

    * wide_decay: log_alpha = -30 on the first third of the key channels (480 nats per 16 tokens:
      the channel forgets everything every token) and exactly 0 on the second third;
    * large_values: v ~ N(0, 2500^2) before the cast (|v| up to about 1e4) and h0 ~ N(0, 300^2);
    * small_values: v ~ N(0, 1e-10) before the cast and h0 ~ N(0, 1e-14) (magnitudes near 1e-5
      and 1e-7, below fp16's normal range);
    * parallel_keys: beta = 1, and the keys of every 8 consecutive tokens are one unit direction
      plus noise of 1e-3 per coordinate (renormalised), with every other key an exact repeat of
      the one before.
    """
    if kind not in ADVERSARIAL_KINDS:
        raise ValueError("unknown kind %r" % kind)
    inp = make_custom_chunk_inputs(lens, n_heads, dk, dv, dtype=dtype, h0_std=0.02, seed=seed, device=device)
    T = int(inp["cu_seqlens"][-1])
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 7919)
    f32 = torch.float32
    if kind == "wide_decay":
        third = dk // 3
        inp["log_alpha"][:, :, :third] = -30.0
        inp["log_alpha"][:, :, third:2 * third] = 0.0
    elif kind in ("large_values", "small_values"):
        vs, hs = (2500.0, 300.0) if kind == "large_values" else (1e-5, 1e-7)
        inp["v"] = (vs * torch.randn(T, n_heads, dv, generator=gen, device=device, dtype=f32)).to(dtype)
        inp["h0"] = hs * torch.randn(len(lens), n_heads, dk, dv, generator=gen, device=device, dtype=f32)
    else:
        n_dir = (T + 7) // 8
        base = torch.randn(n_dir, n_heads, dk, generator=gen, device=device, dtype=f32)
        base = _unit_rows(base).repeat_interleave(8, dim=0)[:T]
        k = _unit_rows(base + 1e-3 * torch.randn(T, n_heads, dk, generator=gen, device=device, dtype=f32))
        k[1::2] = k[0::2][: k[1::2].shape[0]]
        inp["k"] = k.to(dtype)
        inp["beta"] = torch.ones(T, n_heads, device=device, dtype=f32)
    return inp
