"""Rotary position embedding (RoPE) in front of the attention definition (test infrastructure).

The "Flash Attention" notes (14cs17), section "Flash Attention 2 Improvements", list RoPE among
the features FlashAttention-2 supports and say nothing else about it. The readings taken here
(also listed in the design notes):

  * RoPE is the rotary position embedding: the head dimension is cut into d/2 pairs, and pair i
    of a row at position p is rotated by the angle p * theta_i, theta_i = base^(-2 i / d)
    (base 10000 for the standard tables): (a, b) -> (a cos - b sin, a sin + b cos), which is the
    complex product (a + i b) e^(i p theta_i). Query and key rows are rotated by their own
    positions, so their dot product depends on the positions only through their difference.
  * The pairs are either neighbours (2 i, 2 i + 1) ("interleaved") or the two halves of the row
    (i, i + d/2). The caller supplies the cos and sin tables, fp32 [positions, d/2];
    ``rotary_tables`` builds the standard ones.
  * Positions count inside each sequence: key j is at position j; the Nq queries of a chunk
    against Nk keys are the last Nq positions, query t at Nk - Nq + t (the alignment of the
    causal mask), and a position below 0 (queries beyond the keys) is taken as 0.
  * Precision: every rotated element is formed in fp32 from two fp32 products, each rounded,
    and their rounded difference or sum (no fused multiply-add), and then rounded to the input
    type (fp16 or bf16) with round-to-nearest-even. Attention then runs on those rotated and
    rounded Q and K. ``rotate_exact`` is the same rotation in float64 without any rounding;
    the pins bound the difference.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .definition import _key_segments, attention, attention_rows


def rotary_tables(positions: int, head_dim: int, base: float = 10000.0
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of p * theta_i for p < positions and i < head_dim / 2, in float64."""
    if head_dim % 2:
        raise ValueError("RoPE needs an even head dimension")
    theta = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    angle = np.arange(positions, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(angle), np.sin(angle)


def rope_pairs(head_dim: int, interleaved: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Element indices (first, second) of the d/2 rotated pairs; pair i uses frequency i."""
    i = np.arange(head_dim // 2)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + head_dim // 2


def rotate_exact(x: np.ndarray, cos_rows: np.ndarray, sin_rows: np.ndarray,
                 interleaved: bool) -> np.ndarray:
    """x [..., N, d] rotated row by row with the table rows [N, d/2], in float64."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos_rows, dtype=np.float64)
    s = np.asarray(sin_rows, dtype=np.float64)
    ia, ib = rope_pairs(x.shape[-1], interleaved)
    a, b = x[..., ia], x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = a * c - b * s
    out[..., ib] = a * s + b * c
    return out


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values rounded to fp16 ("f16") or bf16 ("bf16"), round-to-nearest-even, returned
    as the exact float64 values of the rounded numbers."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = x32.view(np.uint32).astype(np.uint64)
        keep = (bits >> 16) & 1                      # the last bit that survives
        top = ((bits + 0x7FFF + keep) >> 16) << 16   # round half to even on the dropped 16 bits
        out = (top & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
        out[np.isnan(x32)] = np.nan
        return out
    raise ValueError(f"unknown dtype {dtype}")


def rotate_rounded(x: np.ndarray, cos_rows: np.ndarray, sin_rows: np.ndarray,
                   interleaved: bool, dtype: str) -> np.ndarray:
    """The reading's rotation: fp32 products and sums, each rounded, then rounding to dtype.

    x holds values of the input type (exact in fp32); the tables are fp32."""
    x32 = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos_rows, dtype=np.float32)
    s = np.asarray(sin_rows, dtype=np.float32)
    ia, ib = rope_pairs(x32.shape[-1], interleaved)
    a, b = x32[..., ia], x32[..., ib]
    out = np.empty_like(x32)
    out[..., ia] = (a * c) - (b * s)   # float32 arithmetic: each operation rounds once
    out[..., ib] = (a * s) + (b * c)
    return round_to_dtype(out, dtype)


def rope_positions(n_tokens: int, n_keys: Optional[int] = None) -> np.ndarray:
    """Positions of a sequence's tokens: keys 0..n-1; with n_keys, the n_tokens queries are
    the last positions of n_keys keys (n_keys - n_tokens + t, at least 0)."""
    t = np.arange(n_tokens)
    if n_keys is None:
        return t
    return np.maximum(n_keys - n_tokens + t, 0)


def apply_rope(q: np.ndarray, k: np.ndarray, cos: np.ndarray, sin: np.ndarray,
               interleaved: bool, dtype: str,
               cu_seqlens: Optional[Sequence[int]] = None,
               cu_seqlens_k: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Q [B, Hq, Nq, d] and K [B, Hkv, Nk, d] rotated by their positions (rounded per the
    reading). Packed sequences restart their positions at 0. Tables: [positions, d/2]."""
    nq, nk = q.shape[2], k.shape[2]
    qr = np.empty(q.shape, dtype=np.float64)
    kr = np.empty(k.shape, dtype=np.float64)
    for (s0, s1), (t0, t1) in _key_segments(nq, nk, cu_seqlens, cu_seqlens_k):
        pq = rope_positions(s1 - s0, t1 - t0)
        pk = rope_positions(t1 - t0)
        qr[:, :, s0:s1] = rotate_rounded(q[:, :, s0:s1], cos[pq], sin[pq], interleaved, dtype)
        kr[:, :, t0:t1] = rotate_rounded(k[:, :, t0:t1], cos[pk], sin[pk], interleaved, dtype)
    return qr, kr


def attention_rope(q, k, v, cos, sin, interleaved: bool, dtype: str, scale: float,
                   causal: bool = False, cu_seqlens=None, cu_seqlens_k=None):
    """(O, LSE) of the attention definition on RoPE-rotated Q and K."""
    qr, kr = apply_rope(q, k, cos, sin, interleaved, dtype, cu_seqlens, cu_seqlens_k)
    return attention(qr, kr, v, scale, causal, cu_seqlens=cu_seqlens, cu_seqlens_k=cu_seqlens_k)


def attention_rope_rows(q, k, v, cos, sin, interleaved: bool, dtype: str, scale: float,
                        causal: bool, rows, cu_seqlens=None, cu_seqlens_k=None):
    """``attention_rope`` for selected (batch, q_head, token) rows only."""
    qr, kr = apply_rope(q, k, cos, sin, interleaved, dtype, cu_seqlens, cu_seqlens_k)
    return attention_rows(qr, kr, v, scale, causal, rows, cu_seqlens=cu_seqlens,
                          cu_seqlens_k=cu_seqlens_k)
