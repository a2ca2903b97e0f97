"""The definition of exact attention, evaluated the slow way in float64 (test infrastructure).

Sources (restated, not copied):
  * "Flash Attention" notes (14cs17), section "Prerequisites": self-attention is softmax(Q K^T) V.
  * same page, section "Standard Attention Memory Analysis": (1) S = Q K^T is formed in full,
    (2) the softmax is taken over each row of S, (3) O = softmax(S) V.
  * FromZero2AI "FlashAttention: GPU Memory-Bound Speedups ...", section "Core Mechanisms":
    the softmax subtracts the row maximum m_i = max(x_i) before exponentiating.

Readings where the pages are silent (each also listed in the design notes):
  * a scale multiplies Q K^T before the row maximum and the exponential;
  * causal means key j is visible to query i iff j <= i (the diagonal is always visible);
  * a query chunk may be shorter or longer than its keys (chunked prefill against a key/value
    cache: the "Flash Attention" notes list the KV cache as composable with the method, and the
    xspy page pairs it with chunked prefill). The chunk's Nq queries are the last Nq positions
    of the Nk keys, so causal means key j is visible to query i iff j <= i + (Nk - Nq);
    with Nq == Nk this is the rule above. A query that sees no key gets O = 0, LSE = -inf;
  * packed variable-length sequences attend only within their own [cu[s], cu[s+1]) range
    (their keys within [cu_k[s], cu_k[s+1])), with causality measured inside the sequence;
  * grouped-query attention maps query head h to key/value head h // (Hq // Hkv);
  * the log-sum-exp output is the natural log of sum_j exp(scaled score), per query row.

Inputs are float arrays (the caller decodes fp16/bf16 bit patterns exactly); every product and
sum here runs in float64.
"""
from __future__ import annotations

from collections import defaultdict
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


def kv_head(h: int, heads_q: int, heads_kv: int) -> int:
    """Key/value head serving query head h under grouped-query attention (consecutive groups)."""
    if heads_q % heads_kv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (heads_q // heads_kv)


def _head_scores(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Step 1 of standard attention: S = scale * Q K^T for one head (rows: queries)."""
    return scale * (qh @ kh.T)


def _allowed(nq: int, nk: int, causal: bool) -> np.ndarray:
    """Visibility of key j to query i inside one sequence of nq queries and nk keys."""
    if not causal:
        return np.ones((nq, nk), dtype=bool)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return j <= i + (nk - nq)


def softmax_rows_with_lse(s: np.ndarray, allowed: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Step 2 of standard attention: row softmax over the visible entries, and log-sum-exp.

    P[i, j] = exp(S[i, j] - m_i) / l_i over visible j, with m_i the row maximum and
    l_i = sum_j exp(S[i, j] - m_i); lse_i = m_i + ln(l_i). Invisible entries get P = 0. A row
    with no visible entry gets P = 0 and lse = -inf.
    """
    any_ = allowed.any(axis=1) if allowed.shape[1] else np.zeros(allowed.shape[0], dtype=bool)
    masked = np.where(allowed, s, -np.inf)
    m = np.where(any_, masked.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(allowed, np.exp(masked - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(any_[:, None], e / np.where(any_, l, 1.0)[:, None], 0.0)
    lse = np.where(any_, m + np.log(np.where(any_, l, 1.0)), -np.inf)
    return p, lse


def _mix(p: np.ndarray, vh: np.ndarray) -> np.ndarray:
    """Step 3 of standard attention: O = P V."""
    return p @ vh


def _segments(n: int, cu_seqlens: Optional[Sequence[int]]) -> List[Tuple[int, int]]:
    if cu_seqlens is None:
        return [(0, n)]
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or cu[-1] != n or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, end at N and be non-decreasing")
    return list(zip(cu[:-1], cu[1:]))


def _key_segments(nq: int, nk: int, cu_seqlens, cu_seqlens_k):
    """Query and key ranges of every sequence (keys default to the query packing)."""
    qs = _segments(nq, cu_seqlens)
    if cu_seqlens_k is None:
        if cu_seqlens is not None and nk != nq:
            raise ValueError("packed keys of another length need their own cu_seqlens_k")
        ks = _segments(nk, cu_seqlens)
    else:
        if cu_seqlens is None:
            raise ValueError("cu_seqlens_k needs cu_seqlens")
        ks = _segments(nk, cu_seqlens_k)
        if len(ks) != len(qs):
            raise ValueError("cu_seqlens and cu_seqlens_k must describe the same sequences")
    return list(zip(qs, ks))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              cu_seqlens: Optional[Sequence[int]] = None, return_probs: bool = False,
              cu_seqlens_k: Optional[Sequence[int]] = None):
    """Exact attention by materialising S and P per (batch, head[, sequence]) in float64.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d] (Nk may differ from Nq). Returns
    (o [B, Hq, Nq, d], lse [B, Hq, Nq]) as float64, and with return_probs also the list of
    per-(b, h, segment) P matrices. Packed sequences (cu_seqlens, and cu_seqlens_k for keys
    packed differently from the queries) require B == 1.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_, hq, n, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    if k.shape != (b_, hkv, nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if cu_seqlens is not None and b_ != 1:
        raise ValueError("packed sequences need B == 1")
    o = np.zeros((b_, hq, n, d))
    lse = np.full((b_, hq, n), np.nan)
    probs = []
    for b in range(b_):
        for h in range(hq):
            hk = kv_head(h, hq, hkv)
            for (s0, s1), (t0, t1) in _key_segments(n, nk, cu_seqlens, cu_seqlens_k):
                if s1 == s0:
                    continue
                s = _head_scores(q[b, h, s0:s1], k[b, hk, t0:t1], scale)
                p, l_ = softmax_rows_with_lse(s, _allowed(s1 - s0, t1 - t0, causal))
                o[b, h, s0:s1] = _mix(p, v[b, hk, t0:t1])
                lse[b, h, s0:s1] = l_
                if return_probs:
                    probs.append(p)
    if return_probs:
        return o, lse, probs
    return o, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                   rows: Iterable[Tuple[int, int, int]],
                   cu_seqlens: Optional[Sequence[int]] = None,
                   cu_seqlens_k: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition for selected rows (b, q_head, token) only, one row at a time.

    Tokens are global (packed) indices when cu_seqlens is given. Returns (o [R, d], lse [R])
    in the order of ``rows``. K and V of a head are upcast to float64 once per head.
    """
    rows = list(rows)
    b_, hq, n, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    pairs = _key_segments(n, nk, cu_seqlens, cu_seqlens_k)
    segs = [qs for qs, _ in pairs]
    starts = np.array([a for a, _ in segs])
    o = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    by_head = defaultdict(list)
    for r, (b, h, i) in enumerate(rows):
        by_head[(b, kv_head(h, hq, hkv))].append(r)
    for (b, hk), idx in by_head.items():
        kh = np.asarray(k[b, hk], dtype=np.float64)
        vh = np.asarray(v[b, hk], dtype=np.float64)
        for r in idx:
            _, h, i = rows[r]
            seg = int(np.searchsorted(starts, i, side="right")) - 1
            while segs[seg][1] <= i:  # skip empty sequences that share a start
                seg += 1
            (s0, s1), (t0, t1) = pairs[seg]
            # visible keys: the first (i - s0) + (nk - nq) + 1 of the sequence's keys if causal
            end = min(t1, t0 + (i - s0) + ((t1 - t0) - (s1 - s0)) + 1) if causal else t1
            end = max(end, t0)
            qi = np.asarray(q[b, h, i], dtype=np.float64)
            s = _head_scores(qi[None, :], kh[t0:end], scale)
            p, l_ = softmax_rows_with_lse(s, np.ones_like(s, dtype=bool))
            o[r] = _mix(p, vh[t0:end])[0]
            lse[r] = l_[0]
    return o, lse


def score_matrix_bytes(n: int, bytes_per_element: int) -> int:
    """Bytes of one materialised N x N score matrix (what the tiled method never stores)."""
    return n * n * bytes_per_element
