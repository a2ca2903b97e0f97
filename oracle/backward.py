"""Gradients of exact attention, evaluated the slow way in float64 (test infrastructure).

What the backward pass of the method returns is the exact gradient of the forward definition
(the "Flash Attention" notes, 14cs17, Common Pitfalls, Pitfall 3, and Exercise 5; FromZero2AI
"FlashAttention: GPU Memory-Bound Speedups ...", section "Core Mechanisms", mechanism 3: the
backward pass rebuilds the scores and probabilities block by block instead of storing them,
trading compute for memory). Recomputation changes where P comes from, not what is computed,
so the oracle is the textbook chain rule through the materialised P of ``definition``:

    O = P V,  P = softmax_rows(S),  S = scale * Q K^T   (visible entries only)
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij * (dP_ij - D_i),   D_i = sum_j P_ij dP_ij     (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

for the scalar loss sum(O * dO). Grouped query heads add the contributions of every query head
to its key/value head; packed sequences never mix. Self-attention only (queries and keys of one
length per sequence).
"""
from __future__ import annotations

from collections import defaultdict
from typing import Optional, Sequence, Tuple

import numpy as np

from .definition import _allowed, _head_scores, _segments, kv_head, softmax_rows_with_lse


def softmax_jacobian_product(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = P * (dP - rowsum(P * dP)): the gradient through a row softmax."""
    d = (p * dp).sum(axis=1)
    return p * (dp - d[:, None])


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       scale: float, causal: bool = False,
                       cu_seqlens: Optional[Sequence[int]] = None
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dq, dk, dv) in float64 for the loss sum(O * do), O the forward of ``definition``.

    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d].
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    if k.shape != (b_, hkv, n, d) or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("k, v must be [B, Hkv, N, d] and do [B, Hq, N, d], all of one N")
    if cu_seqlens is not None and b_ != 1:
        raise ValueError("packed sequences need B == 1")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(b_):
        for h in range(hq):
            hk = kv_head(h, hq, hkv)
            for s0, s1 in _segments(n, cu_seqlens):
                if s1 == s0:
                    continue
                qh, kh, vh, doh = q[b, h, s0:s1], k[b, hk, s0:s1], v[b, hk, s0:s1], do[b, h, s0:s1]
                s = _head_scores(qh, kh, scale)
                p, _ = softmax_rows_with_lse(s, _allowed(s1 - s0, s1 - s0, causal))
                dv[b, hk, s0:s1] += p.T @ doh
                dp = doh @ vh.T
                ds = softmax_jacobian_product(p, dp)
                dq[b, h, s0:s1] = scale * (ds @ kh)
                dk[b, hk, s0:s1] += scale * (ds.T @ qh)
    return dq, dk, dv


def output_gradient_rowsum(o: np.ndarray, do: np.ndarray) -> np.ndarray:
    """D_i = sum_c dO_ic O_ic, which equals sum_j P_ij dP_ij because O = P V."""
    return np.einsum("bhnd,bhnd->bhn", np.asarray(do, np.float64), np.asarray(o, np.float64))


def attention_backward_dq_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                               scale: float, causal: bool, rows,
                               cu_seqlens: Optional[Sequence[int]] = None) -> np.ndarray:
    """dQ of selected rows (b, q_head, token) only: every term of dQ_i depends on row i alone
    (its scores, probabilities and dP row, and D_i = sum_j P_ij dP_ij), so a row is computed
    from q_i, do_i and the keys and values it sees. Returns [R, d] in the order of ``rows``."""
    rows = list(rows)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    segs = _segments(n, cu_seqlens)
    starts = np.array([a for a, _ in segs])
    out = np.empty((len(rows), d))
    by_head = defaultdict(list)
    for r, (b, h, i) in enumerate(rows):
        by_head[(b, kv_head(h, hq, hkv))].append(r)
    for (b, hk), idx in by_head.items():
        kh = np.asarray(k[b, hk], dtype=np.float64)
        vh = np.asarray(v[b, hk], dtype=np.float64)
        for r in idx:
            _, h, i = rows[r]
            seg = int(np.searchsorted(starts, i, side="right")) - 1
            while segs[seg][1] <= i:
                seg += 1
            s0, s1 = segs[seg]
            end = i + 1 if causal else s1
            qi = np.asarray(q[b, h, i], dtype=np.float64)[None, :]
            doi = np.asarray(do[b, h, i], dtype=np.float64)[None, :]
            s = _head_scores(qi, kh[s0:end], scale)
            p, _ = softmax_rows_with_lse(s, np.ones_like(s, dtype=bool))
            ds = softmax_jacobian_product(p, doi @ vh[s0:end].T)
            out[r] = scale * (ds @ kh[s0:end])[0]
    return out


def attention_backward_kv_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                               scale: float, causal: bool, rows,
                               chunk: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """dK and dV of selected key rows (b, kv_head, token) of a fixed-length self-attention
    batch: dV_j = sum_i P_ij dO_i and dK_j = scale sum_i dS_ij q_i over every query row i of
    every query head sharing the kv head. Each query row's softmax (P, its LSE) and D_i need
    the whole row, so query rows are evaluated exactly, a batch of rows at a time. Returns
    (dk [R, d], dv [R, d]) in the order of ``rows``."""
    rows = list(rows)
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    dk = np.zeros((len(rows), d))
    dv = np.zeros((len(rows), d))
    by_head = defaultdict(list)
    for r, (b, hk, j) in enumerate(rows):
        by_head[(b, hk)].append(r)
    for (b, hk), idx in by_head.items():
        sel = np.array([rows[r][2] for r in idx])
        kh = np.asarray(k[b, hk], dtype=np.float64)
        vh = np.asarray(v[b, hk], dtype=np.float64)
        for h in range(hk * group, (hk + 1) * group):
            qh = np.asarray(q[b, h], dtype=np.float64)
            doh = np.asarray(do[b, h], dtype=np.float64)
            for i0 in range(0, n, chunk):
                i1 = min(n, i0 + chunk)
                s = scale * (qh[i0:i1] @ kh.T)
                allowed = np.ones_like(s, dtype=bool)
                if causal:
                    allowed = np.arange(n)[None, :] <= np.arange(i0, i1)[:, None]
                p, _ = softmax_rows_with_lse(s, allowed)
                dp = doh[i0:i1] @ vh.T
                ds = softmax_jacobian_product(p, dp)
                dv[idx] += p[:, sel].T @ doh[i0:i1]
                dk[idx] += scale * (ds[:, sel].T @ qh[i0:i1])
    return dk, dv
