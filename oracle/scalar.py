"""Pure-Python float64 references for tiny inputs (test infrastructure).

Sources (restated, not copied):
  * xspy "FlashAttention and chunked prefill mechanics", section 3 (From-Scratch Reference
    Implementation): a standard softmax (subtract the maximum, exponentiate, divide by the sum)
    and a two-pass online normaliser: pass one streams the blocks keeping a running maximum
    and a running denominator, rescaling the denominator by exp(old max - new max) (zero while
    nothing has been seen); pass two divides exp(x - final max) by the final denominator.
  * "Flash Attention" notes (14cs17), section "Prerequisites": attention = softmax(Q K^T) V.

Sums use math.fsum, so these are correctly rounded sums of correctly rounded terms.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def standard_softmax(x: Sequence[float]) -> List[float]:
    m = max(x)
    e = [math.exp(t - m) for t in x]
    s = math.fsum(e)
    return [t / s for t in e]


def online_softmax_two_pass(chunks: Sequence[Sequence[float]]) -> Tuple[List[float], float, float]:
    """Returns (probabilities, final running max, final running denominator)."""
    m_run = -math.inf
    d_run = 0.0
    for blk in chunks:
        m_next = max(m_run, max(blk))
        keep = 0.0 if m_run == -math.inf else math.exp(m_run - m_next)
        d_run = keep * d_run + math.fsum(math.exp(t - m_next) for t in blk)
        m_run = m_next
    probs = [math.exp(t - m_run) / d_run for blk in chunks for t in blk]
    return probs, m_run, d_run


def attention_scalar(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]],
                     v: Sequence[Sequence[float]], scale: float,
                     causal: bool = False) -> Tuple[List[List[float]], List[float]]:
    """One head, lists of rows. Returns (O rows, lse per row).

    The queries are the last len(q) positions of the len(k) keys, so with causal a query i sees
    the keys j <= i + len(k) - len(q); a query that sees no key gets O = 0 and lse = -inf.
    """
    n = len(q)
    d = len(v[0]) if len(v) else len(q[0])
    o_rows, lses = [], []
    for i in range(n):
        keys = range(max(0, min(len(k), i + len(k) - n + 1))) if causal else range(len(k))
        if len(keys) == 0:
            o_rows.append([0.0] * d)
            lses.append(-math.inf)
            continue
        s = [scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in keys]
        m = max(s)
        e = [math.exp(t - m) for t in s]
        l = math.fsum(e)
        o_rows.append([math.fsum(e[t] * v[j][c] for t, j in enumerate(keys)) / l
                       for c in range(d)])
        lses.append(m + math.log(l))
    return o_rows, lses
