"""The tiled FlashAttention forward with online softmax, in float64 (test infrastructure).

Sources (restated in my own code, not copied):
  * "Flash Attention" notes (14cs17), section "Flash Attention Algorithm": for each query block
    Q_i, start from O_i = 0, l_i = 0, m_i = -inf; for each key/value block K_j, V_j form
    S_ij = Q_i K_j^T and update (m_i, l_i, O_i) with the online-softmax rule; write O_i.
  * same page, section "Tiling Strategy" (Definition 3): blocks of B_r x d and B_c x d.
  * same page, Theorem 2 (Online Softmax): the running maximum and running sum are merged
    block by block, rescaling the earlier partial result when a larger maximum appears. The
    update equations (1)-(3) did not survive extraction; the reading used here, consistent
    with the proof sentence and with the xspy page's section 3 update (scale_prev =
    exp(m_running - m_new), zero when m_running is -inf), is
        (1) m = max(m_old, m_new)
        (2) l = exp(m_old - m) l_old + exp(m_new - m) l_new
        (3) O = exp(m_old - m) O_old + exp(m_new - m) O_new      (O unnormalised)
    with the final O divided by l once (the deferred normalisation of FlashAttention-2's
    "reduced non-matmul FLOPs", same page, section "Flash Attention 2 Improvements").

Its only role is to show, in float64, that the tiled result equals the definition in
``oracle.attention`` for arbitrary block partitions.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def _weight(m_part: np.ndarray, m: np.ndarray) -> np.ndarray:
    """exp(m_part - m), taken as 0 where m_part is -inf (nothing seen yet)."""
    out = np.zeros_like(m)
    live = np.isfinite(m_part)
    out[live] = np.exp(m_part[live] - m[live])
    return out


def merge(m_old, l_old, o_old, m_new, l_new, o_new):
    """Online-softmax merge of two partial results, equations (1)-(3) above, per row."""
    m_old = np.asarray(m_old, dtype=np.float64)
    m_new = np.asarray(m_new, dtype=np.float64)
    m = np.maximum(m_old, m_new)
    a_old = _weight(np.atleast_1d(m_old), np.atleast_1d(m)).reshape(m.shape)
    a_new = _weight(np.atleast_1d(m_new), np.atleast_1d(m)).reshape(m.shape)
    l = a_old * l_old + a_new * l_new
    o = None
    if o_old is not None:
        o = a_old[..., None] * o_old + a_new[..., None] * o_new
    return m, l, o


def _block_starts(n: int, sizes: Optional[Sequence[int]], default: int):
    if sizes is None:
        sizes = [default] * ((n + default - 1) // default)
    out, pos = [], 0
    for s in sizes:
        if s <= 0:
            raise ValueError("block sizes must be positive")
        out.append((pos, min(pos + s, n)))
        pos += s
        if pos >= n:
            break
    if pos < n:
        raise ValueError("block sizes do not cover the sequence")
    return out


def flash_forward(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float,
                  causal: bool = False, row_blocks: Optional[Sequence[int]] = None,
                  col_blocks: Optional[Sequence[int]] = None, block_rows: int = 4,
                  block_cols: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """Tiled forward pass for one head: qh, kh, vh are [N, d]; returns (O [N, d], lse [N]).

    Query blocks follow ``row_blocks`` (sizes) or B_r = block_rows; key/value blocks follow
    ``col_blocks`` or B_c = block_cols. Causal visibility is key <= query.
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    n, d = qh.shape
    o_out = np.zeros((n, d))
    lse_out = np.zeros(n)
    for r0, r1 in _block_starts(n, row_blocks, block_rows):
        rows = r1 - r0
        o_acc = np.zeros((rows, d))  # step 2: O_i = 0, l_i = 0, m_i = -inf
        l_acc = np.zeros(rows)
        m_acc = np.full(rows, -np.inf)
        for c0, c1 in _block_starts(n, col_blocks, block_cols):  # step 3
            s = scale * (qh[r0:r1] @ kh[c0:c1].T)  # S_ij, never stored beyond this block
            if causal:
                qi = np.arange(r0, r1)[:, None]
                kj = np.arange(c0, c1)[None, :]
                s = np.where(kj <= qi, s, -np.inf)
            m_blk = s.max(axis=1)
            e = np.zeros_like(s)
            live = np.isfinite(m_blk)
            e[live] = np.exp(s[live] - m_blk[live][:, None])
            l_blk = e.sum(axis=1)
            o_blk = e @ vh[c0:c1]
            m_acc, l_acc, o_acc = merge(m_acc, l_acc, o_acc, m_blk, l_blk, o_blk)
        o_out[r0:r1] = o_acc / l_acc[:, None]  # step 4: normalise once and write O_i
        lse_out[r0:r1] = m_acc + np.log(l_acc)
    return o_out, lse_out


def online_lse(x: Sequence[float], blocks: Sequence[int]) -> Tuple[float, float]:
    """Running (max, sum) of one score row streamed in blocks; returns (m, l)."""
    m, l = -math.inf, 0.0
    pos = 0
    for size in blocks:
        blk = np.asarray(x[pos:pos + size], dtype=np.float64)
        pos += size
        mb = float(blk.max())
        lb = float(np.exp(blk - mb).sum())
        m_arr, l_arr, _ = merge(np.array([m]), np.array([l]), None, np.array([mb]),
                                np.array([lb]), None)
        m, l = float(m_arr[0]), float(l_arr[0])
    return m, l
