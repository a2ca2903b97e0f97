"""FP8 (OCP E4M3) inputs for the attention definition, and the error bound of an FP8 kernel
(test infrastructure).

The xspy page "FlashAttention and chunked prefill mechanics" (section 1, and its reference to
the FlashAttention-3 paper) names FP8 matrix cores as FlashAttention-3's second lever and gives
no recipe. The readings taken here (also listed in the design notes):

  * Q, K and V arrive as E4M3 codes (the OCP 8-bit format: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN, largest finite
    value 448) with one fp32 descale factor per (batch, head): the tensor a code stands for is
    decode(code) * descale. Attention is the definition applied to those decoded values, so
    the oracle is ``attention`` on them.
  * An FP8 kernel forms S = Q K^T from the codes on the E4M3 matrix instructions, applies
    scale * descale_q * descale_k to the scores and descale_v to the output, and rounds the
    probabilities to E4M3 before the P V product: P~ = exp2(s - m) shifted by 2^8 against a
    reference maximum m, then, for each block of 32 keys of a query row, divided by a power of
    two 2^k chosen from the block's sum B (k = max(0, e - 7) for B in [2^e, 2^(e+1)), so every
    value stays below 2^8, inside E4M3's range) and rounded to nearest even; the matrix
    instruction's block scale multiplies 2^k back exactly. The row sum l uses the unrounded
    values (l >= 2^8) and O is rounded to bf16.
  * Error bounds, in two parts.
    1. The matrix instruction's sums (an empirical reading, not a derivation). The E4M3
       matrix instruction of gfx950 (32x32x64) does not add its 64 exact products in full
       fp32. The pages and the public ISA documents give no accumulation precision, so the
       bound takes a measurement: an in-bounds probe on one MI355X over 6 million random
       64-term products of full-range codes found errors up to 2^-11.4 of the largest
       |product| (2^-14 of the sum of |products|), and 30-50 % of the sums exact. The bound
       uses 2^-10 (a margin of 2.6): a score errs by at most e_S = |scale| (d / 64) 2^-10
       max|q| max|k| (``score_error_bound``), the log-sum-exp by at most e_S beyond the
       forward's 1e-5 relative bound (``lse_tolerance``), and each weight moves by a factor
       within exp(+-2 e_S).
    2. The rounding of the probabilities (derived, and pinned by ``simulate_attention``, the
       reading's quantisation in float64 on exact scores). Rounding to E4M3 changes a weight by
       at most 2^-4 of itself while it is a normal number, and by at most 2^(k-10) <=
       max(2^-10, B 2^-17) once it is subnormal, so a block of 32 errs by at most
       max(2^-5, B 2^-12) absolutely; over the n_keys / 32 blocks of a row, relative to
       l >= 2^8, that is at most n_keys 2^-18 + 2^-12. Both terms are reached: a dominant
       weight at an E4M3 rounding midpoint costs 2^-4 / (1 + 2^-4) of its V row, and blocks of
       32 weights at subnormal midpoints, all rounding the same way, cost n_keys 2^-18 of the
       V rows against a dominant weight of 2^8 (the tests build both).
    So |dO| <= max|v| (2^-4 + n_keys 2^-18 + 2^-12 + 2 e_S) per row, plus half a bf16 unit of
    O (``o_tolerance``). Random inputs stay far below it (the errors of many weights cancel),
    so the tests also hold the kernel's mean error to that of the simulation.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """E4M3 (OCP) codes (uint8) -> float64 values, from the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = sign * (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    sub = sign * (man / 8.0) * 2.0 ** -6
    out = np.where(exp == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def dequantize(codes: np.ndarray, descale: np.ndarray) -> np.ndarray:
    """[B, H, N, d] codes times the [B, H] descale factors, in float64."""
    return decode_e4m3(codes) * np.asarray(descale, dtype=np.float64)[:, :, None, None]


# One 64-term E4M3 MFMA sum errs by at most this fraction of its largest |product|: an empirical
# reading (part 1 above: the largest error measured over 6e6 sums was 2^-11.4).
MFMA_E4M3_SUM_ERROR = 2.0 ** -10

# The reading's shift of the probabilities (the row maximum's weight) and block length.
P_SHIFT = 2.0 ** 8
P_BLOCK = 32


def score_error_bound(q_values: np.ndarray, k_values: np.ndarray, scale: float,
                      head_dim: int) -> float:
    """e_S: the largest score error of an FP8 kernel for these (decoded) Q and K values."""
    if q_values.size == 0 or k_values.size == 0:
        return 0.0
    qmax = float(np.abs(q_values).max())
    kmax = float(np.abs(k_values).max())
    return abs(scale) * (head_dim / 64) * MFMA_E4M3_SUM_ERROR * qmax * kmax


def lse_tolerance(lse_ref: np.ndarray, score_err: float) -> np.ndarray:
    """Per-row bound on |LSE_gpu - LSE_ref|: the forward's relative 1e-5 plus e_S."""
    return 1e-5 * np.maximum(np.abs(lse_ref), 1.0) + score_err


def o_tolerance(v_values: np.ndarray, n_keys: int, score_err: float = 0.0) -> float:
    """The bound above for outputs built from these V values (all heads) and n_keys keys."""
    vmax = float(np.abs(v_values).max()) if v_values.size else 0.0
    return vmax * (2.0 ** -4 + n_keys * 2.0 ** -18 + 2.0 ** -12 + 2.0 * score_err) + vmax * 2.0 ** -9


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 with round-to-nearest-even (torch's float8_e4m3fn on the
    CPU, a library routine independent of the kernels), returned as float64."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def block_scaled_probabilities(p: np.ndarray, quantize: bool = True) -> np.ndarray:
    """The reading's P~ for rows of shifted probabilities p ([rows, n], float32 values, the
    largest of a row at most 2^8 times the reference's): each block of 32 keys of a row with
    sum B in [2^e, 2^(e+1)) is divided by 2^k, k = max(0, e - 7), rounded to E4M3 and
    multiplied back by 2^k (exactly, as the matrix instruction's block scale does). Without
    quantize the values are returned unchanged (float64)."""
    p = np.asarray(p, dtype=np.float32)
    if not quantize:
        return p.astype(np.float64)
    rows, n = p.shape
    out = np.zeros((rows, n))
    for b0 in range(0, n, P_BLOCK):
        blk = p[:, b0:b0 + P_BLOCK]
        bsum = blk.astype(np.float64).sum(axis=1)
        e = np.where(bsum > 0, np.floor(np.log2(np.where(bsum > 0, bsum, 1.0))), 0.0)
        k = np.maximum(0.0, e - 7.0)
        scaled = (blk / np.exp2(k)[:, None].astype(np.float32)).astype(np.float32)
        out[:, b0:b0 + P_BLOCK] = round_e4m3(scaled) * np.exp2(k)[:, None]
    return out


def simulate_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       causal: bool = False, ref_offset: float = 0.0,
                       quantize: bool = True):
    """The FP8 reading's arithmetic on exact (float64) scores, for one head: q [n, d], k, v
    [nk, d] (decoded values). Scores s = scale q.k in log2 units; reference m = row maximum
    minus ref_offset (0 <= ref_offset <= 23, the range a lazily raised reference covers);
    p = 2^(s - m + 8) rounded to float32; P~ from block_scaled_probabilities; l = sum of the
    unrounded p; O = sum_j P~_j v_j / l; LSE = (m - 8 + log2 l) ln 2. Returns (O, LSE); rows
    that see no key get O = 0, LSE = -inf. With quantize=False this is the definition."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T) * np.log2(np.e)
    if causal:
        i = np.arange(n)[:, None]
        j = np.arange(nk)[None, :]
        s = np.where(j <= i + (nk - n), s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    seen = np.isfinite(m)
    m_ref = np.where(seen, m - ref_offset, 0.0)
    p = np.exp2(s - m_ref[:, None] + 8.0).astype(np.float32)
    pt = block_scaled_probabilities(p, quantize)
    l = p.astype(np.float64).sum(axis=1)
    o = np.where(seen[:, None], (pt @ v) / np.where(seen, l, 1.0)[:, None], 0.0)
    lse = np.where(seen, (m_ref - 8.0 + np.log2(np.where(seen, l, 1.0))) * np.log(2.0), -np.inf)
    return o, lse
