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
  * Error bounds. The E4M3 matrix instruction of gfx950 (32x32x64) does not add its 64 exact
    products in full fp32: measured on MI355X over 6 million random products of full-range
    codes, one instruction's error reached 2^-11.4 of its largest |product| (2^-14 of the sum
    of |products|), so a score carries an error of at most e_S = |scale| (d / 64) 2^-10
    max|q| max|k| (``score_error_bound``, 2^-10 leaving a margin of 2.6 over that maximum).
    The log-sum-exp then errs by at most e_S beyond the forward's 1e-5 relative bound
    (``lse_tolerance``). Rounding to E4M3 changes each weight by at most 2^-4 of itself while it
    is a normal number, and by at most 2^(k-10) <= max(2^-10, B 2^-17) once it is subnormal, so
    a block of 32 errs by at most max(2^-5, B 2^-12) absolutely; over the n_keys / 32 blocks of
    a row, relative to l >= 2^8, that is at most n_keys 2^-18 + 2^-12. The score error moves
    each weight by a factor within exp(+-2 e_S). So |dO| <= max|v| (2^-4 + n_keys 2^-18 +
    2^-12 + 2 e_S) per row, plus half a bf16 unit of O (``o_tolerance``).
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


# One 64-term E4M3 MFMA sum errs by at most this fraction of its largest |product| (see above).
MFMA_E4M3_SUM_ERROR = 2.0 ** -10


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
