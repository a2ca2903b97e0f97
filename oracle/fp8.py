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
  * An FP8 kernel forms S = Q K^T exactly from the codes (fp32 accumulation), applies
    scale * descale_q * descale_k to the scores and descale_v to the output, and rounds the
    probabilities to E4M3 before the P V product: P~ = exp2(s - m) is shifted by 2^8 (so the
    largest is 256, inside E4M3's range) and rounded to nearest even. The row sum l uses the
    unrounded values and O is rounded to bf16.
  * Error bound (``o_tolerance``): rounding P~ to E4M3 changes each weight by at most 2^-4 of
    itself while it is a normal number, and by at most 2^-10 absolutely (in the shifted units,
    where l >= 256) once it is subnormal, so |dO| <= max|v| (2^-4 + n_keys 2^-18) per row, plus
    half a bf16 unit of O. The log-sum-exp comes from the unrounded sum and keeps the forward's
    1e-5 bound.
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


def o_tolerance(v_values: np.ndarray, n_keys: int) -> float:
    """The bound above for outputs built from these V values (all heads) and n_keys keys."""
    vmax = float(np.abs(v_values).max()) if v_values.size else 0.0
    return vmax * (2.0 ** -4 + n_keys * 2.0 ** -18) + vmax * 2.0 ** -9
