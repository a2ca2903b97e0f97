"""The parity checkers themselves, pinned like the oracle (CPU only).

A checker that passes everything would let every GPU test pass. So each comparison the GPU
tests and the bench rely on is run here on planted differences: one output element off by
1.01 x the tolerance must fail and by 0.99 x must pass (both signs, both input types); the
same for the LSE error, in its relative and its absolute (|LSE| < 1) regime; and a row that
sees no key must match exactly (O = 0, LSE = -inf) on both sides.
"""
import numpy as np
import pytest

import bench
import oracle
import seeded_inputs as si
from gpu_util import LSE_TOL, O_TOL, assert_close, errors
from test_gpu_allrows import _check_unit


def _reference(rng, rows=6, d=8):
    o_ref = rng.standard_normal((rows, d))
    lse_ref = np.array([5.3, -7.25, 0.4, -0.6, 12.0, 1.0])[:rows]
    return o_ref, lse_ref


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_one_output_element_past_the_tolerance_fails(dtype, sign):
    rng = np.random.default_rng(1)
    o_ref, lse_ref = _reference(rng)
    tol = O_TOL[dtype]
    for frac, ok in ((0.99, True), (1.01, False)):
        o = o_ref.copy()
        o[3, 5] += sign * frac * tol
        if ok:
            assert_close(o, lse_ref.copy(), o_ref, lse_ref, dtype)
        else:
            with pytest.raises(AssertionError):
                assert_close(o, lse_ref.copy(), o_ref, lse_ref, dtype)


@pytest.mark.parametrize("row", [0, 1, 4, 2, 3])
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_one_lse_past_the_tolerance_fails(row, sign):
    rng = np.random.default_rng(2)
    o_ref, lse_ref = _reference(rng)
    # relative to |LSE| for |LSE| >= 1 (rows 0, 1, 4), absolute below (rows 2, 3)
    unit = max(abs(lse_ref[row]), 1.0) * LSE_TOL
    for frac, ok in ((0.99, True), (1.01, False)):
        lse = lse_ref.copy()
        lse[row] += sign * frac * unit
        if ok:
            assert_close(o_ref.copy(), lse, o_ref, lse_ref, si.BF16)
        else:
            with pytest.raises(AssertionError):
                assert_close(o_ref.copy(), lse, o_ref, lse_ref, si.BF16)


def test_rows_that_see_no_key_must_match_exactly():
    rng = np.random.default_rng(3)
    o_ref, lse_ref = _reference(rng)
    o_ref[2] = 0.0
    lse_ref[2] = -np.inf
    assert errors(o_ref.copy(), lse_ref.copy(), o_ref, lse_ref) == (0.0, 0.0)
    cases = []
    lse = lse_ref.copy(); lse[2] = 3.0; cases.append((o_ref.copy(), lse))       # finite for empty
    lse = lse_ref.copy(); lse[0] = -np.inf; cases.append((o_ref.copy(), lse))   # -inf for a row
    lse = lse_ref.copy(); lse[1] = np.inf; cases.append((o_ref.copy(), lse))    # +inf anywhere
    lse = lse_ref.copy(); lse[4] = np.nan; cases.append((o_ref.copy(), lse))    # NaN LSE
    o = o_ref.copy(); o[2, 0] = 1e-6; cases.append((o, lse_ref.copy()))         # O != 0, empty row
    o = o_ref.copy(); o[5, 1] = np.nan; cases.append((o, lse_ref.copy()))       # NaN output
    o = o_ref.copy(); o[1, 1] = np.inf; cases.append((o, lse_ref.copy()))       # Inf output
    for o, lse in cases:
        assert errors(o, lse, o_ref, lse_ref) == (np.inf, np.inf)
        with pytest.raises(AssertionError):
            assert_close(o, lse, o_ref, lse_ref, si.BF16)


def _bf16_neighbours(t):
    """(bits, value) of the bf16 numbers around a positive t."""
    b = int(si.round_to_bits(np.array([t], dtype=np.float32), si.BF16)[0])
    bits = np.array([b + k for k in range(-3, 4)], dtype=np.uint16)
    return list(zip(bits, si.bits_to_f64(bits, si.BF16)))


def test_all_rows_unit_checker_catches_one_planted_error():
    """The per-block comparison of the all-rows GPU test, fed the oracle's own rounded output,
    passes; with one element moved just past the bf16 tolerance it reports that element."""
    w = si.Workload("tiny_causal", 1, 2, 1, 700, 64, si.BF16, True, seed=11)
    inp = si.random_inputs(1, 2, 1, 700, 64, si.BF16, 11, causal=True)
    qf, kf, vf = inp.f64()
    o_ref, lse_ref = oracle.attention(qf, kf, vf, w.scale, True)
    o_bits = si.round_to_bits(o_ref.astype(np.float32), si.BF16)
    unit = (1, 0, 700, 512, 700)  # head 1, rows [512, 700)
    r = _check_unit(w, inp, o_bits, lse_ref, unit)
    assert r["do"] <= O_TOL[si.BF16] / 2 and r["dl"] == 0.0
    assert r["counts"].sum() == (700 - 512) * 64
    tol = O_TOL[si.BF16]
    tok = 600
    col = int(np.argmax(o_ref[0, 1, tok]))  # a positive element
    x = o_ref[0, 1, tok, col]
    assert x > 0.1
    near = _bf16_neighbours(x + tol)
    # the nearest bf16 value at least 1.01 tol above x, and the farthest at most 0.99 tol above
    past = min((c for c in near if c[1] - x >= 1.01 * tol), key=lambda c: c[1])
    inside = max((c for c in near if 0 <= c[1] - x <= 0.99 * tol), key=lambda c: c[1])
    for (bits, val), fails in ((past, True), (inside, False)):
        planted = o_bits.copy()
        planted[0, 1, tok, col] = bits
        r = _check_unit(w, inp, planted, lse_ref, unit)
        assert (r["do"] > tol) == fails, (val - x, r["do"])
        if fails:
            assert r["where"][:3] == (1, tok, col) and r["do"] == pytest.approx(val - x)
    lse = lse_ref.copy()
    lse[0, 1, 650] *= 1 + 1.01 * LSE_TOL
    assert _check_unit(w, inp, o_bits, lse, unit)["dl"] > LSE_TOL


def test_bench_band_breakdown():
    o_ref = np.array([0.1, 0.7, 1.5, 3.0, 5.0, 9.0, -5.5])
    o_gpu = o_ref + np.array([1e-4, 2e-4, 3e-4, 4e-4, 5e-4, 6e-4, -7e-4])
    bands = bench.band_errors(o_gpu, o_ref, si.BF16)
    by = {tuple(b["band"]): b for b in bands}
    assert by[(4.0, 8.0)]["n"] == 2 and by[(4.0, 8.0)]["max_abs_dO"] == pytest.approx(7e-4)
    assert by[(4.0, 8.0)]["half_unit_at_max"] == 2.0 ** -6
    assert by[(0.5, 1.0)]["half_unit_at_max"] == 2.0 ** -9
    assert by[(8.0, None)]["half_unit_at_max"] == 2.0 ** -5
    assert sum(b["n"] for b in bands) == o_ref.size
