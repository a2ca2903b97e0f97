"""Pins of the FP8 oracle (oracle/fp8.py): the E4M3 decoder against the format's published
values and a library routine (torch's float8_e4m3fn on the CPU); the E4M3 rounding against the
format's code table; the simulation of the reading's quantisation against the definition; and
the output bound against that simulation, on random rows (never exceeded) and on constructions
that reach it (within a factor 2)."""
import numpy as np
import torch

import oracle
import oracle.fp8 as ofp8


def test_decoder_matches_the_format_landmarks():
    d = ofp8.decode_e4m3(np.array([0x00, 0x80, 0x38, 0x7E, 0xFE, 0x01, 0x08, 0x07, 0x3F, 0x40,
                                   0x7F, 0xFF], dtype=np.uint8))
    assert d[0] == 0.0 and d[1] == 0.0 and np.signbit(d[1])
    assert d[2] == 1.0                       # exponent 7 = bias
    assert d[3] == 448.0 and d[4] == -448.0  # largest finite
    assert d[5] == 2.0 ** -9                 # smallest subnormal
    assert d[6] == 2.0 ** -6                 # smallest normal
    assert d[7] == 7 * 2.0 ** -9             # largest subnormal
    assert d[8] == 1.875 and d[9] == 2.0
    assert np.isnan(d[10]) and np.isnan(d[11])


def test_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = ofp8.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_dequantize_applies_one_factor_per_batch_and_head():
    codes = np.full((2, 3, 4, 8), 0x38, dtype=np.uint8)  # all 1.0
    ds = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    x = ofp8.dequantize(codes, ds)
    for b in range(2):
        for h in range(3):
            assert (x[b, h] == ds[b, h]).all()


def test_rounding_keeps_every_code_and_rounds_midpoints_to_even():
    """round_e4m3 against the format's own code table (decode_e4m3): every finite code value
    is kept, and the midpoint between neighbouring codes goes to the one with an even
    mantissa (the last bit of the code)."""
    codes = np.arange(0x00, 0x7F, dtype=np.uint8)  # non-negative finite codes, ascending
    vals = ofp8.decode_e4m3(codes)
    np.testing.assert_array_equal(ofp8.round_e4m3(vals.astype(np.float32)), vals)
    mids = (vals[:-1] + vals[1:]) / 2
    even = np.where(codes[:-1] % 2 == 0, vals[:-1], vals[1:])
    np.testing.assert_array_equal(ofp8.round_e4m3(mids.astype(np.float32)), even)
    # just off the midpoints: the nearer code
    up = ofp8.round_e4m3((mids * (1 + 1e-6)).astype(np.float32))
    np.testing.assert_array_equal(up[1:], vals[2:])


def test_block_scales_keep_values_in_range_and_are_undone_exactly():
    rng = np.random.default_rng(3)
    p = np.exp2(rng.uniform(-40, 31, (16, 256))).astype(np.float32)  # lazy references: up to 2^31
    pt = ofp8.block_scaled_probabilities(p)
    for b0 in range(0, 256, 32):
        blk = p[:, b0:b0 + 32].astype(np.float64)
        k = np.maximum(0, np.floor(np.log2(blk.sum(axis=1))) - 7)
        scaled = pt[:, b0:b0 + 32] / np.exp2(k)[:, None]
        assert (scaled <= 256).all()                      # inside E4M3's range (448)
        # the scaled values are E4M3 codes: the block scale is undone exactly
        np.testing.assert_array_equal(ofp8.round_e4m3(scaled.astype(np.float32)), scaled)
        rel = np.abs(pt[:, b0:b0 + 32] - blk) / blk
        normal = blk / np.exp2(k)[:, None] >= 2.0 ** -6
        assert (rel[normal] <= 2.0 ** -4 + 1e-12).all()  # normal numbers: half a unit of 3 bits
        sub_err = np.abs(pt[:, b0:b0 + 32] - blk)[~normal]
        assert (sub_err <= np.broadcast_to(np.exp2(k - 10)[:, None], blk.shape)[~normal] + 1e-30).all()


def test_simulation_without_rounding_is_the_definition():
    rng = np.random.default_rng(4)
    for n, nk, causal in ((1, 1, True), (7, 300, True), (200, 200, False), (65, 40, True)):
        q, k, v = rng.standard_normal((n, 64)), rng.standard_normal((nk, 64)), rng.standard_normal((nk, 64))
        o0, l0 = ofp8.simulate_attention(q, k, v, 0.3, causal, ref_offset=5.5, quantize=False)
        o1, l1 = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3, causal)
        np.testing.assert_allclose(o0, o1[0, 0], atol=3e-7)  # p held in float32
        fin = np.isfinite(l1[0, 0])
        np.testing.assert_allclose(l0[fin], l1[0, 0][fin], atol=3e-7)
        assert np.array_equal(np.isneginf(l0), ~fin)


def test_output_bound_holds_on_random_rows_at_every_reference():
    """The rounding part of o_tolerance (no score error: the simulation's scores are exact) is
    never exceeded, over random rows, key counts up to 4096, peaked and flat score spreads, and
    references anywhere in the lazy range."""
    rng = np.random.default_rng(5)
    for trial in range(24):
        nk = int(rng.choice([1, 31, 64, 300, 1024, 4096]))
        n = 8
        spread = float(rng.choice([0.5, 1.0, 3.0]))
        q = rng.standard_normal((n, 64)) * spread
        k = rng.standard_normal((nk, 64)) * spread
        v = rng.standard_normal((nk, 64))
        off = float(rng.uniform(0, 23))
        o_sim, _ = ofp8.simulate_attention(q, k, v, 0.125, False, ref_offset=off)
        o_ref, _ = oracle.attention(q[None, None], k[None, None], v[None, None], 0.125, False)
        err = np.abs(o_sim - o_ref[0, 0]).max()
        bound = ofp8.o_tolerance(v, nk) - np.abs(v).max() * 2.0 ** -9  # without O's bf16 rounding
        assert err <= bound, (trial, err, bound)


def _row_with_scores(t):
    """q [1, d], k [n, d] whose scores scale * q.k in log2 units equal t (scale 1)."""
    n = len(t)
    q = np.zeros((1, 64)); q[0, 0] = 1.0
    k = np.zeros((n, 64)); k[:, 0] = np.asarray(t) / np.log2(np.e)
    return q, k


def test_dominant_weight_at_a_rounding_midpoint_reaches_the_bound():
    """One key's weight, shifted to 2^8 (1 + 2^-4) against the reference, lies halfway between two
    E4M3 values and rounds down by 2^-4 / (1 + 2^-4) of itself: O misses that fraction of its
    V row, 0.94 of the bound's 2^-4 term."""
    q, k = _row_with_scores([0.0, -200.0, -200.0])
    v = np.zeros((3, 64)); v[0] = 1.0
    o_sim, _ = ofp8.simulate_attention(q, k, v, 1.0, ref_offset=np.log2(1 + 2.0 ** -4))
    err = np.abs(o_sim - 1.0).max()
    bound = ofp8.o_tolerance(v, 3) - 2.0 ** -9
    assert np.isclose(err, 2.0 ** -4 / (1 + 2.0 ** -4), rtol=1e-6)
    assert 0.5 * bound <= err <= bound


def test_subnormal_blocks_reach_the_key_count_term():
    """16384 keys: the dominant one as above (its V row -1), every other one at 1.5 2^-9 (just
    above the midpoint between two subnormal E4M3 values, V row +1) in blocks whose sum keeps
    the scale at 1, so all of them round up by about 2^-10. Both errors push O the same way;
    together they reach 0.8 of the bound, whose key-count term n 2^-18 is as large as 2^-4."""
    n = 16384
    t = np.full(n, np.log2(1.5 * (1 + 1e-6)) - 9 - 8 - np.log2(1 + 2.0 ** -4))
    t[0] = 0.0
    q, k = _row_with_scores(t)
    v = np.ones((n, 64)); v[0] = -1.0
    off = np.log2(1 + 2.0 ** -4)
    o_sim, _ = ofp8.simulate_attention(q, k, v, 1.0, ref_offset=off, quantize=True)
    o_ref, _ = ofp8.simulate_attention(q, k, v, 1.0, ref_offset=off, quantize=False)
    err = np.abs(o_sim - o_ref).max()
    bound = ofp8.o_tolerance(v, n) - 2.0 ** -9
    assert n * 2.0 ** -18 == 2.0 ** -4
    assert 0.75 * bound <= err <= bound, (err, bound)


def test_score_error_bound_scales_with_the_operands():
    """e_S = |scale| (d / 64) 2^-10 max|q| max|k| (the empirical summation term), and the LSE
    and output bounds grow with it."""
    q = np.array([[0.5, -2.0]])
    k = np.array([[3.0, 1.0]])
    e = ofp8.score_error_bound(q, k, -0.25, 128)
    assert e == 0.25 * 2 * ofp8.MFMA_E4M3_SUM_ERROR * 2.0 * 3.0
    assert ofp8.score_error_bound(np.zeros((0, 2)), k, 1.0, 64) == 0.0
    assert ofp8.score_error_bound(2 * q, k, -0.25, 128) == 2 * e
    lse = np.array([0.5, -20.0])
    assert (ofp8.lse_tolerance(lse, e) - ofp8.lse_tolerance(lse, 0.0) == e).all()
    v = np.array([2.0])
    assert ofp8.o_tolerance(v, 0, e) - ofp8.o_tolerance(v, 0, 0.0) == 2.0 * 2 * e
