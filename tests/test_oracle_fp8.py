"""Pins of the E4M3 decoder of the FP8 oracle (oracle/fp8.py) against the format's published
values and a library routine (torch's float8_e4m3fn on the CPU)."""
import numpy as np
import torch

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


def test_tolerance_grows_with_the_values_and_the_key_count():
    v = np.array([0.5, -3.0, 2.0])
    assert ofp8.o_tolerance(v, 0) == 3.0 * (2 ** -4 + 2 ** -12) + 3.0 * 2 ** -9
    assert ofp8.o_tolerance(v, 2 ** 14) == 3.0 * (2 ** -4 + 2 ** -4 + 2 ** -12) + 3.0 * 2 ** -9


def test_score_and_lse_bounds():
    q = np.array([[0.5, -2.0]])
    k = np.array([[3.0, 1.0]])
    # |scale| * (d / 64) * 2^-10 * max|q| * max|k|
    assert ofp8.score_error_bound(q, k, -0.25, 128) == 0.25 * 2 * 2 ** -10 * 2.0 * 3.0
    assert ofp8.score_error_bound(np.zeros((0, 2)), k, 1.0, 64) == 0.0
    e = 1e-3
    np.testing.assert_allclose(ofp8.lse_tolerance(np.array([0.5, -20.0]), e),
                               [1e-5 + e, 20 * 1e-5 + e])
    assert ofp8.o_tolerance(np.array([2.0]), 0, e) == 2.0 * (2 ** -4 + 2 ** -12 + 2 * e) + 2.0 * 2 ** -9
