"""The seeded generator: determinism, dtype rounding and the named workloads (CPU only)."""
import math

import numpy as np
import pytest
import torch

import seeded_inputs as si


@pytest.mark.parametrize("dtype,tdt", [(si.F16, torch.float16), (si.BF16, torch.bfloat16)])
def test_rounding_matches_torch_round_to_nearest_even(dtype, tdt):
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(20000).astype(np.float32) * 3,
                        r.standard_normal(2000).astype(np.float32) * 1e4,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-6, -3.5], np.float32)])
    bits = si.round_to_bits(x, dtype)
    want = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)


def test_bf16_ties_go_to_even():
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)  # bf16 has 7 stored mantissa bits
    x = np.array([one + half_ulp, one + 3 * half_ulp, one + half_ulp * np.float32(1.0001)],
                 np.float32)
    assert si.round_to_bits(x, si.BF16).tolist() == [0x3F80, 0x3F82, 0x3F81]


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
def test_decode_is_exact(dtype):
    r = np.random.default_rng(1)
    bits = si.round_to_bits(r.standard_normal(5000).astype(np.float32), dtype)
    back = si.round_to_bits(si.bits_to_f64(bits, dtype).astype(np.float32), dtype)
    np.testing.assert_array_equal(bits, back)


def test_same_seed_same_bits():
    a = si.random_inputs(1, 2, 1, 33, 64, si.BF16, 9, causal=True)
    b = si.random_inputs(1, 2, 1, 33, 64, si.BF16, 9, causal=True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    c = si.random_inputs(1, 2, 1, 33, 64, si.BF16, 10, causal=True)
    assert not np.array_equal(a.q, c.q)


def test_named_workloads():
    w = si.WORKLOADS
    assert list(w) == si.WORKLOAD_ORDER and len(w) == 8
    c5 = w["varlen16_h16_d128_causal_bf16"]
    assert c5.seq_lens == (5664, 6695, 685, 6717, 4113, 4470, 5352, 2707, 8035, 926, 2646,
                           3456, 4899, 3649, 1518, 859)
    assert c5.seqlen == 62391 and c5.cu_seqlens()[-1] == 62391
    assert all(512 <= n <= 8192 for n in c5.seq_lens)
    c3 = w[si.HEADLINE]
    assert math.isclose(c3.flops(), 32 * 4 * 16384 ** 2 * 128 / 2)
    assert math.isclose(c3.scale, 0.08838834764831843)
    assert w["gqa_b1_hq32_hkv8_n32768_d128_causal_bf16"].heads_kv == 8
    ch = w["chunk_b1_hq32_hkv8_q2048_k16384_d128_causal_bf16"]
    assert (ch.seqlen, ch.keys) == (2048, 16384)
    # causal chunk: query i of 2048 sees 16384 - 2048 + i + 1 keys; 4*d per key, 32 heads
    exact = 4 * 128 * 32 * sum(16384 - 2048 + i + 1 for i in range(2048))
    assert abs(ch.flops() - exact) / exact < 1e-3
    dec = w["decode_b16_hq32_hkv8_q1_k16384_d128_bf16"]
    assert dec.splitkv and (dec.batch, dec.seqlen, dec.keys) == (16, 1, 16384)
    # K and V of 16 x 8 heads x 16384 keys x 128 dims, 2 bytes each, dominate the bytes moved
    assert dec.io_bytes() == 2 * (2 * 16 * 32 * 128 + 2 * 16 * 8 * 16384 * 128) + 4 * 16 * 32
    dv = w["decode_varlen32_hq32_hkv8_d128_bf16"]
    assert dv.seq_lens == (1,) * 32 and len(dv.seq_lens_k) == 32
    assert all(256 <= n <= 16384 for n in dv.seq_lens_k)
    assert dv.keys == sum(dv.seq_lens_k) == dv.cu_seqlens_k()[-1]
    # one causal query at the end of each cache sees every key: 4 d flops per key and head
    assert math.isclose(dv.flops(), sum(4.0 * 128 * (nk - 0.5) for nk in dv.seq_lens_k) * 32)


def test_key_length_inputs():
    a = si.random_inputs(1, 4, 2, 10, 64, si.F16, 3, seqlen_k=25)
    assert a.q.shape == (1, 4, 10, 64) and a.k.shape == (1, 2, 25, 64) == a.v.shape
    b = si.random_inputs(1, 2, 2, 6, 64, si.F16, 3, seq_lens=(2, 4), seqlen_k=13,
                         seq_lens_k=(9, 4))
    assert list(b.cu_seqlens) == [0, 2, 6] and list(b.cu_seqlens_k) == [0, 9, 13]
    with pytest.raises(ValueError):
        si.random_inputs(1, 2, 2, 6, 64, si.F16, 3, seq_lens=(2, 4), seqlen_k=13)


def test_row_sample_has_edges_and_stays_in_range():
    w = si.WORKLOADS["varlen16_h16_d128_causal_bf16"]
    rows = si.sample_rows(w, 1 / 4096, seed=1)
    cu = w.cu_seqlens()
    toks = {t for _, _, t in rows}
    for s0, s1 in zip(cu[:-1], cu[1:]):
        assert s0 in toks and s1 - 1 in toks
    assert all(0 <= t < w.seqlen and 0 <= h < w.heads_q and b == 0 for b, h, t in rows)
    assert rows == si.sample_rows(w, 1 / 4096, seed=1)


def test_fp8_inputs_use_the_format_range_per_head():
    a = si.random_inputs_fp8(2, 4, 2, 50, 64, seed=3, causal=True)
    assert a.q.dtype == np.uint8 and a.q.shape == (2, 4, 50, 64) and a.k.shape == (2, 2, 50, 64)
    assert a.q_descale.shape == (2, 4) and a.v_descale.shape == (2, 2)
    # the largest |value| of each head maps to the largest code, 448 (0x7E / 0xFE)
    for codes in (a.q, a.k, a.v):
        mags = codes & 0x7F
        assert (mags.max(axis=(2, 3)) == 0x7E).all()
        assert (mags != 0x7F).all()  # no NaN codes
    b = si.random_inputs_fp8(2, 4, 2, 50, 64, seed=3, causal=True)
    np.testing.assert_array_equal(a.v, b.v)
