"""Pins of the RoPE oracle (oracle/rope.py) against mathematics that does not restate its code:
complex multiplication, rotation invariants, the relative-position property, the permutation
between the two pairings, error bounds of the rounded reading, and attention identities."""
import math

import numpy as np
import pytest

import oracle.rope as rope
from oracle import attention

RNG = np.random.default_rng(20)


def test_tables_start_at_the_identity_and_follow_the_frequency_ladder():
    cos, sin = rope.rotary_tables(50, 8)
    assert cos.shape == sin.shape == (50, 4)
    np.testing.assert_array_equal(cos[0], 1.0)
    np.testing.assert_array_equal(sin[0], 0.0)
    # at position 1 the angle of pair i is theta_i: theta_0 = 1, and theta_i / theta_(i+1)
    # is the constant base^(2/d) = 10000^(1/4) = 10
    theta = np.arctan2(sin[1], cos[1])
    assert math.isclose(theta[0], 1.0, rel_tol=1e-15)
    np.testing.assert_allclose(theta[:-1] / theta[1:], 10.0, rtol=1e-12)
    # positions advance the angle linearly: p * theta_i (checked at p = 3 for the slow pairs)
    np.testing.assert_allclose(np.arctan2(sin[3], cos[3])[1:], 3 * theta[1:], rtol=1e-12)


def test_interleaved_rotation_is_complex_multiplication():
    x = RNG.standard_normal((5, 16))
    cos, sin = rope.rotary_tables(5, 16)
    got = rope.rotate_exact(x, cos, sin, interleaved=True)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.arctan2(sin, cos))
    np.testing.assert_allclose(got[:, 0::2], z.real, atol=1e-14)
    np.testing.assert_allclose(got[:, 1::2], z.imag, atol=1e-14)


def test_half_split_pairing_is_a_permutation_of_the_interleaved_one():
    d = 12
    x = RNG.standard_normal((7, d))
    cos, sin = rope.rotary_tables(7, d)
    perm = np.empty(d, dtype=int)  # interleaved position -> half-split position
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    inter = rope.rotate_exact(x[:, perm], cos, sin, interleaved=True)
    half = rope.rotate_exact(x, cos, sin, interleaved=False)
    np.testing.assert_allclose(inter, half[:, perm], atol=1e-15)


@pytest.mark.parametrize("interleaved", [True, False])
def test_rotation_keeps_pair_norms_and_only_relative_position_matters(interleaved):
    d = 64
    cos, sin = rope.rotary_tables(300, d)
    q = RNG.standard_normal(d)
    k = RNG.standard_normal(d)
    ia, ib = rope.rope_pairs(d, interleaved)

    def at(x, p):
        return rope.rotate_exact(x[None], cos[p:p + 1], sin[p:p + 1], interleaved)[0]

    qr = at(q, 200)
    np.testing.assert_allclose(np.hypot(qr[ia], qr[ib]), np.hypot(q[ia], q[ib]), rtol=1e-13)
    base = at(q, 37) @ at(k, 12)
    for shift in (1, 50, 200):
        assert math.isclose(at(q, 37 + shift) @ at(k, 12 + shift), base, rel_tol=1e-9,
                            abs_tol=1e-9)
    # and the rotation does depend on the offset
    assert not math.isclose(at(q, 38) @ at(k, 12), base, rel_tol=1e-6)


def test_own_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -9, -(3.0 + 2 ** -7 + 2 ** -20),
                  65504.0, np.inf, -0.0, -(3.0 + 2 ** -7)], dtype=np.float32)
    out = rope.round_to_dtype(x, "bf16")
    # ties go to the even neighbour (1 and 3 end in a 0 bit); anything past a tie rounds away
    np.testing.assert_array_equal(out[:4], [1.0, 1.0, 1.015625, 1.0])
    assert out[4] == -(3.0 + 2 ** -6) and out[8] == -3.0
    assert out[5] == 65536.0 and out[6] == np.inf
    assert np.signbit(out[7]) and out[7] == 0.0
    assert np.isnan(rope.round_to_dtype(np.array([np.nan], np.float32), "bf16")[0])


@pytest.mark.parametrize("dtype,rel", [("bf16", 2 ** -8), ("f16", 2 ** -10)])
@pytest.mark.parametrize("interleaved", [True, False])
def test_rounded_rotation_is_within_one_unit_of_the_exact_one(dtype, rel, interleaved):
    x32 = RNG.standard_normal((64, 128)).astype(np.float32)
    x = rope.round_to_dtype(x32, dtype)  # inputs of the input type
    cos, sin = rope.rotary_tables(4096, 128)
    pos = RNG.integers(0, 4096, 64)
    c32, s32 = cos[pos].astype(np.float32), sin[pos].astype(np.float32)
    got = rope.rotate_rounded(x, c32, s32, interleaved, dtype)
    exact = rope.rotate_exact(x, c32.astype(np.float64), s32.astype(np.float64), interleaved)
    assert (np.abs(got - exact) <= rel * np.abs(exact) + 1e-6).all()
    # the rounding is real: most elements moved
    assert np.mean(got != exact) > 0.9


def test_identity_tables_leave_attention_unchanged():
    q, k, v = (rope.round_to_dtype(RNG.standard_normal((1, 4, 30, 16)).astype(np.float32), "bf16")
               for _ in range(3))
    k, v = k[:, :2], v[:, :2]
    ones, zeros = np.ones((64, 8), np.float32), np.zeros((64, 8), np.float32)
    for causal in (False, True):
        o1, l1 = rope.attention_rope(q, k, v, ones, zeros, True, "bf16", 0.25, causal)
        o2, l2 = attention(q, k, v, 0.25, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_query_chunk_positions_are_the_last_key_positions():
    """A chunk of the last 7 queries against 40 keys gives the rows of full self-attention."""
    q, k, v = (rope.round_to_dtype(RNG.standard_normal((1, 2, 40, 32)).astype(np.float32), "f16")
               for _ in range(3))
    cos, sin = (t.astype(np.float32) for t in rope.rotary_tables(64, 32))
    full_o, full_l = rope.attention_rope(q, k, v, cos, sin, False, "f16", 0.2, True)
    part_o, part_l = rope.attention_rope(q[:, :, -7:], k, v, cos, sin, False, "f16", 0.2, True)
    np.testing.assert_allclose(part_o, full_o[:, :, -7:], atol=1e-12)
    np.testing.assert_allclose(part_l, full_l[:, :, -7:], atol=1e-12)


def test_packed_sequences_restart_their_positions():
    lens_q, lens_k = (3, 0, 5), (10, 4, 5)
    q = rope.round_to_dtype(RNG.standard_normal((1, 2, 8, 16)).astype(np.float32), "bf16")
    k, v = (rope.round_to_dtype(RNG.standard_normal((1, 1, 19, 16)).astype(np.float32), "bf16")
            for _ in range(2))
    cu = np.array([0, 3, 3, 8])
    cu_k = np.array([0, 10, 14, 19])
    cos, sin = (t.astype(np.float32) for t in rope.rotary_tables(32, 16))
    o, l = rope.attention_rope(q, k, v, cos, sin, True, "bf16", 0.3, True, cu, cu_k)
    for (s0, s1), (t0, t1) in zip(zip(cu[:-1], cu[1:]), zip(cu_k[:-1], cu_k[1:])):
        if s1 == s0:
            continue
        o1, l1 = rope.attention_rope(q[:, :, s0:s1], k[:, :, t0:t1], v[:, :, t0:t1], cos, sin,
                                     True, "bf16", 0.3, True)
        np.testing.assert_allclose(o[:, :, s0:s1], o1, atol=1e-12)
        np.testing.assert_allclose(l[:, :, s0:s1], l1, atol=1e-12)


def test_queries_beyond_the_keys_sit_at_position_zero():
    assert list(rope.rope_positions(5, 3)) == [0, 0, 0, 1, 2]
    assert list(rope.rope_positions(4)) == [0, 1, 2, 3]
    assert list(rope.rope_positions(2, 9)) == [7, 8]


def test_a_planted_sign_error_is_caught():
    """A rotation by -angle keeps norms and relative positions but fails complex multiplication."""
    x = RNG.standard_normal((3, 8))
    cos, sin = rope.rotary_tables(3, 8)
    wrong = rope.rotate_exact(x, cos, -sin, True)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.arctan2(sin, cos))
    assert not np.allclose(wrong[:, 0::2], z.real, atol=1e-6)
