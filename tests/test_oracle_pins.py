"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage or the mathematical fact it relies on. The mutation tests at the
end plant plausible mistakes in single steps of the oracle and check that the pins catch them.
"""
import json
import math
import pathlib

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import oracle.definition as oa
from oracle import attention, attention_rows, flash_forward, scalar
from oracle.online import online_lse

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(b, hq, hkv, n, d, seed, std=1.0):
    r = _rng(seed)
    return (r.standard_normal((b, hq, n, d)) * std, r.standard_normal((b, hkv, n, d)) * std,
            r.standard_normal((b, hkv, n, d)))


# ------------------------------------------------------------------------------------------
# Worked examples printed on the pages
# ------------------------------------------------------------------------------------------

def test_p1_example2_blocked_equals_standard_softmax():
    """14cs17 notes, Worked Examples, Example 2: [1, 5, 3] as blocks [1, 5] then [3]."""
    g = json.loads((GOLDEN / "p1_example2_online_softmax.json").read_text())
    row = g["row"]
    m, l = online_lse(row, [len(b) for b in g["blocks"]])
    online = [math.exp(x - m) / l for x in row]
    standard = scalar.standard_softmax(row)
    for a, b in zip(online, standard):
        assert abs(a - b) <= g["ulp_budget"] * math.ulp(b)
    np.testing.assert_allclose(standard, scipy.special.softmax(row), rtol=1e-15, atol=0)
    # closed forms: p_j / p_i = e^(x_j - x_i); the running maximum of the merge is the row max
    assert m == 5.0
    assert math.isclose(online[1] / online[0], math.exp(4.0), rel_tol=1e-14)
    assert math.isclose(online[2] / online[0], math.exp(2.0), rel_tol=1e-14)
    assert math.isclose(m + math.log(l), scipy.special.logsumexp(row), rel_tol=1e-15)


def test_p1_example2_embedded_in_attention():
    """The same example as one attention row: q = (1, 5, 3, 0), K = V = (e0, e1, e2), scale 1."""
    g = json.loads((GOLDEN / "p1_example2_online_softmax.json").read_text())
    row = g["row"]
    d, n = 4, 3
    q = np.zeros((1, 1, n, d))
    q[0, 0, 0, :3] = row
    q[0, 0, 1:] = _rng(3).standard_normal((n - 1, d))
    eye = np.eye(n, d)
    k = eye[None, None].copy()
    v = eye[None, None].copy()
    o, lse = attention(q, k, v, 1.0)
    want = scipy.special.softmax(row)
    np.testing.assert_allclose(o[0, 0, 0, :3], want, rtol=1e-15, atol=1e-17)
    assert o[0, 0, 0, 3] == 0.0
    assert math.isclose(lse[0, 0, 0], scipy.special.logsumexp(row), rel_tol=1e-15)
    # the tiled algorithm with the page's split [2, 1] reaches the same row
    o2, lse2 = flash_forward(q[0, 0], k[0, 0], v[0, 0], 1.0, col_blocks=[2, 1], block_rows=1)
    np.testing.assert_allclose(o2[0, :3], want, rtol=4e-16 * 8, atol=1e-17)
    assert math.isclose(lse2[0], lse[0, 0, 0], rel_tol=1e-15)


def test_p3_two_pass_online_normaliser():
    """xspy page, section 3: two-pass online normaliser == standard softmax, diff < 1e-15."""
    g = json.loads((GOLDEN / "p3_online_softmax_chunks.json").read_text())
    chunks = g["chunks"]
    flat = [x for c in chunks for x in c]
    probs, m, d = scalar.online_softmax_two_pass(chunks)
    std = scalar.standard_softmax(flat)
    assert max(abs(a - b) for a, b in zip(probs, std)) < g["max_abs_diff_bound"]
    assert m == max(flat)
    np.testing.assert_allclose(std, scipy.special.softmax(flat), rtol=1e-14, atol=0)
    assert math.isclose(math.log(d) + m, scipy.special.logsumexp(flat), rel_tol=1e-15)
    # the array merge of oracle.online streams the same chunks to the same (max, sum)
    m2, l2 = online_lse(flat, [len(c) for c in chunks])
    assert m2 == m and math.isclose(l2, d, rel_tol=1e-15)


def test_p1_score_matrix_sizes():
    """14cs17 notes, Core Intuition and Example 1: the N x N FP16 matrix never stored."""
    g = json.loads((GOLDEN / "p1_score_matrix_sizes.json").read_text())
    for c in g["cases"]:
        assert oracle.score_matrix_bytes(c["n"], c["bytes_per_element"]) == c["gib"] * 2 ** 30


# ------------------------------------------------------------------------------------------
# Tiling is exact (the pages' central claim) for arbitrary block partitions
# ------------------------------------------------------------------------------------------

def _random_partition(r, n):
    sizes, left = [], n
    while left:
        s = int(r.integers(1, left + 1)) if r.random() < 0.5 else int(r.integers(1, min(left, 8) + 1))
        sizes.append(s)
        left -= s
    return sizes


def test_tiled_online_equals_definition_random_partitions():
    r = _rng(11)
    worst = 0.0
    for _ in range(1000):
        n = int(r.integers(1, 40))
        d = int(r.choice([1, 2, 3, 8]))
        causal = bool(r.random() < 0.5)
        scale = float(r.uniform(-2.0, 2.0))
        q, k, v = (r.standard_normal((n, d)) * 2 for _ in range(3))
        o_ref, lse_ref = attention(q[None, None], k[None, None], v[None, None], scale, causal)
        o, lse = flash_forward(q, k, v, scale, causal, row_blocks=_random_partition(r, n),
                               col_blocks=_random_partition(r, n))
        err = np.abs(o - o_ref[0, 0]).max() / max(1.0, np.abs(o_ref).max())
        err = max(err, (np.abs(lse - lse_ref[0, 0]) / np.maximum(1.0, np.abs(lse_ref[0, 0]))).max())
        worst = max(worst, err)
    assert worst <= 1e-13


# ------------------------------------------------------------------------------------------
# An independent library routine: PyTorch's SDPA math path in float64 on the CPU
# ------------------------------------------------------------------------------------------

SDPA_CASES = [
    (1, 1, 1, 7, 5, False, 0.3),
    (2, 3, 3, 33, 16, True, 0.25),
    (1, 8, 2, 40, 8, True, 1 / math.sqrt(8)),
    (2, 4, 1, 17, 4, False, -0.7),
    (1, 2, 2, 65, 64, True, 0.125),
]


def _sdpa(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    gqa = tq.shape[1] != tk.shape[1]
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=gqa)
    kk = tk.repeat_interleave(tq.shape[1] // tk.shape[1], dim=1)
    sc = scale * torch.matmul(tq, kk.transpose(-1, -2).contiguous())
    if causal:
        n = tq.shape[2]
        sc = sc.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
    return o.numpy(), torch.logsumexp(sc, dim=-1).numpy()


@pytest.mark.parametrize("b,hq,hkv,n,d,causal,scale", SDPA_CASES)
def test_matches_torch_sdpa_float64(b, hq, hkv, n, d, causal, scale):
    q, k, v = _qkv(b, hq, hkv, n, d, seed=n * 31 + d)
    o, lse = attention(q, k, v, scale, causal)
    o_t, lse_t = _sdpa(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------------------------------
# Invariants
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_are_distributions_consistent_with_lse(causal):
    q, k, v = _qkv(1, 2, 2, 50, 8, seed=5, std=1.5)
    scale = 0.4
    o, lse, probs = attention(q, k, v, scale, causal, return_probs=True)
    for h, p in enumerate(probs):
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        s = scale * (q[0, h] @ k[0, h].T)
        vis = np.tril(np.ones_like(s, dtype=bool)) if causal else np.ones_like(s, dtype=bool)
        np.testing.assert_allclose(p[vis], np.exp(s - lse[0, h][:, None])[vis], rtol=1e-13)
        assert (p[~vis] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_output_is_convex_combination_of_values(causal):
    q, k, v = _qkv(1, 3, 3, 64, 16, seed=8, std=2.0)
    o, _ = attention(q, k, v, 0.3, causal)
    for h in range(3):
        for i in range(64):
            keys = slice(0, i + 1) if causal else slice(0, 64)
            lo = v[0, h, keys].min(axis=0)
            hi = v[0, h, keys].max(axis=0)
            assert (o[0, h, i] >= lo - 1e-14).all() and (o[0, h, i] <= hi + 1e-14).all()


def test_joint_permutation_of_keys_and_values():
    q, k, v = _qkv(2, 2, 2, 37, 8, seed=9)
    perm = _rng(10).permutation(37)
    o1, l1 = attention(q, k, v, 0.5, False)
    o2, l2 = attention(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


@pytest.mark.parametrize("delta", [3.0, 1000.0])
def test_shift_of_one_query_row(delta):
    """Adding delta to every score of a row leaves O unchanged and shifts lse by delta."""
    q, k, v = _qkv(1, 1, 1, 20, 6, seed=12)
    k[..., -1] = 1.0
    scale = 1.0
    o1, l1 = attention(q, k, v, scale, True)
    q2 = q.copy()
    q2[0, 0, 7, -1] += delta
    o2, l2 = attention(q2, k, v, scale, True)
    np.testing.assert_allclose(o2[0, 0, 7], o1[0, 0, 7], rtol=0, atol=1e-12)
    assert math.isclose(l2[0, 0, 7] - l1[0, 0, 7], delta * scale, rel_tol=1e-12)
    np.testing.assert_array_equal(o2[0, 0, :7], o1[0, 0, :7])


# ------------------------------------------------------------------------------------------
# Closed forms
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_uniform_when_scores_vanish(causal):
    _, k, v = _qkv(1, 1, 1, 24, 8, seed=13)
    q = np.zeros((1, 1, 24, 8))
    for qq, scale in ((q, 0.7), (_qkv(1, 1, 1, 24, 8, seed=14)[0], 0.0)):
        o, lse = attention(qq, k, v, scale, causal)
        for i in range(24):
            cnt = i + 1 if causal else 24
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, :cnt].mean(axis=0), atol=1e-14)
            assert math.isclose(lse[0, 0, i], math.log(cnt), rel_tol=1e-14, abs_tol=1e-15)


def test_causal_first_row_sees_only_itself():
    q, k, v = _qkv(1, 1, 1, 9, 5, seed=15)
    o, lse = attention(q, k, v, 0.9, True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    assert math.isclose(lse[0, 0, 0], 0.9 * math.fsum(q[0, 0, 0] * k[0, 0, 0]), rel_tol=1e-14)


def test_one_hot_values_return_probabilities():
    n = 12
    q, k, _ = _qkv(1, 1, 1, n, n, seed=16)
    v = np.eye(n)[None, None]
    o, lse, probs = attention(q, k, v, 0.5, False, return_probs=True)
    np.testing.assert_allclose(o[0, 0], probs[0], atol=1e-16)
    np.testing.assert_allclose(o[0, 0].sum(axis=1), 1.0, atol=1e-14)
    want = scipy.special.softmax(0.5 * (q[0, 0] @ k[0, 0].T), axis=1)
    np.testing.assert_allclose(o[0, 0], want, atol=1e-15)


def test_one_dominant_score_selects_its_value():
    n, d = 16, 8
    q, k, v = _qkv(1, 1, 1, n, d, seed=17)
    k[0, 0] *= 0.01
    k[0, 0, 5] = 0.0
    k[0, 0, 5, 0] = 100.0
    q[0, 0, :, 0] = 1.0
    o, lse = attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 5], (n, d)), atol=1e-12)


# ------------------------------------------------------------------------------------------
# Brute force on tiny inputs (pure Python, correctly rounded sums)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(n, d, causal):
    q, k, v = _qkv(1, 1, 1, n, d, seed=100 * n + 10 * d + causal)
    o, lse = attention(q, k, v, 0.8, causal)
    o_s, lse_s = scalar.attention_scalar(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                         0.8, causal)
    np.testing.assert_allclose(o[0, 0], np.array(o_s), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.array(lse_s), rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------------------------------
# Structural reductions
# ------------------------------------------------------------------------------------------

def test_gqa_equals_mha_on_repeated_heads():
    q, k, v = _qkv(2, 8, 2, 21, 8, seed=18)
    o, lse = attention(q, k, v, 0.35, True)
    o2, lse2 = attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.35, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_separate_sequences(causal):
    lens = [5, 0, 11, 1, 7]
    n = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v = _qkv(1, 3, 3, n, 8, seed=19)
    o, lse = attention(q, k, v, 0.5, causal, cu_seqlens=cu)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        o1, l1 = attention(q[:, :, s0:s1], k[:, :, s0:s1], v[:, :, s0:s1], 0.5, causal)
        np.testing.assert_array_equal(o[:, :, s0:s1], o1)
        np.testing.assert_array_equal(lse[:, :, s0:s1], l1)


def test_causal_row_equals_noncausal_prefix():
    q, k, v = _qkv(1, 1, 1, 30, 8, seed=20)
    o, lse = attention(q, k, v, 0.6, True)
    for i in (0, 1, 13, 29):
        o1, l1 = attention(q[:, :, :i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.6, False)
        np.testing.assert_allclose(o[0, 0, i], o1[0, 0, i], atol=1e-15)
        assert math.isclose(lse[0, 0, i], l1[0, 0, i], rel_tol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_row_evaluation_matches_full_evaluation(causal):
    lens = [9, 0, 20, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n = int(cu[-1])
    q, k, v = _qkv(1, 4, 2, n, 8, seed=21)
    o, lse = attention(q, k, v, 0.5, causal, cu_seqlens=cu)
    rows = [(0, h, i) for h in range(4) for i in range(n)]
    o_r, lse_r = attention_rows(q, k, v, 0.5, causal, rows, cu_seqlens=cu)
    np.testing.assert_allclose(o_r, o.reshape(-1, 8), atol=1e-14)
    np.testing.assert_allclose(lse_r, lse.reshape(-1), rtol=1e-14)
    q2, k2, v2 = _qkv(2, 2, 2, 25, 4, seed=22)
    o2, l2 = attention(q2, k2, v2, 0.5, causal)
    rows2 = [(1, 1, 0), (0, 0, 24), (1, 0, 12)]
    o_r2, l_r2 = attention_rows(q2, k2, v2, 0.5, causal, rows2)
    for r, (b, h, i) in enumerate(rows2):
        np.testing.assert_allclose(o_r2[r], o2[b, h, i], atol=1e-14)
        assert math.isclose(l_r2[r], l2[b, h, i], rel_tol=1e-14)


# ------------------------------------------------------------------------------------------
# Queries and keys of different lengths (a query chunk against a key/value cache)
# ------------------------------------------------------------------------------------------

def test_chunked_prefill_rows_equal_full_causal_rows():
    """Chunked prefill (xspy page, section 1; the notes' KV-cache composability) computes the
    same rows as full causal attention: the last c queries against all N keys and values give
    exactly the last c rows of causal self-attention over N tokens."""
    q, k, v = _qkv(1, 2, 1, 37, 8, seed=40)
    o, lse = attention(q, k, v, 0.45, True)
    for c in (1, 5, 36, 37):
        oc, lc = attention(q[:, :, -c:], k, v, 0.45, True)
        np.testing.assert_allclose(oc, o[:, :, -c:], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lc, lse[:, :, -c:], rtol=1e-14, atol=0)


def test_packed_chunks_equal_full_causal_rows():
    """The same for packed sequences, each with its own chunk length and key length."""
    full = [7, 12, 1, 9]
    chunk = [3, 12, 1, 0]
    q, k, v = _qkv(1, 2, 2, sum(full), 4, seed=41)
    cu_full = np.concatenate([[0], np.cumsum(full)])
    cu_chunk = np.concatenate([[0], np.cumsum(chunk)])
    o, lse = attention(q, k, v, 0.7, True, cu_seqlens=cu_full)
    take = np.concatenate([np.arange(e - c, e) for e, c in zip(cu_full[1:], chunk)]).astype(int)
    oc, lc = attention(q[:, :, take], k, v, 0.7, True, cu_seqlens=cu_chunk, cu_seqlens_k=cu_full)
    np.testing.assert_allclose(oc, o[:, :, take], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lc, lse[:, :, take], rtol=1e-14, atol=0)


def test_chunk_longer_than_keys_has_empty_rows():
    """With more queries than keys the first Nq - Nk causal rows see no key (reading: O = 0,
    LSE = -inf); the others are causal self-attention over the Nk keys."""
    q, k, v = _qkv(1, 1, 1, 9, 4, seed=42)
    k, v = k[:, :, :4], v[:, :, :4]
    o, lse = attention(q, k, v, 0.9, True)
    assert np.all(o[0, 0, :5] == 0.0) and np.all(np.isneginf(lse[0, 0, :5]))
    o2, l2 = attention(q[:, :, 5:], k, v, 0.9, True)
    np.testing.assert_array_equal(o[:, :, 5:], o2)
    np.testing.assert_array_equal(lse[:, :, 5:], l2)
    o3, l3 = attention(q, k[:, :, :0], v[:, :, :0], 0.9, False)
    assert np.all(o3 == 0.0) and np.all(np.isneginf(l3))


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 6), (2, 5), (4, 4), (5, 2), (3, 0)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny_unequal_lengths(nq, nk, causal):
    r = _rng(nq * 10 + nk)
    q, k, v = r.standard_normal((1, 1, nq, 3)), r.standard_normal((1, 1, nk, 3)), \
        r.standard_normal((1, 1, nk, 3))
    o, lse = attention(q, k, v, 0.8, causal)
    o_s, lse_s = scalar.attention_scalar(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                         0.8, causal)
    np.testing.assert_allclose(o[0, 0], np.array(o_s), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.array(lse_s), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("nq,nk", [(3, 17), (17, 3), (1, 40)])
def test_unequal_lengths_match_torch_sdpa_float64(nq, nk):
    """Non-causal attention with Nq != Nk against PyTorch SDPA in float64."""
    r = _rng(nq + 100 * nk)
    q = r.standard_normal((2, 4, nq, 8))
    k, v = r.standard_normal((2, 2, nk, 8)), r.standard_normal((2, 2, nk, 8))
    o, lse = attention(q, k, v, 0.3, False)
    o_t, lse_t = _sdpa(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_row_evaluation_matches_full_evaluation_unequal_lengths(causal):
    full = [9, 3, 20]
    chunk = [4, 3, 0]
    cu_k = np.concatenate([[0], np.cumsum(full)])
    cu_q = np.concatenate([[0], np.cumsum(chunk)])
    r = _rng(43)
    q = r.standard_normal((1, 4, sum(chunk), 8))
    k, v = r.standard_normal((1, 2, sum(full), 8)), r.standard_normal((1, 2, sum(full), 8))
    o, lse = attention(q, k, v, 0.5, causal, cu_seqlens=cu_q, cu_seqlens_k=cu_k)
    rows = [(0, h, i) for h in range(4) for i in range(sum(chunk))]
    o_r, lse_r = attention_rows(q, k, v, 0.5, causal, rows, cu_seqlens=cu_q, cu_seqlens_k=cu_k)
    np.testing.assert_allclose(o_r, o.reshape(-1, 8), atol=1e-14)
    np.testing.assert_allclose(lse_r, lse.reshape(-1), rtol=1e-14)


# ------------------------------------------------------------------------------------------
# Planted mistakes: each must be caught by at least one of the pins above
# ------------------------------------------------------------------------------------------

def _pin_failures():
    """Re-runs a selection of the pins against the (possibly patched) oracle."""
    failures = []
    checks = [
        lambda: [test_matches_torch_sdpa_float64(*c) for c in SDPA_CASES],
        lambda: test_shift_of_one_query_row(1000.0),
        lambda: test_causal_first_row_sees_only_itself(),
        lambda: test_uniform_when_scores_vanish(True),
        lambda: test_p1_example2_embedded_in_attention(),
        lambda: test_chunked_prefill_rows_equal_full_causal_rows(),
    ]
    for i, chk in enumerate(checks):
        try:
            with np.errstate(all="ignore"):
                chk()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failures.append(i)
    return failures


def test_pins_pass_on_the_oracle():
    assert _pin_failures() == []


MUTANTS = {
    "causal_excludes_diagonal": ("_allowed", lambda nq, nk, causal: (
        np.arange(nk)[None, :] < np.arange(nq)[:, None] + (nk - nq)) if causal
        else np.ones((nq, nk), bool)),
    "causal_off_by_one_late": ("_allowed", lambda nq, nk, causal: (
        np.arange(nk)[None, :] <= np.arange(nq)[:, None] + (nk - nq) + 1) if causal
        else np.ones((nq, nk), bool)),
    "chunk_aligned_to_key_start": ("_allowed", lambda nq, nk, causal: (
        np.arange(nk)[None, :] <= np.arange(nq)[:, None]) if causal
        else np.ones((nq, nk), bool)),
    "scale_dropped": ("_head_scores", lambda qh, kh, scale: qh @ kh.T),
    "scores_transposed": ("_head_scores", lambda qh, kh, scale: scale * (kh @ qh.T)),
    "gqa_heads_interleaved": ("kv_head", lambda h, hq, hkv: h % hkv),
    "no_max_subtraction": ("softmax_rows_with_lse", lambda s, allowed: (
        (lambda e: (e / e.sum(axis=1)[:, None], np.log(e.sum(axis=1))))(
            np.where(allowed, np.exp(np.where(allowed, s, -np.inf)), 0.0)))),
    "lse_missing_max": ("softmax_rows_with_lse", lambda s, allowed: (
        (lambda p, l: (p, l - np.where(allowed, s, -np.inf).max(axis=1)))(
            *oa.__dict__["_orig_softmax"](s, allowed)))),
    "unnormalised_output": ("_mix", lambda p, vh: (p * 1.5) @ vh),
    "values_transposed": ("_mix", lambda p, vh: p @ vh[::-1]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, "_orig_softmax", oa.softmax_rows_with_lse, raising=False)
    monkeypatch.setattr(oa, attr, fn)
    assert _pin_failures(), f"planted mistake {name} went unnoticed"
