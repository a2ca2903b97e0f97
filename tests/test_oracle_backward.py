"""Pins of the fp64 backward oracle (CPU only).

The oracle's gradients are checked against what fixes them independently of its own formulas:
central finite differences of the forward oracle, PyTorch autograd through SDPA in float64,
identities and invariants of the softmax gradient, closed forms and structural reductions.
Planted mistakes at the end must each be caught.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.backward as ob
from oracle import attention, attention_backward


def _problem(b, hq, hkv, n, d, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((b, hq, n, d)), r.standard_normal((b, hkv, n, d)),
            r.standard_normal((b, hkv, n, d)), r.standard_normal((b, hq, n, d)))


def _loss(q, k, v, w, scale, causal, cu=None):
    o, _ = attention(q, k, v, scale, causal, cu_seqlens=cu)
    return float((o * w).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv,cu,scale", [(2, 2, None, 0.7), (4, 2, None, -0.45),
                                             (2, 1, [0, 3, 3, 7], 1.3)])
def test_matches_central_finite_differences(causal, hq, hkv, cu, scale):
    """d/dx sum(O * W) by central differences of the forward oracle, every coordinate."""
    q, k, v, w = _problem(1, hq, hkv, 7, 3, seed=hq * 10 + hkv + causal)
    eps = 1e-6
    dq, dk, dv = attention_backward(q, k, v, w, scale, causal, cu_seqlens=cu)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _loss(q, k, v, w, scale, causal, cu)
            x[idx] = keep - eps
            dn = _loss(q, k, v, w, scale, causal, cu)
            x[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8)


def _autograd(q, k, v, do, scale, causal):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    rep = q.shape[1] // k.shape[1]
    o = F.scaled_dot_product_attention(tq, tk.repeat_interleave(rep, dim=1),
                                       tv.repeat_interleave(rep, dim=1), is_causal=causal,
                                       scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("b,hq,hkv,n,d,scale", [(2, 3, 3, 17, 8, 0.35), (1, 8, 2, 40, 16, 0.25),
                                                (1, 1, 1, 1, 4, 1.0), (2, 2, 1, 65, 32, 0.2)])
def test_matches_torch_autograd_float64(causal, b, hq, hkv, n, d, scale):
    q, k, v, do = _problem(b, hq, hkv, n, d, seed=n + d)
    got = attention_backward(q, k, v, do, scale, causal)
    want = _autograd(q, k, v, do, scale, causal)
    for g, w_ in zip(got, want):
        np.testing.assert_allclose(g, w_, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_delta_identity(causal):
    """rowsum(P * dP) = rowsum(dO * O) because O = P V."""
    q, k, v, do = _problem(1, 2, 2, 23, 8, seed=5)
    o, _, probs = attention(q, k, v, 0.5, causal, return_probs=True)
    dd = ob.output_gradient_rowsum(o, do)
    for h, p in enumerate(probs):
        dp = do[0, h] @ v[0, h].T
        np.testing.assert_allclose((p * dp).sum(axis=1), dd[0, h], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    """Shifting every key of a sequence by one vector leaves each row's softmax unchanged, so
    the key gradients of a (batch, kv head, sequence) sum to zero; the rows of P sum to one,
    so the value gradients sum to the sum of the output gradients of the rows that see them."""
    lens = [6, 0, 13, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = _problem(1, 4, 2, sum(lens), 8, seed=6)
    dq, dk, dv = attention_backward(q, k, v, do, 0.6, causal, cu_seqlens=cu)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        np.testing.assert_allclose(dk[0, :, s0:s1].sum(axis=1), 0.0, atol=1e-12)
        want = do[0, :, s0:s1].reshape(2, 2, s1 - s0, 8).sum(axis=(1, 2))
        np.testing.assert_allclose(dv[0, :, s0:s1].sum(axis=1), want, rtol=1e-12, atol=1e-12)


def test_zero_scale_closed_form():
    """scale 0: P is uniform over the visible keys, nothing flows to Q or K, and
    dV_j = sum over the rows i that see j of dO_i / |visible(i)|."""
    q, k, v, do = _problem(1, 1, 1, 9, 4, seed=7)
    dq, dk, dv = attention_backward(q, k, v, do, 0.0, True)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.array([sum(do[0, 0, i] / (i + 1) for i in range(j, 9)) for j in range(9)])
    np.testing.assert_allclose(dv[0, 0], want, rtol=1e-13, atol=1e-14)


def test_grouped_heads_equal_summed_repeated_heads():
    q, k, v, do = _problem(2, 6, 2, 11, 8, seed=8)
    dq, dk, dv = attention_backward(q, k, v, do, 0.4, True)
    dq2, dk2, dv2 = attention_backward(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), do,
                                       0.4, True)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(2, 2, 3, 11, 8).sum(axis=2), rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(2, 2, 3, 11, 8).sum(axis=2), rtol=1e-12,
                               atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_separate_sequences(causal):
    lens = [5, 0, 12, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = _problem(1, 2, 1, sum(lens), 8, seed=9)
    got = attention_backward(q, k, v, do, 0.5, causal, cu_seqlens=cu)
    for s0, s1 in zip(cu[:-1], cu[1:]):
        if s1 == s0:
            continue
        sl = slice(s0, s1)
        want = attention_backward(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.5,
                                  causal)
        for g, w_ in zip(got, want):
            np.testing.assert_array_equal(g[:, :, sl], w_)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_full_backward(causal):
    lens = [9, 0, 20, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, do = _problem(1, 4, 2, sum(lens), 8, seed=10)
    dq, _, _ = attention_backward(q, k, v, do, 0.45, causal, cu_seqlens=cu)
    rows = [(0, h, i) for h in range(4) for i in range(sum(lens))]
    got = ob.attention_backward_dq_rows(q, k, v, do, 0.45, causal, rows, cu_seqlens=cu)
    np.testing.assert_allclose(got, dq.reshape(-1, 8), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------------------------------
# Planted mistakes
# ------------------------------------------------------------------------------------------

def _failures():
    checks = [
        lambda: test_matches_torch_autograd_float64(True, 2, 3, 3, 17, 8, 0.35),
        lambda: test_matches_torch_autograd_float64(False, 1, 8, 2, 40, 16, 0.25),
        lambda: test_gradient_invariants(True),
    ]
    out = []
    for i, c in enumerate(checks):
        try:
            c()
        except AssertionError:
            out.append(i)
    return out


def test_pins_pass_on_the_backward_oracle():
    assert _failures() == []


MUTANTS = {
    "no_delta_subtraction": ("softmax_jacobian_product", lambda p, dp: p * dp),
    "delta_of_wrong_axis": ("softmax_jacobian_product",
                            lambda p, dp: p * (dp - (p * dp).sum(axis=0)[None, :])),
    "scale_dropped_in_dq_dk": ("_head_scores", None),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if name == "scale_dropped_in_dq_dk":
        orig = ob.attention_backward

        def patched(q, k, v, do, scale, causal=False, cu_seqlens=None):
            dq, dk, dv = orig(q, k, v, do, scale, causal, cu_seqlens)
            return dq / scale, dk / scale, dv
        monkeypatch.setattr(ob, "attention_backward", patched)
        monkeypatch.setitem(globals(), "attention_backward", patched)
    else:
        monkeypatch.setattr(ob, attr, fn)
    assert _failures(), f"planted mistake {name} went unnoticed"


@pytest.mark.parametrize("causal", [False, True])
def test_kv_rows_match_full_backward(causal):
    """Selected dK / dV rows, evaluated row batch by row batch, equal the full backward's."""
    rng = np.random.default_rng(41)
    q = rng.standard_normal((2, 4, 37, 16))
    k = rng.standard_normal((2, 2, 37, 16))
    v = rng.standard_normal((2, 2, 37, 16))
    do = rng.standard_normal((2, 4, 37, 16))
    _, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, causal)
    rows = [(0, 0, 0), (0, 1, 36), (1, 0, 17), (1, 1, 5), (1, 1, 6)]
    dk_r, dv_r = oracle.attention_backward_kv_rows(q, k, v, do, 0.3, causal, rows, chunk=10)
    for r, (b, hk, j) in enumerate(rows):
        np.testing.assert_allclose(dk_r[r], dk[b, hk, j], atol=1e-12)
        np.testing.assert_allclose(dv_r[r], dv[b, hk, j], atol=1e-12)
