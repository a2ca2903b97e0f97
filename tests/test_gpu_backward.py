"""GPU parity of the backward pass (dQ, dK, dV) against the fp64 oracle, through the C-ABI.

Tolerance (a reading; the pages state none for gradients): the forward's bf16 / fp16 bounds
(1.6e-2 and 2e-3 on outputs of unit size) applied relative to each gradient's largest entry,
with the same floor of 1 that the LSE check uses: max |dX - dX_ref| <= tol * max(max |dX_ref|, 1).
The kernel rounds P and dS to the input type before the matrix products, which bounds the
error in that relative sense, not element by element (a gradient that is exactly 0 in fp64,
such as dQ of a row with one visible key, comes out as rounding noise).
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import download_bits, upload

pytestmark = pytest.mark.gpu

GRAD_TOL = {si.F16: 2e-3, si.BF16: 1.6e-2}


def run_backward(inp, dout_bits, max_seqlen=None):
    import exact_tiled_attention_39_amd as fa

    q, k, v = (upload(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    dout = upload(dout_bits, inp.dtype)
    cu = None
    if inp.cu_seqlens is not None:
        cu = torch.from_numpy(inp.cu_seqlens).cuda()
        if max_seqlen is None:
            max_seqlen = int(np.diff(inp.cu_seqlens).max()) if len(inp.cu_seqlens) > 1 else 0
    o, lse = fa.attention(q, k, v, scale=inp.scale, causal=inp.causal, cu_seqlens=cu,
                          max_seqlen=max_seqlen)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, dout, scale=inp.scale, causal=inp.causal,
                                       cu_seqlens=cu, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    return tuple(si.bits_to_f64(download_bits(x), inp.dtype) for x in (dq, dk, dv))


def oracle_backward(inp, dout_bits):
    q, k, v = inp.f64()
    do = si.bits_to_f64(dout_bits, inp.dtype)
    return oracle.attention_backward(q, k, v, do, inp.scale, inp.causal,
                                     cu_seqlens=inp.cu_seqlens)


def assert_grads_close(got, want, dtype, what):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        assert np.isfinite(g).all(), f"{what}: {name} not finite"
        ref = float(np.abs(w).max()) if w.size else 0.0
        err = float(np.abs(g - w).max()) if w.size else 0.0
        assert err <= GRAD_TOL[dtype] * max(ref, 1.0), \
            f"{what}: max|d{name}| = {err:.3e} > {GRAD_TOL[dtype]} x {ref:.3e}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 128, 129, 200, 257, 520])
def test_backward_small_shapes(n, d, dtype, causal):
    print(f"backward n={n} d={d} {dtype} causal={causal}", flush=True)
    inp = si.random_inputs(2 if n < 100 else 1, 2, 2, n, d, dtype, seed=500 + n + d,
                           causal=causal)
    dout = si.random_output_grad(inp, seed=n)
    assert_grads_close(run_backward(inp, dout), oracle_backward(inp, dout), dtype,
                       f"n={n} d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (6, 3), (4, 1)])
def test_backward_grouped_query_heads(hq, hkv, causal):
    inp = si.random_inputs(2, hq, hkv, 300, 128, si.BF16, seed=hq * 7 + hkv, causal=causal)
    dout = si.random_output_grad(inp, seed=3)
    assert_grads_close(run_backward(inp, dout), oracle_backward(inp, dout), si.BF16,
                       f"gqa {hq}/{hkv}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.BF16, 128), (si.F16, 64)])
def test_backward_packed_sequences(dtype, d, causal):
    lens = (0, 1, 127, 128, 129, 300, 0, 64, 5)
    inp = si.random_inputs(1, 4, 2, sum(lens), d, dtype, seed=81, causal=causal, seq_lens=lens)
    dout = si.random_output_grad(inp, seed=4)
    assert_grads_close(run_backward(inp, dout), oracle_backward(inp, dout), dtype, "varlen")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_scales(scale, causal):
    inp = si.random_inputs(1, 2, 2, 150, 64, si.F16, seed=32, causal=causal, scale=scale)
    dout = si.random_output_grad(inp, seed=5)
    got = run_backward(inp, dout)
    want = oracle_backward(inp, dout)
    assert_grads_close(got, want, si.F16, f"scale={scale}")
    if scale == 0.0:
        assert np.all(got[0] == 0) and np.all(got[1] == 0)


def test_backward_gradient_sums():
    """Key gradients of a head sum to ~0 (shift invariance of each row's softmax), and value
    gradients sum to the sum of the output gradients (rows of P sum to 1)."""
    inp = si.random_inputs(1, 4, 4, 1000, 128, si.BF16, seed=33, causal=True)
    dout = si.random_output_grad(inp, seed=6)
    dq, dk, dv = run_backward(inp, dout)
    do = si.bits_to_f64(dout, si.BF16)
    scale_k = np.abs(dk).sum(axis=2)
    assert np.all(np.abs(dk.sum(axis=2)) <= 2e-2 * scale_k)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=0,
                               atol=2e-2 * np.abs(dv).sum(axis=2).max())


@pytest.mark.parametrize("dtype,d,hq,hkv", [(si.BF16, 128, 8, 2), (si.F16, 64, 4, 4)])
def test_backward_is_deterministic(dtype, d, hq, hkv):
    """Every gradient accumulates in one workgroup's registers, in a fixed order: repeated calls
    give the same bits (the two wave groups of a step may run out of phase, never out of order
    on shared data). 3K tokens, causal, so that many ring steps run."""
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(1, hq, hkv, 3072, d, dtype, seed=91, causal=True)
    dout = upload(si.random_output_grad(inp, seed=92), dtype)
    q, k, v = (upload(x, dtype) for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention(q, k, v, scale=inp.scale, causal=True)
    first = None
    for _ in range(4):
        grads = fa.attention_backward(q, k, v, o, lse, dout, scale=inp.scale, causal=True)
        torch.cuda.synchronize()
        bits = [download_bits(g) for g in grads]
        if first is None:
            first = bits
        else:
            for a, b in zip(first, bits):
                np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("packed", [False, True])
def test_backward_workspace_contents(packed):
    """fa_bwd's workspace after a call: D = rowsum(dO * O) per query row (against the fp64 sum
    of the same dO and O values) in the first array, and -log2(e) * LSE in the second, the fp32
    product of the forward's LSE, bit for bit."""
    import exact_tiled_attention_39_amd as fa

    if packed:
        inp = si.random_inputs(1, 4, 2, 837, 128, si.BF16, seed=71, causal=True,
                               seq_lens=(300, 17, 520))
    else:
        inp = si.random_inputs(2, 4, 2, 333, 64, si.F16, seed=72, causal=False)
    dtype = inp.dtype
    q, k, v = (upload(x, dtype) for x in (inp.q, inp.k, inp.v))
    dout = upload(si.random_output_grad(inp, seed=73), dtype)
    cu = torch.from_numpy(inp.cu_seqlens).cuda() if packed else None
    max_seqlen = int(np.diff(inp.cu_seqlens).max()) if packed else None
    o, lse = fa.attention(q, k, v, scale=inp.scale, causal=inp.causal, cu_seqlens=cu,
                          max_seqlen=max_seqlen)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.full((2, *q.shape[:3]), float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, scale=inp.scale, causal=inp.causal,
              cu_seqlens=cu, max_seqlen=max_seqlen)
    torch.cuda.synchronize()
    got = delta.cpu().numpy()
    o64 = si.bits_to_f64(download_bits(o), dtype)
    do64 = si.bits_to_f64(download_bits(dout), dtype)
    d_ref = (o64 * do64).sum(axis=-1)
    # fp32 sums of d products: within 1e-5 of the sum of their magnitudes
    assert np.all(np.abs(got[0] - d_ref) <= 1e-5 * np.abs(o64 * do64).sum(axis=-1))
    nlse = (lse.cpu() * torch.tensor(-1.4426950408889634, dtype=torch.float32)).numpy()
    np.testing.assert_array_equal(got[1].view(np.uint32), nlse.view(np.uint32))


def test_backward_packed_with_larger_max_seqlen_bound():
    """max_seqlen only sizes the backward's grids: a loose upper bound (the packed total) gives
    the same gradients, bit for bit, as the longest sequence."""
    lens = (300, 17, 520, 64)
    inp = si.random_inputs(1, 4, 2, sum(lens), 128, si.BF16, seed=81, causal=True, seq_lens=lens)
    dout = si.random_output_grad(inp, seed=82)
    tight = run_backward(inp, dout)
    loose = run_backward(inp, dout, max_seqlen=sum(lens))
    for a, b in zip(tight, loose):
        np.testing.assert_array_equal(a, b)
    assert_grads_close(tight, oracle_backward(inp, dout), si.BF16, "packed, loose max_seqlen")
