"""The backward pass, RoPE and FP8 at the headline workload's full size (B=1, H=32, N=16384,
d=128, causal), in the launch configuration bench.py times, against the oracle on sampled rows.

Backward: dQ of a seeded 1/64 of the query rows, and dK / dV of 16 keys of every kv head
(first, last, tile- and block-edge, and seeded keys), with the backward tolerance
max|dX - dX_ref| <= tol(dtype) * max(max|dX_ref|, 1); the oracle runs on 16 host threads. RoPE: every
rotated key bit for bit, sampled O / LSE rows with the forward's tolerances. FP8: sampled rows
with the bounds of oracle.fp8.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
import oracle.rope as orope
import seeded_inputs as si
from gpu_util import assert_close, download_bits, upload

pytestmark = pytest.mark.gpu

W = si.WORKLOADS[si.HEADLINE]
GRAD_TOL = {si.F16: 2e-3, si.BF16: 1.6e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_39_amd as fa
    fa.load_library()  # fails loudly if the HIP library is missing


@pytest.fixture(scope="module")
def inputs():
    return si.workload_inputs(W)


def _f32(x):
    return si.bits_to_f64(x, W.dtype).astype(np.float32)


@pytest.fixture(scope="module")
def backward_result(inputs):
    """dQ, dK, dV bits of one fa_bwd call on the headline workload, and its dO bits."""
    import exact_tiled_attention_39_amd as fa

    print("backward at full size", flush=True)
    dout = si.random_output_grad(inputs, seed=W.seed + 100)
    q, k, v, do = (upload(x, W.dtype) for x in (inputs.q, inputs.k, inputs.v, dout))
    o, lse = fa.attention(q, k, v, scale=W.scale, causal=W.causal)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, scale=W.scale, causal=W.causal)
    torch.cuda.synchronize()
    out = dout, download_bits(dq), download_bits(dk), download_bits(dv)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def _pool_map(fn, items):
    import os
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as pool:
        return list(pool.map(fn, items))


def test_backward_dq_rows_full_size(inputs, backward_result):
    """dQ of a seeded 1/64 of the query rows (8,192 rows plus the edge rows) of every head."""
    dout, dq_b, _, _ = backward_result
    qf, kf, vf, dof = (_f32(x) for x in (inputs.q, inputs.k, inputs.v, dout))
    rows = si.sample_rows(W, 1 / 64, seed=21)
    chunks = [rows[i:i + 256] for i in range(0, len(rows), 256)]
    refs = _pool_map(lambda c: oracle.attention_backward_dq_rows(qf, kf, vf, dof, W.scale,
                                                                 W.causal, c), chunks)
    ref = np.concatenate(refs)
    got = si.bits_to_f64(dq_b[tuple(np.array(rows).T)], W.dtype)
    err, top = float(np.abs(got - ref).max()), float(np.abs(ref).max())
    print(f"dQ: {len(rows)} rows, max err {err:.3e}, max |ref| {top:.3e}, "
          f"ratio to the bound {err / (GRAD_TOL[W.dtype] * max(top, 1.0)):.3f}", flush=True)
    assert len(rows) >= W.batch * W.heads_q * W.seqlen // 64
    assert err <= GRAD_TOL[W.dtype] * max(top, 1.0)


def test_backward_dkdv_rows_full_size(inputs, backward_result):
    """dK and dV of 16 keys of every kv head (512 key rows): the first and last keys, tile and
    block edges, and seeded keys, each against every query row that sees it."""
    dout, _, dk_b, dv_b = backward_result
    qf, kf, vf, dof = (_f32(x) for x in (inputs.q, inputs.k, inputs.v, dout))
    n = W.seqlen
    rng = np.random.default_rng(23)
    fixed = [0, 1, 63, 64, 255, 256, n // 2, n - 257, n - 2, n - 1]
    per_head = []
    for hk in range(W.heads_kv):
        extra = sorted(set(rng.integers(0, n, 32).tolist()) - set(fixed))[:6]
        per_head.append([(0, hk, j) for j in fixed + extra])
    res = _pool_map(lambda kr: oracle.attention_backward_kv_rows(qf, kf, vf, dof, W.scale,
                                                                 W.causal, kr), per_head)
    krows = [r for kr in per_head for r in kr]
    dk_ref = np.concatenate([r[0] for r in res])
    dv_ref = np.concatenate([r[1] for r in res])
    assert len(krows) >= 256 and len({hk for _, hk, _ in krows}) == W.heads_kv
    idx = tuple(np.array(krows).T)
    for name, got_b, r in (("dK", dk_b, dk_ref), ("dV", dv_b, dv_ref)):
        got = si.bits_to_f64(got_b[idx], W.dtype)
        err, top = float(np.abs(got - r).max()), float(np.abs(r).max())
        print(f"{name}: {len(krows)} key rows, max err {err:.3e}, max |ref| {top:.3e}, "
              f"ratio to the bound {err / (GRAD_TOL[W.dtype] * max(top, 1.0)):.3f}", flush=True)
        assert err <= GRAD_TOL[W.dtype] * max(top, 1.0), name


def test_rope_full_size(inputs):
    import exact_tiled_attention_39_amd as fa

    print("RoPE at full size", flush=True)
    cos, sin = (t.astype(np.float32) for t in orope.rotary_tables(W.seqlen, W.head_dim))
    q, k, v = (upload(x, W.dtype) for x in (inputs.q, inputs.k, inputs.v))
    o, lse, k_rot = fa.attention(q, k, v, scale=W.scale, causal=W.causal,
                                 rope_cos=torch.from_numpy(cos).cuda(),
                                 rope_sin=torch.from_numpy(sin).cuda(), return_k_rot=True)
    torch.cuda.synchronize()
    o_b, kr_b = download_bits(o), download_bits(k_rot)
    lse = lse.cpu().numpy().astype(np.float64)
    del q, k, v, o, k_rot
    qf, kf, vf = (_f32(x) for x in (inputs.q, inputs.k, inputs.v))
    kr_ref = orope.rotate_rounded(kf, cos, sin, False, "bf16")
    assert np.array_equal(si.bits_to_f64(kr_b, W.dtype), kr_ref), "rotated keys differ"
    rows = si.sample_rows(W, 1 / 2048, seed=22)
    o_ref, lse_ref = orope.attention_rope_rows(qf, kf, vf, cos, sin, False, "bf16", W.scale,
                                               W.causal, rows)
    idx = tuple(np.array(rows).T)
    assert_close(si.bits_to_f64(o_b[idx], W.dtype), lse[idx], o_ref, lse_ref, W.dtype,
                 f"RoPE full size ({len(rows)} rows)")


def test_fp8_full_size():
    import exact_tiled_attention_39_amd as fa

    print("FP8 at full size", flush=True)
    inp = si.random_inputs_fp8(W.batch, W.heads_q, W.heads_kv, W.seqlen, W.head_dim, W.seed,
                               causal=W.causal, scale=W.scale)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    o, lse = fa.attention_fp8(up(inp.q), up(inp.k), up(inp.v), up(inp.q_descale),
                              up(inp.k_descale), up(inp.v_descale), scale=W.scale,
                              causal=W.causal)
    torch.cuda.synchronize()
    o_b = download_bits(o)
    lse = lse.cpu().numpy().astype(np.float64)
    q, k, v = (ofp8.dequantize(c, d).astype(np.float32) for c, d in
               ((inp.q, inp.q_descale), (inp.k, inp.k_descale), (inp.v, inp.v_descale)))
    rows = si.sample_rows(W, 1 / 2048, seed=23)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, W.scale, W.causal, rows)
    idx = tuple(np.array(rows).T)
    e_s = ofp8.score_error_bound(q, k, W.scale, W.head_dim)
    tol = ofp8.o_tolerance(v, W.seqlen, e_s)
    err = np.abs(si.bits_to_f64(o_b[idx], si.BF16) - o_ref)
    dl = np.abs(lse[idx] - lse_ref)
    print(f"FP8 full size ({len(rows)} rows): max|dO| {err.max():.3e} (bound {tol:.3e}), "
          f"max|dLSE| {dl.max():.3e} (e_S {e_s:.3e})", flush=True)
    assert err.max() <= tol and err.mean() <= tol / 16
    assert (dl <= ofp8.lse_tolerance(lse_ref, e_s)).all()
    assert np.isfinite(lse).all()
