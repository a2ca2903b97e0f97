"""Parity of the HIP forward pass (through the C-ABI) with the fp64 oracle, on a gfx950 GPU.

Tolerances: max |O_gpu - O_ref| <= 2e-3 (fp16) or 1.6e-2 (bf16) per element, and
|LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) <= 1e-5 per row. Small shapes are compared on every
row; the full-size workloads on seeded row samples plus properties checked on every row.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import seeded_inputs as si
from gpu_util import LSE_TOL, O_TOL, assert_close, download_bits, run, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_39_amd as fa
    fa.load_library()  # fails loudly if the HIP library is missing


def _oracle(inp: si.Inputs):
    q, k, v = inp.f64()
    return oracle.attention(q, k, v, inp.scale, inp.causal, cu_seqlens=inp.cu_seqlens,
                            cu_seqlens_k=inp.cu_seqlens_k)


SMALL_N = [1, 2, 3, 63, 64, 65, 127, 128, 129, 200, 257, 520]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", SMALL_N)
def test_small_shapes(n, d, dtype, causal):
    hq, hkv = (2, 1) if n % 2 else (2, 2)
    inp = si.random_inputs(2 if n < 100 else 1, hq, hkv, n, d, dtype, seed=1000 + n + d,
                           causal=causal)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, f"n={n} d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (8, 1), (6, 3)])
def test_grouped_query_heads(hq, hkv, causal):
    inp = si.random_inputs(2, hq, hkv, 300, 128, si.BF16, seed=hq * 10 + hkv, causal=causal)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.BF16, f"gqa {hq}/{hkv}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.BF16, 128), (si.F16, 64)])
def test_packed_variable_lengths(dtype, d, causal):
    lens = (0, 1, 127, 128, 129, 300, 0, 64, 5)
    inp = si.random_inputs(1, 4, 2, sum(lens), d, dtype, seed=77, causal=causal, seq_lens=lens)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, "varlen")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv,lens", [(8, 8, None), (16, 8, None), (8, 8, (0, 129, 300, 5, 520)),
                                         (24, 8, (257, 1, 64))])
def test_kv_heads_dealt_over_xcds(hq, hkv, lens, causal):
    """heads_kv a multiple of 8 selects the head-strided workgroup order (every XCD takes every
    eighth kv head with its query heads); the result must not depend on the order."""
    n = 300 if lens is None else sum(lens)
    inp = si.random_inputs(1 if lens else 2, hq, hkv, n, 64, si.F16, seed=hq + hkv + n,
                           causal=causal, seq_lens=lens)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.F16, f"heads {hq}/{hkv} lens={lens}")


# Query chunks against key/value contexts of another length (chunked prefill, KV cache).
CHUNK_CASES = [(1, 300), (64, 192), (100, 1000), (257, 520), (200, 200), (300, 100), (65, 1),
               (40, 0)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.F16, 64), (si.BF16, 128)])
@pytest.mark.parametrize("nq,nk", CHUNK_CASES)
def test_query_chunk_against_other_key_length(nq, nk, dtype, d, causal):
    inp = si.random_inputs(2, 4, 2, nq, d, dtype, seed=3 * nq + nk + d, causal=causal,
                           seqlen_k=nk)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, f"nq={nq} nk={nk} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d,hq,hkv", [(si.BF16, 128, 4, 2), (si.F16, 64, 16, 8)])
def test_packed_chunks_with_their_own_key_ranges(dtype, d, hq, hkv, causal):
    lens_q = (0, 1, 127, 64, 5, 300, 2, 3)
    lens_k = (3, 1, 300, 64, 0, 300, 700, 1)
    inp = si.random_inputs(1, hq, hkv, sum(lens_q), d, dtype, seed=91, causal=causal,
                           seq_lens=lens_q, seqlen_k=sum(lens_k), seq_lens_k=lens_k)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, "packed chunks")


def test_packed_with_larger_max_seqlen_bound():
    """max_seqlen only sizes the grid: a loose upper bound gives the same result."""
    lens = (100, 260, 3)
    inp = si.random_inputs(1, 2, 2, sum(lens), 128, si.BF16, seed=78, causal=True, seq_lens=lens)
    o1, l1 = run(inp)
    o2, l2 = run(inp, max_seqlen=sum(lens))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0, 1e-3])
@pytest.mark.parametrize("causal", [False, True])
def test_scales(scale, causal):
    inp = si.random_inputs(1, 2, 2, 150, 64, si.F16, seed=31, causal=causal, scale=scale)
    o, lse = run(inp)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.F16, f"scale={scale}")


@pytest.mark.parametrize("dtype", [si.F16, si.BF16])
def test_worked_example_row_1_5_3(dtype):
    """14cs17 notes, Worked Examples, Example 2, as one attention row: q = (1, 5, 3, 0, ...),
    keys and values e0, e1, e2, scale 1 -> O row 0 = softmax([1, 5, 3]) padded with zeros."""
    d, n = 64, 3
    q = np.zeros((1, 1, n, d))
    q[0, 0, 0, :3] = [1.0, 5.0, 3.0]
    q[0, 0, 1, :3] = [2.0, -1.0, 0.5]
    q[0, 0, 2, :3] = [0.25, 0.0, -2.0]
    kv = np.zeros((1, 1, n, d))
    kv[0, 0, np.arange(3), np.arange(3)] = 1.0
    inp = si.Inputs(si.f64_to_bits(q, dtype), si.f64_to_bits(kv, dtype), si.f64_to_bits(kv, dtype),
                    dtype, 1.0, False)
    o, lse = run(inp)
    want = scipy.special.softmax([1.0, 5.0, 3.0])
    assert np.abs(o[0, 0, 0, :3] - want).max() <= O_TOL[dtype]
    assert (o[0, 0, 0, 3:] == 0).all()
    lse_want = scipy.special.logsumexp([1.0, 5.0, 3.0])
    assert abs(lse[0, 0, 0] - lse_want) / lse_want <= LSE_TOL
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, "worked example")


def test_token_major_strided_layout():
    """[B, N, H, d] storage viewed as [B, H, N, d]; O written into a strided view as well."""
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(2, 4, 2, 333, 128, si.BF16, seed=5, causal=True)
    q = upload(inp.q, si.BF16).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    k = upload(inp.k, si.BF16).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    v = upload(inp.v, si.BF16).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert q.stride() == (333 * 4 * 128, 128, 4 * 128, 1)
    o_store = torch.zeros(2, 333, 4, 128, dtype=torch.bfloat16, device="cuda")
    o = o_store.permute(0, 2, 1, 3)
    lse = torch.empty(2, 4, 333, dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=inp.scale, causal=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(inp)
    assert_close(si.bits_to_f64(download_bits(o), si.BF16), lse.cpu().numpy().astype(np.float64),
                 o_ref, lse_ref, si.BF16, "strided")


def test_runs_on_a_side_stream_and_is_deterministic():
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(1, 4, 4, 700, 128, si.BF16, seed=6, causal=True)
    q, k, v = (upload(x, si.BF16) for x in (inp.q, inp.k, inp.v))
    o1, l1 = fa.attention(q, k, v, causal=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_allocates_no_device_memory():
    """Theorem 3 of the 14cs17 notes: memory is O(N); the library itself allocates nothing."""
    import exact_tiled_attention_39_amd as fa

    n = 8192
    inp = si.random_inputs(1, 8, 8, n, 128, si.BF16, seed=7, causal=True)
    q, k, v = (upload(x, si.BF16) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty(1, 8, n, dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=inp.scale, causal=True)  # first call loads the code object
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        fa.fa_fwd(q, k, v, o, lse, scale=inp.scale, causal=True)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    # the scores of one head alone would take N^2 fp32 words; nothing of that size appeared
    assert oracle.score_matrix_bytes(n, 4) == 256 * 2 ** 20


# ------------------------------------------------------------------------------------------
# Full-size workloads
# ------------------------------------------------------------------------------------------

def _segments(w):
    if w.seq_lens is None:
        return [(0, w.seqlen)]
    cu = w.cu_seqlens()
    return list(zip(cu[:-1].tolist(), cu[1:].tolist()))


def _check_properties(w, inp, o_bits, lse):
    """On every row: O lies in the per-column range of the visible values; for causal rows the
    log-sum-exp is at least the diagonal score and at most ln(#keys) + max visible score bound."""
    tol = O_TOL[w.dtype]
    group = w.heads_q // w.heads_kv
    for b in range(w.batch):
        for hk in range(w.heads_kv):
            vh = si.bits_to_f64(inp.v[b, hk], w.dtype).astype(np.float32)
            kh = si.bits_to_f64(inp.k[b, hk], w.dtype)
            knorm = np.linalg.norm(kh, axis=1)
            for s0, s1 in _segments(w):
                if s1 == s0:
                    continue
                seg = vh[s0:s1]
                if w.causal:
                    lo = np.minimum.accumulate(seg, axis=0)
                    hi = np.maximum.accumulate(seg, axis=0)
                    kmax = np.maximum.accumulate(knorm[s0:s1])
                else:
                    lo = np.broadcast_to(seg.min(axis=0), seg.shape)
                    hi = np.broadcast_to(seg.max(axis=0), seg.shape)
                    kmax = np.full(s1 - s0, knorm[s0:s1].max())
                for h in range(hk * group, (hk + 1) * group):
                    oh = si.bits_to_f64(o_bits[b, h, s0:s1], w.dtype).astype(np.float32)
                    assert np.isfinite(oh).all()
                    assert (oh >= lo - tol).all() and (oh <= hi + tol).all(), (b, h, s0)
                    qh = si.bits_to_f64(inp.q[b, h, s0:s1], w.dtype)
                    lh = lse[b, h, s0:s1]
                    cnt = np.arange(1, s1 - s0 + 1) if w.causal else np.full(s1 - s0, s1 - s0)
                    upper = np.log(cnt) + abs(w.scale) * np.linalg.norm(qh, axis=1) * kmax
                    assert (lh <= upper * (1 + 1e-5) + 1e-5).all(), (b, h, s0)
                    if w.causal:
                        diag = w.scale * np.einsum("nd,nd->n", qh, kh[s0:s1])
                        assert (lh >= diag - LSE_TOL * np.maximum(1, np.abs(diag))).all()


@pytest.mark.parametrize("name", si.WORKLOAD_ORDER)
def test_workload_full_size(name):
    import exact_tiled_attention_39_amd as fa

    w = si.WORKLOADS[name]
    print(f"workload {name}", flush=True)
    inp = si.workload_inputs(w)
    q, k, v = (upload(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens).cuda() if w.varlen else None
    cu_k = torch.from_numpy(inp.cu_seqlens_k).cuda() if inp.cu_seqlens_k is not None else None
    kw = dict(scale=w.scale, causal=w.causal, cu_seqlens=cu,
              max_seqlen=w.max_seqlen() if w.varlen else None, cu_seqlens_k=cu_k)
    # decode workloads run through both entry points
    runs = [("fa_fwd", fa.attention(q, k, v, **kw))]
    if w.splitkv:
        runs.append(("fa_fwd_splitkv", fa.attention_splitkv(q, k, v, **kw)))
    assert k.shape[2] == w.keys
    torch.cuda.synchronize()
    results = [(entry, download_bits(o), l.cpu().numpy().astype(np.float64))
               for entry, (o, l) in runs]
    del q, k, v, runs
    qf, kf, vf = (si.bits_to_f64(x, w.dtype).astype(np.float32) for x in (inp.q, inp.k, inp.v))
    if w.batch * w.heads_q * w.seqlen <= 2 ** 17:
        o_ref, lse_ref = oracle.attention(qf, kf, vf, w.scale, w.causal, cu_seqlens=inp.cu_seqlens,
                                          cu_seqlens_k=inp.cu_seqlens_k)
        for entry, o_bits, lse in results:
            assert_close(si.bits_to_f64(o_bits, w.dtype), lse, o_ref, lse_ref, w.dtype,
                         f"{name} via {entry}")
    else:
        (_, o_bits, lse), = results
        rows = si.sample_rows(w, 1 / 512, seed=w.seed)
        o_ref, lse_ref = oracle.attention_rows(qf, kf, vf, w.scale, w.causal, rows,
                                               cu_seqlens=inp.cu_seqlens)
        idx = tuple(np.array(rows).T)
        assert_close(si.bits_to_f64(o_bits[idx], w.dtype), lse[idx], o_ref, lse_ref, w.dtype,
                     f"{name} ({len(rows)} sampled rows)")
        _check_properties(w, inp, o_bits, lse)
