"""Parity of the split-KV forward (fa_fwd_splitkv through the C-ABI) with the fp64 oracle on a
gfx950 GPU: few query tokens per sequence against many keys (decode with a KV cache).

The split kernels compute the same function as fa_fwd, so the oracle and the tolerances are the
forward's: max |O_gpu - O_ref| <= 2e-3 (fp16) or 1.6e-2 (bf16) per element and
|LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) <= 1e-5 per row, on every row.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import assert_close, download_bits, run, upload

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


@pytest.mark.parametrize("splits", [0, 1, 7])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.F16, 64), (si.BF16, 128)])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 4)])
@pytest.mark.parametrize("nk", [1, 33, 1000, 4097])
@pytest.mark.parametrize("nq", [1, 3])
def test_decode_shapes(nq, nk, hq, hkv, dtype, d, causal, splits):
    print(f"splitkv nq={nq} nk={nk} hq={hq} hkv={hkv} {dtype} d={d} causal={causal} "
          f"splits={splits}", flush=True)
    inp = si.random_inputs(2, hq, hkv, nq, d, dtype, seed=nq * 7919 + nk + hq + d, causal=causal,
                           seqlen_k=nk)
    o, lse = run(inp, splits=splits)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, f"nq={nq} nk={nk} splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv,nq", [(8, 1, 5), (16, 1, 4), (4, 2, 40), (2, 2, 100)])
def test_several_row_blocks(hq, hkv, nq, causal):
    """group * nq above 32: packed rows span several 32-row blocks, each with its own causal
    key range."""
    inp = si.random_inputs(1, hq, hkv, nq, 128, si.BF16, seed=hq * 31 + nq, causal=causal,
                           seqlen_k=700)
    for splits in (0, 3):
        o, lse = run(inp, splits=splits)
        o_ref, lse_ref = _oracle(inp)
        assert_close(o, lse, o_ref, lse_ref, si.BF16, f"hq={hq} nq={nq} splits={splits}")


@pytest.mark.parametrize("splits", [0, 4])
def test_more_queries_than_keys(splits):
    """Causal queries before the first key position see nothing: O = 0, LSE = -inf."""
    inp = si.random_inputs(2, 4, 2, 40, 64, si.F16, seed=404, causal=True, seqlen_k=8)
    o, lse = run(inp, splits=splits)
    o_ref, lse_ref = _oracle(inp)
    assert np.isneginf(lse_ref).sum() == 2 * 4 * 32
    assert_close(o, lse, o_ref, lse_ref, si.F16, "nq > nk")


@pytest.mark.parametrize("splits", [1, 16, 256])
def test_more_splits_than_tiles(splits):
    """Most splits hold no tile: their partials are skipped by the merge."""
    inp = si.random_inputs(3, 8, 2, 2, 128, si.BF16, seed=55, causal=True, seqlen_k=40)
    o, lse = run(inp, splits=splits)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.BF16, f"splits={splits}")


@pytest.mark.parametrize("splits", [0, 1, 5])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.F16, 64), (si.BF16, 128)])
def test_packed_cache_lengths(dtype, d, causal, splits):
    lens_q = (1, 1, 3, 0, 2, 1, 1)
    lens_k = (1000, 0, 50, 7, 2, 4097, 31)
    inp = si.random_inputs(1, 8, 2, sum(lens_q), d, dtype, seed=606, causal=causal,
                           seq_lens=lens_q, seqlen_k=sum(lens_k), seq_lens_k=lens_k)
    o, lse = run(inp, splits=splits)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, dtype, f"packed splits={splits}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 2.0])
def test_scales(scale):
    inp = si.random_inputs(2, 8, 2, 1, 128, si.BF16, seed=77, causal=True, seqlen_k=2000,
                           scale=scale)
    o, lse = run(inp, splits=6)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.BF16, f"scale={scale}")


def test_workspace_contents_do_not_matter_and_results_repeat():
    """A workspace full of NaN bit patterns gives the same bits as a fresh one, call after
    call, on a side stream."""
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(4, 16, 4, 1, 128, si.BF16, seed=12, causal=True, seqlen_k=3000)
    q, k, v = (upload(x, si.BF16) for x in (inp.q, inp.k, inp.v))
    outs = []
    for fill in (0, 0xFF, 0xFF):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        p = fa.make_params(q, k, v, o, lse, inp.scale, True, None, None)
        _, nbytes = fa.fa_splitkv_plan(p, 9)
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        fa.fa_fwd_splitkv(q, k, v, o, lse, ws, scale=inp.scale, causal=True, num_splits=9,
                          stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        outs.append((download_bits(o), lse.cpu().numpy()))
    for o_bits, l in outs[1:]:
        np.testing.assert_array_equal(o_bits, outs[0][0])
        np.testing.assert_array_equal(l, outs[0][1])
    o_ref, lse_ref = _oracle(inp)
    assert_close(si.bits_to_f64(outs[0][0], si.BF16), outs[0][1].astype(np.float64), o_ref,
                 lse_ref, si.BF16, "NaN-filled workspace")


def test_split_count_changes_only_rounding():
    """Every split count computes the same function; results agree to the tolerance."""
    inp = si.random_inputs(2, 8, 8, 1, 64, si.F16, seed=99, causal=False, seqlen_k=5000)
    o_ref, lse_ref = _oracle(inp)
    for splits in (1, 2, 13, 64, 157):
        o, lse = run(inp, splits=splits)
        assert_close(o, lse, o_ref, lse_ref, si.F16, f"splits={splits}")


@pytest.mark.parametrize("n_seqs", [64, 65])
@pytest.mark.parametrize("splits", [0, 5])
def test_many_packed_sequences_with_tied_lengths(n_seqs, splits):
    """Up to 64 packed sequences run longest first (ties by index); more run in launch order.
    Both orders cover every (sequence, kv head, range) once: lengths with ties, zero-length
    caches and sequences without queries, against the oracle."""
    rng = np.random.default_rng(640 + n_seqs)
    lens_k = [int(x) for x in rng.choice([0, 31, 32, 300, 300, 300, 777, 1500], size=n_seqs)]
    lens_q = [int(x) for x in rng.choice([0, 1, 1, 2], size=n_seqs)]
    inp = si.random_inputs(1, 4, 2, sum(lens_q), 64, si.F16, seed=641, causal=True,
                           seq_lens=tuple(lens_q), seqlen_k=sum(lens_k), seq_lens_k=tuple(lens_k))
    o, lse = run(inp, splits=splits)
    o_ref, lse_ref = _oracle(inp)
    assert_close(o, lse, o_ref, lse_ref, si.F16, f"{n_seqs} packed sequences, splits={splits}")
