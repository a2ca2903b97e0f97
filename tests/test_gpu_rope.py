"""RoPE on the GPU (through the C-ABI) against the oracle (oracle/rope.py).

The rotated keys written by the key pass must equal the oracle's rotation bit for bit (the
rotation's fp32 steps and its rounding are fixed by the library's reading). O and LSE are
compared with the forward's tolerances against the attention definition on the oracle's rotated
Q and K: max |dO| <= 2e-3 (fp16) or 1.6e-2 (bf16), LSE error <= 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle.rope as orope
import seeded_inputs as si
from gpu_util import TORCH_DTYPE, assert_close, download_bits, upload

pytestmark = pytest.mark.gpu

ODT = {si.F16: "f16", si.BF16: "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_39_amd as fa
    fa.load_library()  # fails loudly if the HIP library is missing


def _tables(rows, d):
    cos, sin = orope.rotary_tables(max(rows, 1), d)
    return cos.astype(np.float32), sin.astype(np.float32)


def _run(inp: si.Inputs, interleaved, *, keys_rotated=False, splits=None, table_rows=None,
         in_place=False):
    """(O, LSE, rotated keys as float64 or None) from the GPU."""
    import exact_tiled_attention_39_amd as fa

    d = inp.q.shape[-1]
    rows = table_rows if table_rows is not None else inp.k.shape[2]
    cos, sin = _tables(rows, d)
    kbits = inp.k
    if keys_rotated:  # K handed over already rotated (the oracle's rotation, as a cache holds)
        _, kr = orope.apply_rope(*_f64(inp)[:2], cos, sin, interleaved, ODT[inp.dtype],
                                 inp.cu_seqlens, inp.cu_seqlens_k)
        kbits = si.f64_to_bits(kr, inp.dtype)
    q, k, v = upload(inp.q, inp.dtype), upload(kbits, inp.dtype), upload(inp.v, inp.dtype)
    tc, ts = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    cu = torch.from_numpy(inp.cu_seqlens).cuda() if inp.cu_seqlens is not None else None
    cu_k = torch.from_numpy(inp.cu_seqlens_k).cuda() if inp.cu_seqlens_k is not None else None
    max_seqlen = (int(np.diff(inp.cu_seqlens).max()) if inp.cu_seqlens is not None else None)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    k_rot = None if keys_rotated else (k if in_place else torch.empty_like(k))
    kw = dict(scale=inp.scale, causal=inp.causal, cu_seqlens=cu, max_seqlen=max_seqlen,
              cu_seqlens_k=cu_k, rope_cos=tc, rope_sin=ts, rope_interleaved=interleaved,
              k_rot=k_rot)
    if splits is None:
        fa.fa_fwd(q, k, v, o, lse, **kw)
    else:
        p = fa.make_params(q, k, v, o, lse, inp.scale, inp.causal, cu, max_seqlen, cu_k, tc, ts,
                           interleaved, k_rot)
        _, nbytes = fa.fa_splitkv_plan(p, splits)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
        fa.fa_fwd_splitkv(q, k, v, o, lse, ws, num_splits=splits, **kw)
    torch.cuda.synchronize()
    kr = None if k_rot is None else si.bits_to_f64(download_bits(k_rot), inp.dtype)
    return (si.bits_to_f64(download_bits(o), inp.dtype), lse.cpu().numpy().astype(np.float64),
            kr, cos, sin)


def _f64(inp):
    return inp.f64()


def _check(inp, interleaved, what, **kw):
    o, lse, kr, cos, sin = _run(inp, interleaved, **kw)
    q, k, v = _f64(inp)
    qr, kr_ref = orope.apply_rope(q, k, cos, sin, interleaved, ODT[inp.dtype], inp.cu_seqlens,
                                  inp.cu_seqlens_k)
    if kr is not None:
        assert np.array_equal(kr, kr_ref), f"{what}: rotated keys differ from the oracle's"
    from oracle import attention
    o_ref, lse_ref = attention(qr, kr_ref, v, inp.scale, inp.causal, cu_seqlens=inp.cu_seqlens,
                               cu_seqlens_k=inp.cu_seqlens_k)
    assert_close(o, lse, o_ref, lse_ref, inp.dtype, what)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.F16, 64), (si.BF16, 128)])
@pytest.mark.parametrize("n", [1, 65, 300])
def test_self_attention(n, dtype, d, causal, interleaved):
    inp = si.random_inputs(2, 4, 2, n, d, dtype, seed=700 + n + d, causal=causal)
    _check(inp, interleaved, f"n={n} d={d} causal={causal} interleaved={interleaved}")


@pytest.mark.parametrize("interleaved", [False, True])
def test_keys_already_rotated(interleaved):
    inp = si.random_inputs(1, 8, 2, 200, 128, si.BF16, seed=711, causal=True)
    _check(inp, interleaved, "keys rotated", keys_rotated=True)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(64, 300), (1, 500), (300, 100)])
def test_query_chunk_positions(nq, nk, causal, interleaved):
    inp = si.random_inputs(2, 4, 4, nq, 64, si.F16, seed=720 + nq, causal=causal, seqlen_k=nk)
    _check(inp, interleaved, f"chunk nq={nq} nk={nk}", table_rows=nk)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("dtype,d", [(si.F16, 64), (si.BF16, 128)])
def test_packed_sequences(dtype, d, interleaved):
    lens_q = (0, 1, 127, 64, 5, 300, 2)
    lens_k = (3, 1, 300, 64, 0, 300, 700)
    inp = si.random_inputs(1, 4, 2, sum(lens_q), d, dtype, seed=730, causal=True,
                           seq_lens=lens_q, seqlen_k=sum(lens_k), seq_lens_k=lens_k)
    _check(inp, interleaved, "packed", table_rows=max(lens_k))


@pytest.mark.parametrize("keys_rotated", [False, True])
@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("nq", [1, 3])
def test_split_kv_decode(nq, splits, keys_rotated):
    inp = si.random_inputs(2, 8, 2, nq, 128, si.BF16, seed=740 + nq, causal=True, seqlen_k=1000)
    _check(inp, False, f"split-KV nq={nq} splits={splits}", splits=splits,
           keys_rotated=keys_rotated)


def test_rotation_in_place():
    inp = si.random_inputs(1, 2, 2, 150, 128, si.BF16, seed=750, causal=True)
    _check(inp, True, "in place", in_place=True)


def test_negative_scale_rotates_before_negating():
    inp = si.random_inputs(1, 4, 4, 129, 64, si.F16, seed=751, causal=False, scale=-0.3)
    _check(inp, False, "scale -0.3")


def test_identity_tables_give_the_plain_forward_bit_for_bit():
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(1, 4, 2, 257, 128, si.BF16, seed=752, causal=True)
    q, k, v = (upload(x, si.BF16) for x in (inp.q, inp.k, inp.v))
    ones = torch.ones(257, 64, dtype=torch.float32, device="cuda")
    zeros = torch.zeros(257, 64, dtype=torch.float32, device="cuda")
    o1, l1, kr = fa.attention(q, k, v, scale=inp.scale, causal=True, rope_cos=ones,
                              rope_sin=zeros, return_k_rot=True)
    o2, l2 = fa.attention(q, k, v, scale=inp.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(kr.view(torch.int16), k.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
