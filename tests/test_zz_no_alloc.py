"""fa_fwd_splitkv_noalloc against fa_fwd_splitkv, through the C-ABI, on a gfx950 GPU.

The allocation-free entry point runs the same split and merge kernels as fa_fwd_splitkv, with
the split partials in the library's static per-GPU scratch instead of a caller workspace, so
its O and LSE must equal fa_fwd_splitkv's bit for bit. Two calls run back to back, the second
on a smaller problem: whatever the first left in the shared scratch must not reach the second's
output. Both results are also held to the forward's tolerances against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import assert_close, download_bits, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_39_amd as fa
    fa.load_library()  # fails loudly if the HIP library is missing


def _device_inputs(inp: si.Inputs):
    q, k, v = (upload(x, inp.dtype) for x in (inp.q, inp.k, inp.v))
    cu = torch.from_numpy(inp.cu_seqlens).cuda() if inp.cu_seqlens is not None else None
    cu_k = torch.from_numpy(inp.cu_seqlens_k).cuda() if inp.cu_seqlens_k is not None else None
    max_seqlen = (int(np.diff(inp.cu_seqlens).max()) if inp.cu_seqlens is not None else None)
    return q, k, v, dict(scale=inp.scale, causal=inp.causal, cu_seqlens=cu,
                         max_seqlen=max_seqlen, cu_seqlens_k=cu_k)


def _noalloc(fa, dev, splits):
    q, k, v, kw = dev
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, num_splits=splits, **kw)
    return o, lse


def _with_workspace(fa, dev, splits):
    q, k, v, kw = dev
    return fa.attention_splitkv(q, k, v, num_splits=splits, **kw)


def _same_bits(a, b):
    return np.array_equal(download_bits(a[0]), download_bits(b[0])) and np.array_equal(
        a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32))


def _check_oracle(inp, res):
    qf, kf, vf = inp.f64()
    o_ref, lse_ref = oracle.attention(qf, kf, vf, inp.scale, inp.causal,
                                      cu_seqlens=inp.cu_seqlens, cu_seqlens_k=inp.cu_seqlens_k)
    o = si.bits_to_f64(download_bits(res[0]), inp.dtype)
    assert_close(o, res[1].cpu().numpy().astype(np.float64), o_ref, lse_ref, inp.dtype,
                 "fa_fwd_splitkv_noalloc")


CASES = [
    # (first, larger call; second, smaller call; split count, 0 = the library's choice)
    (dict(batch=8, heads_q=32, heads_kv=8, seqlen=1, seqlen_k=4097, head_dim=128,
          dtype=si.BF16, causal=True, seed=71),
     dict(batch=2, heads_q=8, heads_kv=2, seqlen=3, seqlen_k=1000, head_dim=128,
          dtype=si.BF16, causal=True, seed=72), 0),
    (dict(batch=4, heads_q=16, heads_kv=4, seqlen=2, seqlen_k=3000, head_dim=64,
          dtype=si.F16, causal=False, seed=73),
     dict(batch=1, heads_q=4, heads_kv=4, seqlen=1, seqlen_k=33, head_dim=64,
          dtype=si.F16, causal=False, seed=74), 7),
]


@pytest.mark.parametrize("big,small,splits", CASES)
def test_two_calls_match_the_workspace_entry_point(big, small, splits):
    import exact_tiled_attention_39_amd as fa

    inp_big, inp_small = si.random_inputs(**big), si.random_inputs(**small)
    print(f"noalloc: {big} then {small}, splits {splits}", flush=True)
    dev_big, dev_small = _device_inputs(inp_big), _device_inputs(inp_small)
    torch.cuda.synchronize()
    got_big = _noalloc(fa, dev_big, splits)
    got_small = _noalloc(fa, dev_small, splits)  # right after, on the same scratch
    torch.cuda.synchronize()
    ref_big = _with_workspace(fa, dev_big, splits)
    ref_small = _with_workspace(fa, dev_small, splits)
    torch.cuda.synchronize()
    assert _same_bits(got_big, ref_big)
    assert _same_bits(got_small, ref_small)
    _check_oracle(inp_big, got_big)
    _check_oracle(inp_small, got_small)


def test_packed_sequences_then_smaller():
    import exact_tiled_attention_39_amd as fa

    big = si.random_inputs(batch=1, heads_q=32, heads_kv=8, seqlen=6, seqlen_k=4922,
                           head_dim=128, dtype=si.BF16, causal=True, seed=75,
                           seq_lens=(1, 2, 0, 3),
                           seq_lens_k=(3000, 17, 5, 1900))
    small = si.random_inputs(batch=1, heads_q=8, heads_kv=8, seqlen=2, seqlen_k=601,
                             head_dim=128, dtype=si.BF16, causal=True, seed=76,
                             seq_lens=(1, 1), seq_lens_k=(600, 1))
    print("noalloc: packed sequences then a smaller packed call", flush=True)
    db, ds = _device_inputs(big), _device_inputs(small)
    torch.cuda.synchronize()
    gb = _noalloc(fa, db, 0)
    gs = _noalloc(fa, ds, 0)
    torch.cuda.synchronize()
    assert _same_bits(gb, _with_workspace(fa, db, 0))
    assert _same_bits(gs, _with_workspace(fa, ds, 0))
    _check_oracle(big, gb)
    _check_oracle(small, gs)


def test_allocates_nothing_and_rejects_oversized_plans():
    import exact_tiled_attention_39_amd as fa

    inp = si.random_inputs(batch=8, heads_q=32, heads_kv=8, seqlen=1, seqlen_k=2048,
                           head_dim=128, dtype=si.BF16, causal=True, seed=77)
    dev = _device_inputs(inp)
    q, k, v, kw = dev
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, num_splits=16, **kw)  # first call on the device
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(5):
        fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, num_splits=16, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert _same_bits((o, lse), _with_workspace(fa, dev, 16))
    # a plan whose partials exceed the static scratch is refused before any device call
    p = fa.make_params(q, k, v, o, lse, inp.scale, inp.causal, None, None, None)
    splits, need = fa.fa_splitkv_plan(p, 256)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, num_splits=256, **kw)
    assert e.value.status == fa.FA_ERR_SCRATCH
