"""Helpers shared by the GPU parity tests: upload seeded bits, run libfa, compare to the oracle."""
from __future__ import annotations

import numpy as np
import torch

import seeded_inputs as si

# Tolerances of the forward pass against the fp64 oracle: max |O_gpu - O_ref| per element by
# input type, and |LSE_gpu - LSE_ref| / max(|LSE_ref|, 1) per row.
O_TOL = {si.F16: 2e-3, si.BF16: 1.6e-2}
LSE_TOL = 1e-5

TORCH_DTYPE = {si.F16: torch.float16, si.BF16: torch.bfloat16}


def upload(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DTYPE[dtype])
    return t.to(device)


def download_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(inp: si.Inputs, device="cuda", max_seqlen=None, splits=None):
    """O (float64 of the output bits) and LSE of fa_fwd, or of fa_fwd_splitkv with `splits`
    (0: the library's choice)."""
    import exact_tiled_attention_39_amd as fa

    q = upload(inp.q, inp.dtype, device)
    k = upload(inp.k, inp.dtype, device)
    v = upload(inp.v, inp.dtype, device)
    cu = cu_k = None
    if inp.cu_seqlens is not None:
        cu = torch.from_numpy(inp.cu_seqlens).to(device)
        if max_seqlen is None:
            max_seqlen = int(np.diff(inp.cu_seqlens).max()) if len(inp.cu_seqlens) > 1 else 0
    if inp.cu_seqlens_k is not None:
        cu_k = torch.from_numpy(inp.cu_seqlens_k).to(device)
    if splits is None:
        o, lse = fa.attention(q, k, v, scale=inp.scale, causal=inp.causal, cu_seqlens=cu,
                              max_seqlen=max_seqlen, cu_seqlens_k=cu_k)
    else:
        o, lse = fa.attention_splitkv(q, k, v, scale=inp.scale, causal=inp.causal,
                                      num_splits=splits, cu_seqlens=cu, max_seqlen=max_seqlen,
                                      cu_seqlens_k=cu_k)
    torch.cuda.synchronize()
    return si.bits_to_f64(download_bits(o), inp.dtype), lse.cpu().numpy().astype(np.float64)


def errors(o, lse, o_ref, lse_ref):
    """(max |dO|, max LSE error) over the rows given (NaN anywhere counts as infinite). Rows
    that see no key must match exactly: O = 0 and LSE = -inf on both sides."""
    if not np.isfinite(o).all() or np.isnan(lse).any():
        return float("inf"), float("inf")
    empty = np.isneginf(lse_ref)
    if not np.array_equal(np.isneginf(lse), empty) or np.isposinf(lse).any():
        return float("inf"), float("inf")
    if empty.any() and (o[empty] != 0).any():
        return float("inf"), float("inf")
    do = float(np.abs(o - o_ref).max()) if o.size else 0.0
    lf, lr = lse[~empty], lse_ref[~empty]
    dl = float((np.abs(lf - lr) / np.maximum(np.abs(lr), 1.0)).max()) if lf.size else 0.0
    return do, dl


def assert_close(o, lse, o_ref, lse_ref, dtype, what=""):
    do, dl = errors(o, lse, o_ref, lse_ref)
    assert do <= O_TOL[dtype], f"{what}: max|dO| = {do:.3e} > {O_TOL[dtype]}"
    assert dl <= LSE_TOL, f"{what}: LSE error = {dl:.3e} > {LSE_TOL}"
    return do, dl
