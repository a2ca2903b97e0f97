"""Large sizes on a gfx950 GPU: 64-bit offsets and long loops, checked on sampled rows against the
oracle (the forward's tolerances).

* fa_fwd with N = 131072 (one head, causal bf16): 2048 key tiles per row block, offsets past 2^31
  elements in the score index space.
* fa_fwd_splitkv against a 1,200,000-key cache (8 kv heads, 2.3 GiB per K and V tensor; kv head 7
  starts past 2^31 bytes), one query per head.
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


def test_forward_131072_tokens():
    import exact_tiled_attention_39_amd as fa

    n = 131072
    print(f"forward N={n}", flush=True)
    inp = si.random_inputs(1, 1, 1, n, 128, si.BF16, seed=901, causal=True)
    q, k, v = (upload(x, si.BF16) for x in (inp.q, inp.k, inp.v))
    o, lse = fa.attention(q, k, v, scale=inp.scale, causal=True)
    torch.cuda.synchronize()
    o_b, lse = download_bits(o), lse.cpu().numpy().astype(np.float64)
    rows = [(0, 0, t) for t in (0, 1, 255, 256, 65535, 65536, n - 257, n - 256, n - 2, n - 1)]
    qf, kf, vf = (si.bits_to_f64(x, si.BF16).astype(np.float32) for x in (inp.q, inp.k, inp.v))
    o_ref, lse_ref = oracle.attention_rows(qf, kf, vf, inp.scale, True, rows)
    idx = tuple(np.array(rows).T)
    assert_close(si.bits_to_f64(o_b[idx], si.BF16), lse[idx], o_ref, lse_ref, si.BF16, "N=131072")


def test_splitkv_against_1200000_keys():
    import exact_tiled_attention_39_amd as fa

    nk, hkv, hq, d = 1_200_000, 8, 32, 128
    print(f"split-KV decode against {nk} keys", flush=True)
    rng = np.random.default_rng(902)
    # K and V repeat a seeded block of 4099 rows (a prime, so no tile sees an aligned copy)
    block = 4099
    kb = si.round_to_bits(rng.standard_normal((hkv, block, d), dtype=np.float32), si.BF16)
    vb = si.round_to_bits(rng.standard_normal((hkv, block, d), dtype=np.float32), si.BF16)
    qb = si.round_to_bits(rng.standard_normal((1, hq, 1, d), dtype=np.float32), si.BF16)
    reps = -(-nk // block)
    k = upload(kb, si.BF16).repeat(1, reps, 1)[:, :nk].unsqueeze(0).contiguous()
    v = upload(vb, si.BF16).repeat(1, reps, 1)[:, :nk].unsqueeze(0).contiguous()
    q = upload(qb, si.BF16)
    assert k.shape == (1, hkv, nk, d) and k.stride(1) * 2 * (hkv - 1) > 2 ** 31  # head 7
    o, lse = fa.attention_splitkv(q, k, v, scale=d ** -0.5, causal=True)
    torch.cuda.synchronize()
    o_b, lse = download_bits(o), lse.cpu().numpy().astype(np.float64)
    del k, v

    # the oracle on the query heads of kv heads 0 and 7 (the last sits past 2^31 bytes)
    def decode(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32)

    heads = [0, 7]
    kf = decode(np.tile(kb[heads], (1, reps, 1))[:, :nk])[None]
    vf = decode(np.tile(vb[heads], (1, reps, 1))[:, :nk])[None]
    qh = [h for g in heads for h in range(4 * g, 4 * g + 4)]
    qf = decode(qb[:, qh])
    rows = [(0, i, 0) for i in range(len(qh))]
    o_ref, lse_ref = oracle.attention_rows(qf, kf, vf, d ** -0.5, True, rows)
    got = si.bits_to_f64(o_b[0, qh, 0], si.BF16)
    assert_close(got, lse[0, qh, 0], o_ref, lse_ref, si.BF16, "1M-key split-KV")
