"""Seeded synthetic inputs for exact tiled attention, shared by the tests, the bench and smoke().

This module holds no attention arithmetic. It only draws random numbers, rounds them to the
storage dtype (fp16 or bf16, round-to-nearest-even) and decodes stored bit patterns back to
float64. Both the HIP path and the fp64 oracle consume exactly the same bit patterns, so a
parity tolerance measures the kernel's error and not the input quantisation.

The first five workloads mirror the problem statement of the forward pass (Q, K, V and O as
batch x heads x N x d, a scale, a causal flag, a GQA head ratio, packed variable-length
sequences). The shape of the second one is the SDPA usage example on the FromZero2AI page
("FlashAttention: GPU Memory-Bound Speedups for Long-Context LLMs", section "Code Verification").
The sixth is a query chunk against a longer key/value context (chunked prefill with a KV
cache, xspy page "FlashAttention and chunked prefill mechanics", section 1). The last two are
decode steps against a KV cache (one new query token per sequence; the cache the notes list
among the compositions of the method, "Connection to the Broader Curriculum"): a batch of equal
cache lengths, and packed sequences whose cache lengths are drawn uniformly from a range.

Draw order per workload: (varlen only) the sequence lengths, then Q, then K, then V, each as
float32 standard normals in C order of shape [B, H, N, d] (K and V with the key length); the
optional multiplier is applied before rounding.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask mode and the recipe of its random values."""

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int  # tokens per batch entry; total packed tokens for varlen
    head_dim: int
    dtype: str
    causal: bool
    seed: int
    qk_multiplier: float = 1.0
    seq_lens: Optional[Tuple[int, ...]] = None  # varlen only (batch == 1)
    seqlen_k: Optional[int] = None  # keys per batch entry when it differs from seqlen
    seq_lens_k: Optional[Tuple[int, ...]] = None  # varlen keys, when packed unlike the queries
    splitkv: bool = False  # run by the split-KV entry point (few queries per sequence)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def varlen(self) -> bool:
        return self.seq_lens is not None

    def cu_seqlens(self) -> Optional[np.ndarray]:
        if self.seq_lens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)

    def cu_seqlens_k(self) -> Optional[np.ndarray]:
        if self.seq_lens_k is None:
            return None
        return np.concatenate([[0], np.cumsum(self.seq_lens_k)]).astype(np.int32)

    def max_seqlen(self) -> int:
        return max(self.seq_lens) if self.seq_lens is not None else self.seqlen

    @property
    def keys(self) -> int:
        """Key tokens per batch entry (packed total for varlen)."""
        return self.seqlen if self.seqlen_k is None else self.seqlen_k

    def flops(self) -> float:
        """FLOPs by the metric convention: 4*N^2*d per (batch, head), halved when causal.

        For packed sequences the count is summed per sequence. With Nq queries against Nk keys
        it is 4*Nq*Nk*d, less 2*Nq^2*d when causal (the same convention at Nq == Nk).
        """
        if self.seq_lens_k is not None:
            per = sum(4.0 * self.head_dim * (nq * nk - (nq * nq / 2.0 if self.causal else 0.0))
                      for nq, nk in zip(self.seq_lens, self.seq_lens_k))
            return per * self.heads_q
        if self.seqlen_k is not None:
            nq, nk = self.seqlen, self.seqlen_k
            per = 4.0 * self.head_dim * (nq * nk - (nq * nq / 2.0 if self.causal else 0.0))
            return per * self.heads_q * self.batch
        lens = self.seq_lens if self.seq_lens is not None else (self.seqlen,) * self.batch
        per = sum(4.0 * n * n * self.head_dim for n in lens) * self.heads_q
        return per / 2.0 if self.causal else per


    def io_bytes(self) -> int:
        """Bytes one forward call must move at least: Q, K, V read once, O written (all in the
        2-byte input type), fp32 LSE written."""
        q_elems = self.batch * self.heads_q * self.seqlen * self.head_dim
        kv_elems = self.batch * self.heads_kv * self.keys * self.head_dim
        return 2 * (2 * q_elems + 2 * kv_elems) + 4 * self.batch * self.heads_q * self.seqlen


def _varlen_lengths(seed: int, count: int, lo: int, hi: int) -> Tuple[int, ...]:
    rng = np.random.default_rng(seed)
    return tuple(int(x) for x in rng.integers(lo, hi + 1, count))


def _c5() -> Workload:
    lens = _varlen_lengths(5, 16, 512, 8192)
    return Workload("varlen16_h16_d128_causal_bf16", 1, 16, 16, sum(lens), 128, BF16, True, 5,
                    seq_lens=lens)


def _decode_varlen() -> Workload:
    lens_k = _varlen_lengths(8, 32, 256, 16384)
    return Workload("decode_varlen32_hq32_hkv8_d128_bf16", 1, 32, 8, 32, 128, BF16, True, 8,
                    seq_lens=(1,) * 32, seqlen_k=sum(lens_k), seq_lens_k=lens_k, splitkv=True)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("b1_h1_n256_d64_fp16", 1, 1, 1, 256, 64, F16, False, 1),
        Workload("b2_h8_n4096_d64_fp16", 2, 8, 8, 4096, 64, F16, False, 2),
        Workload("b1_h32_n16384_d128_causal_bf16", 1, 32, 32, 16384, 128, BF16, True, 3,
                 qk_multiplier=1.5),
        Workload("gqa_b1_hq32_hkv8_n32768_d128_causal_bf16", 1, 32, 8, 32768, 128, BF16, True, 4),
        _c5(),
        Workload("chunk_b1_hq32_hkv8_q2048_k16384_d128_causal_bf16", 1, 32, 8, 2048, 128, BF16,
                 True, 6, seqlen_k=16384),
        Workload("decode_b16_hq32_hkv8_q1_k16384_d128_bf16", 16, 32, 8, 1, 128, BF16, True, 7,
                 seqlen_k=16384, splitkv=True),
        _decode_varlen(),
    ]
}
WORKLOAD_ORDER: List[str] = list(WORKLOADS)
HEADLINE = "b1_h32_n16384_d128_causal_bf16"


# ----------------------------------------------------------------------------------------
# dtype rounding and decoding (storage formats only)
# ----------------------------------------------------------------------------------------

def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16 or bf16 with round-to-nearest-even; return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        # u + 0x7FFF + lsb only wraps past 2^32 for NaN patterns, which are replaced below
        u = x.view(np.uint32)
        r = (u >> 16) & np.uint32(1)
        r += u
        r += np.uint32(0x7FFF)
        r >>= 16
        out = r.astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            out[nan] = 0x7FC0
        return out
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode fp16 / bf16 bit patterns to float64 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def f64_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact values that are representable in the dtype -> bits (used for hand-built cases)."""
    bits = round_to_bits(np.asarray(x, dtype=np.float32), dtype)
    if not np.array_equal(bits_to_f64(bits, dtype), np.asarray(x, dtype=np.float64)):
        raise ValueError("value not exactly representable in " + dtype)
    return bits


# ----------------------------------------------------------------------------------------
# random tensors
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    """Host bit patterns of Q, K, V ([B, H, N, d] uint16) plus the problem parameters."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    scale: float
    causal: bool
    cu_seqlens: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None  # packed keys, when packed unlike the queries

    @property
    def shape(self) -> Tuple[int, int, int, int, int]:
        b, hq, n, d = self.q.shape
        return b, hq, self.k.shape[1], n, d

    def f64(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        return (bits_to_f64(self.q, self.dtype), bits_to_f64(self.k, self.dtype),
                bits_to_f64(self.v, self.dtype))


def random_inputs(batch: int, heads_q: int, heads_kv: int, seqlen: int, head_dim: int,
                  dtype: str, seed: int, *, causal: bool = False, scale: Optional[float] = None,
                  qk_multiplier: float = 1.0, seq_lens: Optional[Tuple[int, ...]] = None,
                  std: float = 1.0, seqlen_k: Optional[int] = None,
                  seq_lens_k: Optional[Tuple[int, ...]] = None) -> Inputs:
    """Q, K, V ~ N(0, std^2) (Q and K times qk_multiplier) rounded to dtype, from one seed.

    K and V have seqlen_k tokens (default seqlen); packed keys follow seq_lens_k (default
    seq_lens)."""
    rng = np.random.default_rng(seed)
    if seq_lens is not None:
        if batch != 1 or sum(seq_lens) != seqlen:
            raise ValueError("packed sequences need batch == 1 and seqlen == sum(seq_lens)")
    nk = seqlen if seqlen_k is None else seqlen_k
    if seq_lens_k is not None:
        if seq_lens is None or len(seq_lens_k) != len(seq_lens) or sum(seq_lens_k) != nk:
            raise ValueError("seq_lens_k needs seq_lens of the same count and sums to seqlen_k")
    elif seq_lens is not None and nk != seqlen:
        raise ValueError("packed keys of another length need seq_lens_k")
    q = rng.standard_normal((batch, heads_q, seqlen, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, heads_kv, nk, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, heads_kv, nk, head_dim), dtype=np.float32)
    if std != 1.0:
        q *= np.float32(std)
        k *= np.float32(std)
        v *= np.float32(std)
    if qk_multiplier != 1.0:
        q *= np.float32(qk_multiplier)
        k *= np.float32(qk_multiplier)
    cu = cu_k = None
    if seq_lens is not None:
        cu = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int32)
    if seq_lens_k is not None:
        cu_k = np.concatenate([[0], np.cumsum(seq_lens_k)]).astype(np.int32)
    return Inputs(round_to_bits(q, dtype), round_to_bits(k, dtype), round_to_bits(v, dtype),
                  dtype, 1.0 / math.sqrt(head_dim) if scale is None else scale, causal, cu, cu_k)


@dataclasses.dataclass
class Inputs8:
    """E4M3 (OCP) codes of Q, K, V ([B, H, N, d] uint8) with one fp32 descale per (batch, head):
    code value times descale is the tensor the code stands for."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_descale: np.ndarray  # [B, Hq]
    k_descale: np.ndarray  # [B, Hkv]
    v_descale: np.ndarray  # [B, Hkv]
    scale: float
    causal: bool
    cu_seqlens: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None


def quantize_e4m3(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-(batch, head) amax scaling of a float32 [B, H, N, d] tensor to E4M3 codes: descale
    = amax / 448 (1 for an all-zero head), codes = x / descale clamped to +-448 and rounded to
    nearest even (storage conversion through torch's float8_e4m3fn on the CPU)."""
    import torch

    amax = np.abs(x).max(axis=(2, 3)) if x.size else np.zeros(x.shape[:2], np.float32)
    descale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    y = np.clip(x / descale[:, :, None, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), descale


def random_inputs_fp8(batch: int, heads_q: int, heads_kv: int, seqlen: int, head_dim: int,
                      seed: int, *, causal: bool = False, scale: Optional[float] = None,
                      seq_lens: Optional[Tuple[int, ...]] = None, seqlen_k: Optional[int] = None,
                      seq_lens_k: Optional[Tuple[int, ...]] = None) -> Inputs8:
    """Q, K, V ~ N(0, 1) in float32 (the draw order of random_inputs), quantized per
    (batch, head) to E4M3."""
    rng = np.random.default_rng(seed)
    nk = seqlen if seqlen_k is None else seqlen_k
    q = rng.standard_normal((batch, heads_q, seqlen, head_dim), dtype=np.float32)
    k = rng.standard_normal((batch, heads_kv, nk, head_dim), dtype=np.float32)
    v = rng.standard_normal((batch, heads_kv, nk, head_dim), dtype=np.float32)
    (qc, qd), (kc, kd), (vc, vd) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    cu = cu_k = None
    if seq_lens is not None:
        if batch != 1 or sum(seq_lens) != seqlen:
            raise ValueError("packed sequences need batch == 1 and seqlen == sum(seq_lens)")
        cu = np.concatenate([[0], np.cumsum(seq_lens)]).astype(np.int32)
    if seq_lens_k is not None:
        cu_k = np.concatenate([[0], np.cumsum(seq_lens_k)]).astype(np.int32)
    return Inputs8(qc, kc, vc, qd, kd, vd, 1.0 / math.sqrt(head_dim) if scale is None else scale,
                   causal, cu, cu_k)


def random_output_grad(inp: Inputs, seed: int) -> np.ndarray:
    """dL/dO for a backward check: N(0, 1) rounded to the dtype, shaped like Q (bit patterns)."""
    rng = np.random.default_rng(seed)
    return round_to_bits(rng.standard_normal(inp.q.shape, dtype=np.float32), inp.dtype)


def workload_inputs(w: Workload) -> Inputs:
    """The seeded inputs of a named workload (the varlen lengths are part of the workload)."""
    return random_inputs(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim, w.dtype, w.seed,
                         causal=w.causal, scale=w.scale, qk_multiplier=w.qk_multiplier,
                         seq_lens=w.seq_lens, seqlen_k=w.seqlen_k, seq_lens_k=w.seq_lens_k)


# ----------------------------------------------------------------------------------------
# row samples for checks and timing at full size
# ----------------------------------------------------------------------------------------

def sample_rows(w: Workload, fraction: float, seed: int, tile_rows: int = 128,
                max_rows: Optional[int] = None) -> List[Tuple[int, int, int]]:
    """A seeded sample of (batch, q_head, token) rows plus mandatory edge rows.

    Mandatory rows: the first and last token of every sequence, tokens 1 and N-2, and both
    sides of every multiple of tile_rows (capped to at most 64 boundaries, spread evenly),
    each on a seeded head. The token index is global (packed) for varlen workloads.
    """
    rng = np.random.default_rng(seed)
    rows = set()
    if w.seq_lens is not None:
        starts = np.concatenate([[0], np.cumsum(w.seq_lens)[:-1]])
        segments = [(int(s), int(n)) for s, n in zip(starts, w.seq_lens)]
    else:
        segments = [(0, w.seqlen)]
    nb = w.batch
    for b in range(nb):
        for s0, n in segments:
            if n == 0:
                continue
            edge = {0, n - 1, min(1, n - 1), max(n - 2, 0)}
            bounds = list(range(tile_rows, n, tile_rows))
            if len(bounds) > 64:
                idx = np.linspace(0, len(bounds) - 1, 64).round().astype(int)
                bounds = [bounds[i] for i in idx]
            for t in bounds:
                edge.update({t - 1, t})
            for i in edge:
                h = int(rng.integers(0, w.heads_q))
                rows.add((b, h, s0 + i))
            count = int(round(fraction * n * w.heads_q))
            if count:
                hs = rng.integers(0, w.heads_q, count)
                ts = rng.integers(0, n, count)
                rows.update((b, int(h), s0 + int(t)) for h, t in zip(hs, ts))
    out = sorted(rows)
    if max_rows is not None and len(out) > max_rows:
        pick = np.sort(rng.choice(len(out), max_rows, replace=False))
        out = [out[i] for i in pick]
    return out
