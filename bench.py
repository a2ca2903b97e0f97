#!/usr/bin/env python3
"""Throughput of the exact tiled attention forward pass (libfa) on one MI355X.

One step = one full forward pass (every query block, head and K/V tile) over the workload's
seeded synthetic inputs, already resident in device memory. Prints one JSON line:
TFLOP/s by the convention 4*N^2*d per (batch, head), halved when causal; the fraction of the
MI355X dense MFMA peak of the input type; and the fp64 CPU oracle timed on a bounded, seeded
sample of query rows of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--cpu-seconds S]

The default run (the headline workload) also times, after the headline and outside its timed
region, the forward kernel on the other multi-tile workloads and the headline's backward pass,
reported under "other_configs" (--no-other-configs skips them, as the profiler runs do).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import re
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

import seeded_inputs as si  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of MFMA peak, N=16K d=128 causal bf16"
# MI355X published dense matrix peaks (TFLOP/s), per input type
MFMA_PEAK_TFLOPS = {si.BF16: 2500.0, si.F16: 2500.0, "e4m3": 5000.0}
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
# Transcendental issue ceiling: v_exp_f32 occupies a SIMD's vector ALU for 16 cycles per 64-lane
# instruction (measured with a single-SIMD issue probe), so 256 CUs x 4 SIMDs x 64 / 16 lanes
# per cycle at the 2.4 GHz peak clock.
EXP2_PEAK_PER_S = 256 * 4 * 64 / 16 * 2.4e9
KERNEL_SOURCES = ["exact_tiled_attention_39_amd/csrc/fa_fwd.hip",
                  "exact_tiled_attention_39_amd/csrc/fa_device.h"]
SPLITKV_SOURCES = ["exact_tiled_attention_39_amd/csrc/fa_splitkv.hip",
                   "exact_tiled_attention_39_amd/csrc/fa_device.h"]
FP8_SOURCES = ["exact_tiled_attention_39_amd/csrc/fa_fwd_fp8.hip",
               "exact_tiled_attention_39_amd/csrc/fa_device.h"]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        h.update((ROOT / rel).read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "fa_fwd"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = ROOT / "profiles" / f"{kernel}_{workload}_traffic.md"
    if not path.exists():
        return None
    text = path.read_text()
    src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    sources = {"fa_splitkv": SPLITKV_SOURCES, "fa_fwd_fp8": FP8_SOURCES}.get(kernel, KERNEL_SOURCES)
    if not src or not val or src.group(1) != kernel_source_hash(sources):
        return None
    return float(val.group(1))


def cpu_baseline(w: si.Workload, inp, seconds: float, bytes_metric: bool = False,
                 arrays=None) -> dict:
    """The fp64 oracle, as it stands, on seeded query rows until the time budget is spent.

    Q, K and V are decoded to float64 once, before the clock starts, so the timed region holds
    only the oracle's own work (oracle.attention_rows). The sampled rows are taken head by head
    (32 rows of one head per call, heads in a seeded order), so each call upcasts nothing.
    Reported in TFLOP/s (4*keys*d per row), or with bytes_metric in GB/s: the rows' share of
    the workload's FLOPs times the workload's minimum bytes, per second."""
    import oracle
    from threadpoolctl import threadpool_info

    if arrays is None:
        arrays = tuple(si.bits_to_f64(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in arrays)
    total_rows = w.batch * w.heads_q * w.seqlen
    if total_rows <= 4096:  # few query rows (decode): every row
        rows = [(b, h, t) for b in range(w.batch) for h in range(w.heads_q)
                for t in range(w.seqlen)]
    else:
        rows = si.sample_rows(w, 1 / 4, seed=1234)  # more than the budget: stops at `seconds`
    by_head = {}
    for r in rows:
        by_head.setdefault((r[0], r[1]), []).append(r)
    heads = list(by_head)
    order = np.random.default_rng(99).permutation(len(heads))
    chunks = []
    for i in order:
        hr = by_head[heads[i]]
        chunks += [hr[j:j + 32] for j in range(0, len(hr), 32)]
    cu, cu_k = inp.cu_seqlens, inp.cu_seqlens_k
    starts = cu[:-1] if cu is not None else None

    def row_flops(i):
        if cu is not None:
            s = int(np.searchsorted(starts, i, side="right")) - 1
            while cu[s + 1] <= i:
                s += 1
            s0, s1 = int(cu[s]), int(cu[s + 1])
        else:
            s, s0, s1 = 0, 0, w.seqlen
        if cu is None:
            nk = w.keys
        elif cu_k is not None:
            nk = int(cu_k[s + 1] - cu_k[s])
        else:
            nk = s1 - s0
        shift = nk - (s1 - s0)  # the queries are the last positions of the keys
        keys = min(nk, i - s0 + shift + 1) if w.causal else nk
        return 4.0 * max(keys, 0) * w.head_dim

    done, flops, elapsed = 0, 0.0, 0.0
    for chunk in chunks:
        if elapsed >= seconds:
            break
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, w.scale, w.causal, chunk, cu_seqlens=cu,
                              cu_seqlens_k=cu_k)
        elapsed += time.perf_counter() - t0
        flops += sum(row_flops(i) for _, _, i in chunk)
        done += len(chunk)
    blas = max([p.get("num_threads", 1) for p in threadpool_info()
                if p.get("user_api") == "blas"] or [1])
    if bytes_metric:
        value, unit = flops / w.flops() * w.io_bytes() / elapsed / 1e9, "GB/s"
    else:
        value, unit = flops / elapsed / 1e12, "TFLOP/s"
    return {
        "value": value,
        "unit": unit,
        "cores": len(os.sched_getaffinity(0)),
        "blas_threads": int(blas),
        "kind": "oracle",
        "seconds": round(elapsed, 3),
        "sample_fraction_of_flops": flops / w.flops(),
        # the whole workload through the oracle at the sample's rate (FLOP-weighted rows)
        "extrapolated_full_workload_s": round(elapsed * w.flops() / flops, 1) if flops else None,
        "oracle_gflops_fp64": round(flops / elapsed / 1e9, 3) if elapsed else None,
        "sample": (f"{done} seeded query rows of {total_rows} ({done / total_rows:.2e} of the "
                   f"workload), 32 rows of one head per oracle call, {elapsed:.1f} s of oracle "
                   f"time (inputs decoded to fp64 beforehand, untimed), fp64, "
                   + ("rows weighted by their share of the workload's FLOPs (4*keys*d), "
                      "times its minimum bytes" if bytes_metric else
                      "same FLOP convention per row (4*keys*d)")),
    }


class ClockSampler:
    """Samples the GPU's shader clock (the active level of pp_dpm_sclk) and board power
    (hwmon power1_input) from sysfs every 5 ms while the timed launches run (instantaneous
    readings: a short timed region holds few samples, and its first ones may precede the
    clock's settling under load). Reports null fields where the files are not readable or
    several cards are visible."""

    def __init__(self):
        import glob
        import threading

        self.sclk_files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.power_files = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.mhz, self.watts = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read_mhz(path):
        with open(path) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    return float(m.group(1)) if m else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                if len(self.sclk_files) == 1:
                    v = self._read_mhz(self.sclk_files[0])
                    if v is not None:
                        self.mhz.append(v)
                if len(self.power_files) == 1:
                    with open(self.power_files[0]) as f:
                        self.watts.append(float(f.read().strip()) / 1e6)
            except OSError:
                pass
            self._stop.wait(0.005)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self) -> dict:
        out = {"samples": len(self.mhz), "source": "sysfs pp_dpm_sclk active level, hwmon power1_input"}
        if self.mhz:
            q = np.percentile(self.mhz, [10, 50, 90])
            out["sclk_mhz_p10_p50_p90"] = [round(float(x)) for x in q]
        else:
            out["sclk_mhz_p10_p50_p90"] = None
        out["board_power_w_mean"] = round(float(np.mean(self.watts)), 1) if self.watts else None
        return out


def copy_calibration(torch, mib: int) -> int:
    """A plain copy of a known number of bytes: its FETCH_SIZE / WRITE_SIZE readings per launch
    against mib * 2^20 give the factor that turns those counters into bytes."""
    n = mib * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)
    return 0


def time_calls(torch, step, warmup: int, steps: int):
    """Warm-up calls, then `steps` timed calls: (wall ms per call over the timed region, list
    of per-call HIP-event ms recorded on torch's current stream, where libfa launches). The
    clock and power samples of the timed region are left in time_calls.clocks."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        for a, b in events:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    time_calls.clocks = clocks.summary()
    return (t1 - t0) * 1e3 / steps, [a.elapsed_time(b) for a, b in events]


def launch_percentiles(ms) -> list:
    """p10, median and p90 of the per-launch durations (ms), the spread of the timed launches."""
    q = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return [round(float(x), 4) for x in q]


def rope_tables(positions: int, head_dim: int, base: float = 10000.0):
    """Standard RoPE tables, fp32 [positions, head_dim / 2]: cos and sin of p * base^(-2i/d)."""
    inv = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def bits(t, torch) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_leg(kind: str, w: si.Workload, inp: si.Inputs, gpu: dict, args) -> dict:
    """The CPU baseline (the oracle timed on a bounded sample) and a quick parity check of
    seeded rows of the GPU result against the oracle: the only part of the bench that runs
    the oracle."""
    import oracle
    import oracle.rope

    out = {"cpu_baseline": cpu_baseline(w, inp, args.cpu_seconds, bytes_metric=(kind == "splitkv"))}
    qf, kf, vf = (si.bits_to_f64(x, w.dtype).astype(np.float32) for x in (inp.q, inp.k, inp.v))
    if kind == "backward":
        rows = si.sample_rows(w, 0.0, seed=8, max_rows=32)
        dof = si.bits_to_f64(gpu["dout_bits"], w.dtype).astype(np.float32)
        dq_ref = oracle.attention_backward_dq_rows(qf, kf, vf, dof, w.scale, w.causal, rows,
                                                   cu_seqlens=inp.cu_seqlens)
        idx = tuple(np.array(rows).T)
        dq_gpu = si.bits_to_f64(gpu["dq_bits"][idx], w.dtype)
        out["parity"] = {"dq_rows": len(rows), "max_abs_ddQ": float(np.abs(dq_gpu - dq_ref).max()),
                         "max_abs_dQ_ref": float(np.abs(dq_ref).max())}
        return out
    rows = si.sample_rows(w, 0.0, seed=7, max_rows=48)
    if "rope" in gpu:
        cos, sin, inter = gpu["rope"]
        o_ref, lse_ref = oracle.rope.attention_rope_rows(
            qf, kf, vf, cos, sin, inter, "bf16" if w.dtype == si.BF16 else "f16", w.scale,
            w.causal, rows, cu_seqlens=inp.cu_seqlens, cu_seqlens_k=inp.cu_seqlens_k)
    else:
        o_ref, lse_ref = oracle.attention_rows(qf, kf, vf, w.scale, w.causal, rows,
                                               cu_seqlens=inp.cu_seqlens,
                                               cu_seqlens_k=inp.cu_seqlens_k)
    idx = tuple(np.array(rows).T)
    o_gpu = si.bits_to_f64(gpu["o_bits"][idx], w.dtype)
    lse_gpu = gpu["lse"][idx]
    out["parity"] = {
        "rows": len(rows),
        "max_abs_dO": float(np.abs(o_gpu - o_ref).max()),
        "max_lse_err": float((np.abs(lse_gpu - lse_ref) / np.maximum(np.abs(lse_ref), 1)).max()),
        "max_abs_dO_by_abs_O_ref": band_errors(o_gpu, o_ref, w.dtype),
    }
    return out


# |O_ref| bands for the error breakdown: rounding the output alone costs up to half a unit of
# the output type, so a band's error is read against half a unit at its largest |O_ref|.
BAND_EDGES = [0.5, 1.0, 2.0, 4.0, 8.0]


def band_errors(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str) -> list:
    """Max |dO| and element count per |O_ref| band, with half an output unit at the band's
    largest |O_ref| (significand of 8 bits for bf16, 11 for fp16)."""
    mant = 8 if dtype == si.BF16 else 11
    edges = [0.0] + BAND_EDGES + [np.inf]
    err = np.abs(o_gpu - o_ref).ravel()
    mag = np.abs(o_ref).ravel()
    out = []
    for lo, hi in zip(edges[:-1], edges[1:]):
        sel = (mag >= lo) & (mag < hi)
        if sel.any():
            top = float(mag[sel].max())
            half_unit = float(2.0 ** (np.floor(np.log2(top)) - mant)) if top > 0 else 0.0
            out.append({"band": [lo, hi if np.isfinite(hi) else None], "n": int(sel.sum()),
                        "max_abs_dO": float(err[sel].max()), "half_unit_at_max": half_unit})
    return out


def common_line(args, w: si.Workload, metric: str, value: float, unit: str, ms_per_step: float):
    return {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, see seeded_inputs.py)",
    }


def workload_config(w: si.Workload) -> dict:
    return {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
            "seqlen": w.seqlen, "seqlen_k": w.keys, "head_dim": w.head_dim, "causal": w.causal,
            "num_seqs": len(w.seq_lens) if w.varlen else None}


def kv_stream_bytes(w: si.Workload, block_m: int = 256, block_n: int = 64) -> int:
    """K and V bytes the forward kernel streams from L2/HBM into LDS per launch: every query
    block of every (batch entry or sequence, query head) reads the K and V rows of the key
    tiles it visits (64-key tiles, whole up to the last key; a causal block visits the tiles up
    to its last row, with blocks aligned to the sequence end), each key row d elements of 2
    bytes per tensor."""
    if w.seq_lens is not None:
        pairs = list(zip(w.seq_lens, w.seq_lens_k if w.seq_lens_k is not None else w.seq_lens))
    else:
        pairs = [(w.seqlen, w.keys)] * w.batch
    rows = 0
    for nq, nk in pairs:
        shift = nk - nq
        pad = (-nq) % block_m if w.causal else 0
        for qb in range((nq + block_m - 1) // block_m):
            q0 = block_m * qb - pad
            kv_end = min(nk, q0 + block_m + shift) if w.causal else nk
            if kv_end > 0:  # whole tiles up to kv_end; rows past the last key read nothing
                rows += min((kv_end + block_n - 1) // block_n * block_n, nk)
    return rows * w.heads_q * 2 * w.head_dim * 2


OTHER_FORWARD = ("b2_h8_n4096_d64_fp16", "gqa_b1_hq32_hkv8_n32768_d128_causal_bf16",
                 "varlen16_h16_d128_causal_bf16")


def other_configs(torch, fa, w: si.Workload, inp: si.Inputs, q, k, v, o, lse) -> dict:
    """Kernel time (HIP events, 5 warm-up and 20 timed calls, 100 for a workload of 0.1 ms calls)
    of fa_fwd on the other multi-tile workloads and of fa_bwd on the headline workload, each on
    its own seeded inputs. Informative only: none of it enters `value`."""
    dev = q.device
    out = {}
    for name in OTHER_FORWARD:
        ow = si.WORKLOADS[name]
        oi = si.workload_inputs(ow)
        tdt = torch.bfloat16 if ow.dtype == si.BF16 else torch.float16
        oq, ok, ov = (torch.from_numpy(x.view(np.int16)).view(tdt).to(dev)
                      for x in (oi.q, oi.k, oi.v))
        oo = torch.empty_like(oq)
        ol = torch.empty(oq.shape[:3], dtype=torch.float32, device=dev)
        cu = torch.from_numpy(oi.cu_seqlens).to(dev) if ow.varlen else None
        kw = dict(scale=ow.scale, causal=ow.causal, cu_seqlens=cu,
                  max_seqlen=ow.max_seqlen() if ow.varlen else None)
        timed = 100 if ow.flops() < 1e11 else 20
        _, ms = time_calls(torch, lambda: fa.fa_fwd(oq, ok, ov, oo, ol, **kw), 5, timed)
        avg = float(np.mean(ms))
        tf = ow.flops() / (avg * 1e-3) / 1e12
        out[name] = {"pass": "forward", "timed_calls": timed, "avg_launch_ms": round(avg, 4),
                     "tflops": round(tf, 2),
                     "pct_of_peak": round(100.0 * tf / MFMA_PEAK_TFLOPS[ow.dtype], 2),
                     "launch_ms_p10_p50_p90": launch_percentiles(ms)}
        del oq, ok, ov, oo, ol, oi
        torch.cuda.empty_cache()
    tdt = q.dtype
    do = torch.from_numpy(si.random_output_grad(inp, seed=w.seed + 100).view(np.int16)).view(
        tdt).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((2, *q.shape[:3]), dtype=torch.float32, device=dev)
    _, ms = time_calls(torch, lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta,
                                                scale=w.scale, causal=w.causal), 5, 20)
    avg = float(np.mean(ms))
    tf = 2.5 * w.flops() / (avg * 1e-3) / 1e12
    out[w.name] = {"pass": "backward (delta, dK/dV and dQ kernels; 2.5x the forward's FLOPs)",
                   "timed_calls": 20, "avg_launch_ms": round(avg, 4), "tflops": round(tf, 2),
                   "pct_of_peak": round(100.0 * tf / MFMA_PEAK_TFLOPS[w.dtype], 2),
                   "launch_ms_p10_p50_p90": launch_percentiles(ms)}
    del do, dq, dk, dv, delta
    torch.cuda.empty_cache()
    return out


def bench_forward(args, torch, fa, w: si.Workload, inp: si.Inputs, q, k, v) -> int:
    """fa_fwd over the workload; with --rope, RoPE on Q (as it is loaded) and K (the key pass)."""
    dev = q.device
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if w.varlen else None
    cu_k = torch.from_numpy(inp.cu_seqlens_k).to(dev) if inp.cu_seqlens_k is not None else None
    max_seqlen = w.max_seqlen() if w.varlen else None
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kw = dict(scale=w.scale, causal=w.causal, cu_seqlens=cu, max_seqlen=max_seqlen,
              cu_seqlens_k=cu_k)
    gpu = {}
    if args.rope:
        cos, sin = rope_tables(max(w.keys, 1), w.head_dim)
        gpu["rope"] = (cos, sin, False)
        kw.update(rope_cos=torch.from_numpy(cos).to(dev), rope_sin=torch.from_numpy(sin).to(dev))
        k_rot = torch.empty_like(k)

        def step():
            fa.fa_fwd(q, k, v, o, lse, k_rot=k_rot, **kw)

        def kernel_only():  # the attention kernel alone: keys already rotated, Q rotated on load
            fa.fa_fwd(q, k_rot, v, o, lse, **kw)
    else:
        def step():
            fa.fa_fwd(q, k, v, o, lse, **kw)
        kernel_only = step

    ms_per_step, launch_ms = time_calls(torch, step, args.warmup, args.steps)
    if kernel_only is not step:
        _, kernel_ms = time_calls(torch, kernel_only, 3, args.steps)
        step()  # leaves o, lse from the full call
        torch.cuda.synchronize()
    else:
        kernel_ms = launch_ms
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_kernel_ms = float(np.mean(kernel_ms))
    achieved = flops / (avg_kernel_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    metric = METRIC if (w.name == si.HEADLINE and not args.rope) else (
        f"attention fwd TFLOP/s and % of MFMA peak, {w.name}" + (" + RoPE" if args.rope else ""))
    line = common_line(args, w, metric, round(value, 2), "TFLOP/s", ms_per_step)
    line["config"] = {**workload_config(w), "flop_count": flops,
                      "flop_convention": ("4*N^2*d per (batch, head), halved for causal"
                                          if w.seqlen_k is None else
                                          "4*Nq*Nk*d per (batch, head), less 2*Nq^2*d for causal")}
    if args.rope:
        line["config"]["rope"] = ("half-split pairs, standard tables; K rotated by the key pass, "
                                  "Q as it is loaded")
    line["pct_of_peak"] = round(100.0 * value / peak, 2)
    line["roofline"] = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": None if args.rope else measured_traffic(w.name),
        "kernel": "fa_fwd_kernel",
        "avg_launch_ms": round(avg_kernel_ms, 4),
        "launch_ms_min_max": [round(min(kernel_ms), 4), round(max(kernel_ms), 4)],
        "launch_ms_p10_p50_p90": launch_percentiles(kernel_ms),
    }
    if args.rope:
        line["roofline"]["avg_call_ms_with_key_pass"] = round(float(np.mean(launch_ms)), 4)
    # secondary bound: one exponential per visible score (flops / (4 d) by the convention)
    exps = flops / (4.0 * w.head_dim)
    line["exp2_bound"] = {
        "exps_per_launch": exps,
        "achieved_per_s": exps / (avg_kernel_ms * 1e-3),
        "peak_per_s": EXP2_PEAK_PER_S,
        "frac": round(exps / (avg_kernel_ms * 1e-3) / EXP2_PEAK_PER_S, 4),
        "note": "v_exp_f32 issue ceiling; the kernel also issues about 3 full-rate VALU "
                "instructions per score (scale-and-shift FMA, row sums, conversion to the input type)",
    }
    # secondary volume: K/V rows streamed into LDS (re-read per query block and query head),
    # served by L2 and the last-level cache; roofline.traffic is what reached HBM
    kv = kv_stream_bytes(w)
    traffic = line["roofline"]["traffic"]
    line["kv_stream"] = {
        "bytes_per_launch": kv,
        "achieved_GBps": round(kv / (avg_kernel_ms * 1e-3) / 1e9, 1),
        "hbm_bytes_over_stream_bytes": round(traffic / kv, 4) if traffic else None,
        "note": "K and V tiles read into LDS by every 256-query block of every query head; "
                "they come from L2 or the last-level cache, and the HBM traffic is a fraction of them",
    }
    line["gpu_clocks"] = time_calls.clocks
    line["kernel_source_sha256"] = kernel_source_hash()
    if not args.no_cpu_baseline:
        gpu.update(o_bits=bits(o, torch), lse=lse.cpu().numpy().astype(np.float64))
    if w.name == si.HEADLINE and not args.rope and not args.no_other_configs:
        line["other_configs"] = other_configs(torch, fa, w, inp, q, k, v, o, lse)
    if not args.no_cpu_baseline:
        line.update(oracle_leg("forward", w, inp, gpu, args))
    print(json.dumps(line), flush=True)
    return 0


def bench_fp8(args, torch, fa, w: si.Workload) -> int:
    """fa_fwd on E4M3 inputs of the workload's shape (per-head amax scaling of the same seeded
    N(0, 1) draws), bfloat16 output."""
    inp = si.random_inputs_fp8(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim, w.seed,
                               causal=w.causal, scale=w.scale, seq_lens=w.seq_lens,
                               seqlen_k=w.seqlen_k, seq_lens_k=w.seq_lens_k)
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    qd, kd, vd = up(inp.q_descale), up(inp.k_descale), up(inp.v_descale)
    cu = up(inp.cu_seqlens) if inp.cu_seqlens is not None else None
    cu_k = up(inp.cu_seqlens_k) if inp.cu_seqlens_k is not None else None
    max_seqlen = w.max_seqlen() if w.varlen else None
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale=w.scale, causal=w.causal, cu_seqlens=cu,
                  max_seqlen=max_seqlen, cu_seqlens_k=cu_k, q_descale=qd, k_descale=kd,
                  v_descale=vd)

    ms_per_step, launch_ms = time_calls(torch, step, args.warmup, args.steps)
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_ms = float(np.mean(launch_ms))
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS["e4m3"]
    line = common_line(args, w, f"attention fwd TFLOP/s and % of MFMA peak, {w.name} in FP8 E4M3",
                       round(value, 2), "TFLOP/s", ms_per_step)
    line["dtype"] = "e4m3"
    line["data"] = ("synthetic (the workload's seeded N(0,1) draws, per-(batch, head) amax "
                    "scaled to E4M3, see seeded_inputs.py)")
    line["config"] = {**workload_config(w), "flop_count": flops, "output": "bf16",
                      "flop_convention": "the bf16 workload's convention"}
    line["pct_of_peak"] = round(100.0 * value / peak, 2)
    line["roofline"] = {
        "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name, "fa_fwd_fp8"),
        "kernel": "fa_fwd_fp8_kernel",
        "avg_launch_ms": round(avg_ms, 4),
        "launch_ms_min_max": [round(min(launch_ms), 4), round(max(launch_ms), 4)],
        "launch_ms_p10_p50_p90": launch_percentiles(launch_ms),
    }
    line["gpu_clocks"] = time_calls.clocks
    line["kernel_source_sha256"] = kernel_source_hash(FP8_SOURCES)
    if not args.no_cpu_baseline:
        import oracle
        import oracle.fp8

        arrays = tuple(oracle.fp8.dequantize(c, d).astype(np.float32) for c, d in
                       ((inp.q, inp.q_descale), (inp.k, inp.k_descale), (inp.v, inp.v_descale)))
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, arrays=arrays)
        rows = si.sample_rows(w, 0.0, seed=7, max_rows=48)
        o_ref, lse_ref = oracle.attention_rows(*arrays, w.scale, w.causal, rows,
                                               cu_seqlens=inp.cu_seqlens,
                                               cu_seqlens_k=inp.cu_seqlens_k)
        idx = tuple(np.array(rows).T)
        o_gpu = si.bits_to_f64(bits(o, torch)[idx], si.BF16)
        lse_gpu = lse.cpu().numpy().astype(np.float64)[idx]
        line["parity"] = {
            "rows": len(rows), "max_abs_dO": float(np.abs(o_gpu - o_ref).max()),
            "o_tolerance": oracle.fp8.o_tolerance(arrays[2], w.keys),
            "max_lse_err": float((np.abs(lse_gpu - lse_ref)
                                  / np.maximum(np.abs(lse_ref), 1)).max())}
    print(json.dumps(line), flush=True)
    return 0


def bench_backward(args, torch, fa, w: si.Workload, inp: si.Inputs, q, k, v, up) -> int:
    """The backward pass (delta, dK/dV and dQ kernels) of a self-attention workload."""
    if w.seqlen_k is not None:
        print("the backward pass covers self-attention workloads only", file=sys.stderr)
        return 2
    dev = q.device
    dout_bits = si.random_output_grad(inp, seed=w.seed + 100)
    do = up(dout_bits)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if w.varlen else None
    max_seqlen = w.max_seqlen() if w.varlen else None
    o, lse = fa.attention(q, k, v, scale=w.scale, causal=w.causal, cu_seqlens=cu,
                          max_seqlen=max_seqlen)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((2, *q.shape[:3]), dtype=torch.float32, device=dev)

    def step():
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, scale=w.scale, causal=w.causal,
                  cu_seqlens=cu, max_seqlen=max_seqlen)

    ms_per_step, launch_ms = time_calls(torch, step, args.warmup, args.steps)
    flops = 2.5 * w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    avg_ms = float(np.mean(launch_ms))
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    line = common_line(args, w, f"attention bwd TFLOP/s and % of MFMA peak, {w.name}",
                       round(value, 2), "TFLOP/s", ms_per_step)
    line["data"] = "synthetic (seeded N(0,1) inputs and output gradient, see seeded_inputs.py)"
    line["config"] = {**workload_config(w), "flop_count": flops,
                      "flop_convention": ("2.5 x the forward's convention: 5 products (S, dP, dV, "
                                          "dK, dQ); the kernels run 7 (S and dP again for dQ)")}
    line["pct_of_peak"] = round(100.0 * value / peak, 2)
    line["roofline"] = {
        "bound": "mfma",
        "achieved": round(flops / (avg_ms * 1e-3) / 1e12, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(flops / (avg_ms * 1e-3) / 1e12 / peak, 4),
        "traffic": None,
        "kernel": "fa_bwd (fa_bwd_delta_kernel, fa_bwd_dkdv_kernel, fa_bwd_dq_kernel)",
        "avg_launch_ms": round(avg_ms, 4),
        "launch_ms_min_max": [round(min(launch_ms), 4), round(max(launch_ms), 4)],
        "launch_ms_p10_p50_p90": launch_percentiles(launch_ms),
    }
    line["gpu_clocks"] = time_calls.clocks
    if not args.no_cpu_baseline:
        line.update(oracle_leg("backward", w, inp, {"dout_bits": dout_bits,
                                                    "dq_bits": bits(dq, torch)}, args))
    print(json.dumps(line), flush=True)
    return 0


def bench_splitkv(args, torch, fa, w: si.Workload, inp: si.Inputs, q, k, v) -> int:
    """The split-KV forward (split and merge kernels) of a decode workload, in GB/s of the
    bytes it must move."""
    dev = q.device
    cu = torch.from_numpy(inp.cu_seqlens).to(dev) if w.varlen else None
    cu_k = torch.from_numpy(inp.cu_seqlens_k).to(dev) if inp.cu_seqlens_k is not None else None
    max_seqlen = w.max_seqlen() if w.varlen else None
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    params = fa.make_params(q, k, v, o, lse, w.scale, w.causal, cu, max_seqlen, cu_k)
    splits, ws_bytes = fa.fa_splitkv_plan(params, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        fa.fa_fwd_splitkv(q, k, v, o, lse, ws, scale=w.scale, causal=w.causal, num_splits=0,
                          cu_seqlens=cu, max_seqlen=max_seqlen, cu_seqlens_k=cu_k)

    ms_per_step, launch_ms = time_calls(torch, step, args.warmup, args.steps)
    nbytes = w.io_bytes()
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    avg_ms = float(np.mean(launch_ms))
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    line = common_line(args, w, f"attention decode GB/s (Q, K, V read, O, LSE written), {w.name}",
                       round(value, 1), "GB/s", ms_per_step)
    line["config"] = {**workload_config(w), "splits": splits, "workspace_bytes": ws_bytes,
                      "io_bytes": nbytes}
    line["roofline"] = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": measured_traffic(w.name, "fa_splitkv"),
        "kernel": "fa_fwd_splitkv (fa_splitkv_kernel + fa_splitkv_merge_kernel)",
        "avg_launch_ms": round(avg_ms, 4),
        "launch_ms_min_max": [round(min(launch_ms), 4), round(max(launch_ms), 4)],
        "launch_ms_p10_p50_p90": launch_percentiles(launch_ms),
    }
    line["gpu_clocks"] = time_calls.clocks
    line["kernel_source_sha256"] = kernel_source_hash(SPLITKV_SOURCES)
    if not args.no_cpu_baseline:
        line.update(oracle_leg("splitkv", w, inp, {"o_bits": bits(o, torch),
                                                   "lse": lse.cpu().numpy().astype(np.float64)},
                               args))
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=si.HEADLINE, choices=si.WORKLOAD_ORDER)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rope", action="store_true",
                    help="forward with rotary position embedding (standard tables, half-split "
                         "pairs): Q rotated as it is loaded, K by the key pass")
    ap.add_argument("--fp8", action="store_true",
                    help="forward on E4M3 (FP8) inputs of the workload's shape")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fa_bwd) of the workload instead of the forward")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the informative timings of the other workloads and of the "
                         "backward pass that follow the headline forward")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 launches), the "
                         "known-size reference that scales the HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: libfa has no multi-GPU path (heads would shard "
              "across GPUs with no communication between them)", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration_mib:
        return copy_calibration(torch, args.copy_calibration_mib)

    import exact_tiled_attention_39_amd as fa

    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = si.WORKLOADS[args.workload]
    if args.fp8:
        return bench_fp8(args, torch, fa, w)
    inp = si.workload_inputs(w)
    tdt = torch.bfloat16 if w.dtype == si.BF16 else torch.float16

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(tdt).to(dev)

    q, k, v = up(inp.q), up(inp.k), up(inp.v)
    if args.backward:
        return bench_backward(args, torch, fa, w, inp, q, k, v, up)
    if w.splitkv:
        return bench_splitkv(args, torch, fa, w, inp, q, k, v)
    return bench_forward(args, torch, fa, w, inp, q, k, v)


if __name__ == "__main__":
    sys.exit(main())
