"""The bench's one-line JSON contract: every key a bench line must carry, their types and the
relations between them, and the refusal of more than one GPU (the library measures one)."""
from __future__ import annotations

import json
import pathlib
import subprocess
import sys

import pytest

import seeded_inputs as si

ROOT = pathlib.Path(__file__).resolve().parents[1]
BENCH = str(ROOT / "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_kv_stream_bytes_closed_forms():
    """The K/V volume streamed into LDS, against closed forms of the 256 x 64 tiling."""
    import bench
    tile = 64 * 2 * 2  # one key row of K and V per head-dim element: 64 rows x 2 tensors x 2 B
    # causal 16K, 32 heads: block b (256 queries) visits 4 (b + 1) tiles of 64 keys
    w = si.WORKLOADS[si.HEADLINE]
    assert bench.kv_stream_bytes(w) == 32 * sum(4 * (b + 1) for b in range(64)) * tile * 128
    # non-causal: every block of every head reads all keys
    w = si.WORKLOADS["b2_h8_n4096_d64_fp16"]
    assert bench.kv_stream_bytes(w) == 2 * 8 * 16 * 4096 * 64 * 2 * 2
    # GQA: the K/V of a kv head are read once per query head that shares it
    w = si.WORKLOADS["gqa_b1_hq32_hkv8_n32768_d128_causal_bf16"]
    assert bench.kv_stream_bytes(w) == 32 * sum(4 * (b + 1) for b in range(128)) * tile * 128
    # a 2K query chunk at the end of 16K keys: block b visits the 14336 earlier keys plus its own
    w = si.WORKLOADS["chunk_b1_hq32_hkv8_q2048_k16384_d128_causal_bf16"]
    assert bench.kv_stream_bytes(w) == 32 * sum(14336 + 256 * (b + 1) for b in range(8)) * 128 * 4
    # a causal sequence of 300 tokens: blocks aligned to its end (pad 212), so block 0 covers
    # rows -212..43 (one tile) and block 1 rows 44..299 (all 300 keys, five tiles clamped at 300)
    w = si.Workload(name="t", batch=1, heads_q=1, heads_kv=1, seqlen=300, head_dim=64,
                    causal=True, dtype=si.F16, seed=0)
    assert bench.kv_stream_bytes(w) == (64 + 300) * 64 * 2 * 2


@pytest.mark.gpu
def test_headline_bench_line_carries_the_contract():
    print("bench.py --steps 3 --warmup 1 --cpu-seconds 1 (headline workload)", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1",
                        "--cpu-seconds", "1"], capture_output=True, text=True, timeout=600,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    line = json.loads(lines[0])

    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                     ("steps", int), ("warmup", int), ("ms_per_step", float),
                     ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)]:
        assert isinstance(line[key], typ), key
    assert "vs_baseline" in line and line["vs_baseline"] is None
    assert line["unit"] == "TFLOP/s" and line["higher_is_better"] is True
    assert (line["n_gpus"], line["steps"], line["warmup"]) == (1, 3, 1)
    assert line["scaling"] == "weak" and line["dtype"] == si.BF16
    assert line["config"]["workload"] == si.HEADLINE
    # value is the workload's FLOPs over the wall time of one step
    flop = line["config"]["flop_count"]
    assert flop == 32 * 4 * 16384 ** 2 * 128 / 2
    assert line["value"] == pytest.approx(flop / (line["ms_per_step"] * 1e-3) / 1e12, rel=2e-3)

    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert 0.0 < roof["achieved"] < roof["peak"]
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-3)
    assert roof["traffic"] is None or roof["traffic"] > 0
    lo, hi = roof["launch_ms_min_max"]
    p10, p50, p90 = roof["launch_ms_p10_p50_p90"]
    assert lo <= p10 <= p50 <= p90 <= hi

    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "TFLOP/s"
    assert cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]

    assert cpu["blas_threads"] >= 1
    # the extrapolation to the whole workload is the sample's time over its share of the FLOPs
    assert 0.0 < cpu["sample_fraction_of_flops"] <= 1.0
    assert cpu["extrapolated_full_workload_s"] == pytest.approx(
        cpu["seconds"] / cpu["sample_fraction_of_flops"], rel=2e-2)
    assert cpu["oracle_gflops_fp64"] == pytest.approx(cpu["value"] * 1e3, rel=2e-2)

    par = line["parity"]
    assert par["max_abs_dO"] <= 1.6e-2 and par["max_lse_err"] <= 1e-5
    bands = par["max_abs_dO_by_abs_O_ref"]
    assert sum(b["n"] for b in bands) == par["rows"] * 128
    assert max(b["max_abs_dO"] for b in bands) == pytest.approx(par["max_abs_dO"])

    ex = line["exp2_bound"]
    assert ex["exps_per_launch"] == flop / (4 * 128)
    assert 0.0 < ex["frac"] < 1.0
    # avg_launch_ms is rounded to 1e-4 ms in the line
    assert ex["achieved_per_s"] == pytest.approx(ex["exps_per_launch"] / (roof["avg_launch_ms"] * 1e-3),
                                                 rel=1e-3)
    assert "gpu_clocks" in line and "samples" in line["gpu_clocks"]
    kv = line["kv_stream"]
    assert kv["bytes_per_launch"] == 32 * sum(4 * (b + 1) for b in range(64)) * 64 * 4 * 128
    assert kv["achieved_GBps"] == pytest.approx(
        kv["bytes_per_launch"] / (roof["avg_launch_ms"] * 1e-3) / 1e9, rel=1e-3)

    # the informative timings that follow the headline: the other multi-tile forward workloads
    # and the headline's backward, none of them part of `value`
    other = line["other_configs"]
    assert set(other) == {"b2_h8_n4096_d64_fp16", "gqa_b1_hq32_hkv8_n32768_d128_causal_bf16",
                          "varlen16_h16_d128_causal_bf16", si.HEADLINE}
    assert other[si.HEADLINE]["pass"].startswith("backward")
    for name, o in other.items():
        assert 0.0 < o["tflops"] < 2500.0, name
        assert o["pct_of_peak"] == pytest.approx(100.0 * o["tflops"] / 2500.0, abs=0.02), name
        w = si.WORKLOADS[name]
        mult = 2.5 if name == si.HEADLINE else 1.0
        assert o["tflops"] == pytest.approx(mult * w.flops() / (o["avg_launch_ms"] * 1e-3) / 1e12,
                                            rel=2e-3), name
