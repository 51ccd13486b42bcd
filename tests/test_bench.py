"""The bench's accounting on the CPU: the algorithmic bytes and flops per
call follow the per-unit formulas (kernel 1: K and V read once, codebooks
once, aggregates written once, 2 d (M0 + C) flops per key; kernel 2: Q read
once, Y written once in fp32, codebooks and aggregates read once,
4 d (M0 + P C) MFMA flops per query), with the 128x128-grid workload's
figures; and the one-GPU contract (a multi-GPU request exits with status 2)."""
import os
import subprocess
import sys

import bench
from adaptive_vector_quantized_amd import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts_grid128():
    cfg = gen.CONFIGS["grid128"]
    alg = bench.algorithmic(cfg, cfg.P)
    BH, N, d, M0, C, Mt = cfg.BH, cfg.N, cfg.d, cfg.M0, cfg.C, cfg.Mt
    k1b, k1f = alg["avq_assign_aggregate"]
    k2b, k2f = alg["avq_attention_fwd"]
    cb = cfg.H * Mt * d * 2
    aggr = BH * Mt * (4 * d + 4)
    assert k1b == 2 * BH * N * d * 2 + cb + aggr
    assert k2b == BH * N * d * 2 + BH * N * d * 4 + cb + aggr
    assert k1f == 2 * d * (M0 + C) * BH * N
    assert k2f == 4 * d * (M0 + cfg.P * C) * BH * N
    # the figures the roofline is quoted with
    assert round(k1b / 1e6, 1) == 140.2 and round(k2b / 1e6, 1) == 207.3
    assert round(k1f / 1e9, 2) == 4.83 and round(k2f / 1e9, 1) == 25.8
    # per query: 49152 MFMA flops at this workload (Tab. 1's O((M0 + P C) d))
    assert k2f / (BH * N) == 49152
    # the call split in two: the preparation moves the value sums (float in,
    # fp16 operands out); the attention kernel reads the operands instead
    pb, pf = alg["avq_attention_prepare"]
    kb, kf = alg["avq_attention_fwd_prepared"]
    assert pb == BH * Mt * d * (4 + 2) and pf == 0
    assert kb == BH * N * d * (2 + 4) + cb + BH * Mt * 4 + BH * Mt * d * 2
    assert kf == k2f
    assert round(kb / 1e6, 1) == 204.9


def test_refinement_budget_enters_kernel2_only():
    cfg = gen.CONFIGS["sweep"]
    a0, a64 = bench.algorithmic(cfg, 0), bench.algorithmic(cfg, 64)
    assert a0["avq_assign_aggregate"] == a64["avq_assign_aggregate"]
    assert a64["avq_attention_fwd"][1] - a0["avq_attention_fwd"][1] == 4 * cfg.d * 64 * cfg.C * cfg.BH * cfg.N
    assert a0["avq_attention_prepare"] == a64["avq_attention_prepare"]
    assert a64["avq_attention_fwd_prepared"][1] == a64["avq_attention_fwd"][1]


def test_multi_gpu_request_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "shard" in r.stderr
    assert r.stdout == ""


def test_metric_is_the_headline():
    assert bench.METRIC.startswith("AVQ fwd Mtokens/s at N=16384,H=16,d=64,M0=64,C=8,P=16")


def test_dominant_kernel_names():
    """The roofline's kernel follows the launcher's choice: the pipelined
    kernel for the bf16 d = 64 shapes with one parent pass and children to
    refine, the general kernel otherwise; large heads get the split maximum
    before the preparation (their traces in profiles/ show the same names)."""
    C = gen.CONFIGS
    assert bench.attention_launches(C["grid128"], 16) == ("attention_prep_kernel", "attention_pipe_kernel")
    assert bench.attention_launches(C["sweep"], 0)[1] == "attention_kernel"
    assert bench.attention_launches(C["sweep"], 64)[1] == "attention_pipe_kernel"
    assert bench.attention_launches(C["grid256"], 32) == ("attention_absmax_kernel + attention_prep_kernel",
                                                          "attention_kernel")
    assert bench.attention_launches(C["flat512"], 0) == ("attention_prep_kernel", "attention_kernel")
    assert bench.attention_launches(C["tiny"], 4)[1] == "attention_kernel"  # fp32
    with open(os.path.join(ROOT, "profiles", "kernels_grid128_stats.txt")) as f:
        assert "attention_pipe_kernel" in f.read()
    with open(os.path.join(ROOT, "profiles", "kernels_grid256_stats.txt")) as f:
        text = f.read()
        assert "attention_absmax_kernel" in text and "avq::attention_kernel<" in text


def test_recorded_bench_lines_parse():
    """Every recorded bench line under profiles/ is one JSON object (the
    line bench.py prints and nothing else) naming its metric, unit, dtype,
    workload and step counts; the headline workload's line also carries the
    roofline and the CPU baseline."""
    import glob
    import json
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))
    assert paths
    for p in paths:
        with open(p) as f:
            lines = [l for l in f.read().splitlines() if l.strip()]
        assert len(lines) == 1, p
        rec = json.loads(lines[0])
        for key in ("metric", "unit", "steps", "warmup", "dtype", "config"):
            assert key in rec, (p, key)
    with open(os.path.join(ROOT, "profiles", "bench_grid128.json")) as f:
        rec = json.load(f)
    assert rec["metric"] == bench.METRIC and rec["n_gpus"] == 1
    assert {"bound", "achieved", "peak", "unit", "frac"} <= set(rec["roofline"])
    assert rec["cpu_baseline"]["kind"] == "oracle"


def test_traced_roofline_record(monkeypatch):
    """The committed record of the dominant call on the headline workload is
    current (taken on the kernel source as it stands) and carries the kernel
    trace's average duration, which the bench line turns into the traced
    roofline fractions beside the live ones; a record of another source is
    not used."""
    cfg = gen.CONFIGS["grid128"]
    rec = bench.load_record("avq_attention_fwd_prepared", "grid128")
    assert rec is not None and rec["trace_avg_us"] > 0
    with open(os.path.join(ROOT, rec["trace_stats"])) as f:
        assert any(rec["kernel"] in l and f"{rec['trace_avg_us']:.3f}" in l for l in f)
    b, fl = bench.algorithmic(cfg, cfg.P)["avq_attention_fwd_prepared"]
    tr = bench.traced_fractions(rec, b, fl, 2500.0)
    assert abs(tr["frac"] - b / (rec["trace_avg_us"] * 1e-6) / 8e12) < 1e-4
    assert abs(tr["mfma_frac"] - fl / (rec["trace_avg_us"] * 1e-6) / 2.5e15) < 1e-4
    assert bench.traced_fractions(None, b, fl, 2500.0) is None
    # once the kernel sources change, the record no longer counts
    monkeypatch.setattr(bench, "source_hash", lambda call: "0" * 16)
    assert bench.load_record("avq_attention_fwd_prepared", "grid128") is None
    assert bench.load_traffic("avq_attention_fwd_prepared", "grid128") is None
