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


def test_refinement_budget_enters_kernel2_only():
    cfg = gen.CONFIGS["sweep"]
    a0, a64 = bench.algorithmic(cfg, 0), bench.algorithmic(cfg, 64)
    assert a0["avq_assign_aggregate"] == a64["avq_assign_aggregate"]
    assert a64["avq_attention_fwd"][1] - a0["avq_attention_fwd"][1] == 4 * cfg.d * 64 * cfg.C * cfg.BH * cfg.N


def test_multi_gpu_request_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "shard" in r.stderr
    assert r.stdout == ""


def test_metric_is_the_headline():
    assert bench.METRIC.startswith("AVQ fwd Mtokens/s at N=16384,H=16,d=64,M0=64,C=8,P=16")
