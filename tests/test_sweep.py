"""Approximation error of the GPU forward pass against exact softmax attention
(Eq. 1) as the refinement budget P grows, on the refinement-sweep workload
(B1 H16 N16384 on the 128x128 grid, d64, M0 64, C 8, block 128).

This is a report with one property checked: refining more parents brings the
output closer to exact attention (relative RMS error non-increasing in P, with
a small slack).  The exact reference is the oracle's Eq. 1 in double precision
on the same rounded inputs, for two query tiles of every head.
"""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import run_gpu, say

pytestmark = pytest.mark.gpu


def test_error_falls_with_refinement():
    cfg = gen.CONFIGS["sweep"]
    data = gen.make(cfg)
    o = oracle.Oracle.for_cfg(cfg)
    tiles = [(0, cfg.block_q), (cfg.N // 2, cfg.N // 2 + cfg.block_q)]
    exact = [o.exact_attention(data["Q"], data["K"], data["V"], cfg.scale, i0, i1) for i0, i1 in tiles]
    rows = []
    for P in cfg.sweep_P:
        Y = run_gpu(data, P, want_assign=False, want_topp=False, want_importance=False)["Y"]
        diff = np.concatenate([Y[:, i0:i1] - ex for (i0, i1), ex in zip(tiles, exact)], axis=1)
        ref = np.concatenate(exact, axis=1)
        rel_rms = float(np.sqrt((diff ** 2).sum() / (ref ** 2).sum()))
        max_abs = float(np.abs(diff).max())
        rows.append((P, rel_rms, max_abs))
        say(f"[sweep] P={P:3d}  relative RMS error {rel_rms:.4e}  max abs error {max_abs:.4e}  (max|Y| {np.abs(ref).max():.3f})")
    for (p0, e0, _), (p1, e1, _) in zip(rows, rows[1:]):
        assert e1 <= e0 * 1.05, f"error grew from P={p0} ({e0:.3e}) to P={p1} ({e1:.3e})"
