"""Selection quality of the approximate tiled denominator (App. B, the
synthetic analogue of Tab. 5): the fraction of the true attention mass that
falls on the keys of the P parents each selection picks.

True mass of parent p for a query tile I: the mean over the queries of I of
the exact softmax weights (Eq. 1) summed over the keys assigned to p.  The
queries are the keys themselves (self-attention over the 64x64 token grid with
8x8-patch clusters), so that the attention of a tile concentrates on a few
clusters, as in the pages' image workloads.  Three
selections, all from the oracle: exact (the P parents of largest true mass --
the best any P-set can do), non-tiled (Eq. 7 importance with the exact
denominator) and tiled (Eq. 13-14 with tiles of 64 parents).  CPU only.
"""
import numpy as np

import pytest

import oracle
from adaptive_vector_quantized_amd import gen, gilbert


def _capture(mass, sel):
    return np.take_along_axis(mass, sel.astype(np.int64), axis=-1).sum(-1)


def test_tiled_selection_capture():
    cfg = gen.CONFIGS["grid64"].replace(M0=256, H=2, dtype="f32")
    data = gen.make(cfg)
    data["Q"] = data["K"]
    o = oracle.Oracle.for_cfg(cfg)
    parent, _ = o.assign(data["K"], data["codebook"])
    _, counts = o.aggregate(data["V"], parent, parent)
    Q, K = data["Q"].astype(np.float64), data["K"].astype(np.float64)
    bq, T = cfg.block_q, cfg.N // cfg.block_q
    mass = np.zeros((cfg.BH, T, cfg.M0))
    for bh in range(cfg.BH):
        S = cfg.scale * Q[bh] @ K[bh].T
        A = np.exp(S - S.max(axis=1, keepdims=True))
        A /= A.sum(axis=1, keepdims=True)
        onehot = np.zeros((cfg.N, cfg.M0))
        onehot[np.arange(cfg.N), parent[bh]] = 1.0
        per_parent = A @ onehot                      # [N queries, M0]
        mass[bh] = per_parent.reshape(T, bq, cfg.M0).mean(axis=1)
    w = o.importance(data["Q"], data["codebook"], counts, bq, cfg.scale)
    wt = o.importance_tiled_f64(data["Q"], data["codebook"], counts, bq, cfg.scale, 64)
    for P in (4, 8, 16, 32):
        caps = {
            "exact": _capture(mass, o.select(mass, P)),
            "non-tiled": _capture(mass, o.select(w, P)),
            "tiled (64)": _capture(mass, o.select(wt, P)),
        }
        print(f"[capture] M0 {cfg.M0} P {P:2d}: " +
              "  ".join(f"{k} {v.mean() * 100:6.2f}%" for k, v in caps.items()))
        assert np.all(caps["exact"] >= caps["non-tiled"] - 1e-9)
        assert np.all(caps["exact"] >= caps["tiled (64)"] - 1e-9)
        # the extrapolated denominator keeps most of what the exact one captures
        assert caps["tiled (64)"].mean() >= 0.9 * caps["non-tiled"].mean()


def _per_query_mass(cfg, data, o):
    """Exact softmax weights (Eq. 1) of every query summed over the keys of
    each parent: [BH, N, M0]; also the parent of every key and the counts."""
    parent, _ = o.assign(data["K"], data["codebook"])
    _, counts = o.aggregate(data["V"], parent, parent)
    Q, K = data["Q"].astype(np.float64), data["K"].astype(np.float64)
    per = np.zeros((cfg.BH, cfg.N, cfg.M0))
    for bh in range(cfg.BH):
        S = cfg.scale * Q[bh] @ K[bh].T
        A = np.exp(S - S.max(axis=1, keepdims=True))
        A /= A.sum(axis=1, keepdims=True)
        onehot = np.zeros((cfg.N, cfg.M0))
        onehot[np.arange(cfg.N), parent[bh]] = 1.0
        per[bh] = A @ onehot
    return per, counts


@pytest.mark.parametrize("grid,patch", [(64, 8), (60, 6), (30, 5)])
def test_query_order_capture(grid, patch):
    """Query order and selection quality (the synthetic analogue of Tab. 8):
    capture, the mean over queries of the exact attention mass on the keys of
    the P parents their tile selects (Eq. 7 importance), with the tiles taken
    along the Gilbert curve, in raster order and in a random order, for tiles
    of 32, 64 and 128 queries.  Self-attention over a grid of patch clusters
    (M0 = 64, C = 8; the 60x60 and 30x30 grids have patches that do not line up
    with the curve's power-of-two blocks).  Curve tiles are compact regions
    and keep up with or beat raster strips; a random order spreads every tile
    over the whole image and loses most of the mass at small P."""
    cfg = gen.CONFIGS["grid64"].replace(N=grid * grid, grid=grid, patch=patch, H=2, dtype="f32")
    data = gen.make(cfg)
    data["Q"] = data["K"]
    o = oracle.Oracle.for_cfg(cfg)
    per, counts = _per_query_mass(cfg, data, o)
    orders = {"gilbert": gilbert.query_order(grid, grid), "raster": np.arange(cfg.N, dtype=np.int32),
              "random": np.random.default_rng(5).permutation(cfg.N).astype(np.int32)}
    for bq in (32, 64, 128):
        for P in (4, 8, 16):
            cap = {}
            for name, order in orders.items():
                oq, Qo, rows = o.ordered(data["Q"], order)
                sel = oq.select(oq.importance(Qo, data["codebook"], counts, bq, cfg.scale), P)
                got = [per[bh][np.ix_(rows[t * bq:(t + 1) * bq], sel[bh, t])].sum(1)
                       for bh in range(cfg.BH) for t in range(sel.shape[1])]
                cap[name] = float(np.concatenate(got).mean())
            print(f"[capture] grid {grid} patch {patch} tile {bq:3d} P {P:2d}: " +
                  "  ".join(f"{k} {v * 100:6.2f}%" for k, v in cap.items()))
            assert cap["gilbert"] >= cap["raster"] - 1e-3
            assert cap["random"] < cap["raster"] - 0.05
        assert cap["gilbert"] > 0.98  # P = 16: nearly all of the mass
