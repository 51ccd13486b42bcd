"""Seeded synthetic inputs for the AVQ-Attention forward pass.

This module draws data and performs none of the method's steps.  It builds the
per-head hierarchical codebooks, keys from a spatially smooth cluster mixture,
queries and values, with the shapes and structure of the image-token workloads
the paper times (ViT / DPT / SD1.5 token grids; Sec. 5, Sec. E, Tab. 2).

Construction:

* Codebook, per head (Sec. 4.1 and Eq. 5: each parent equals the mean of its
  children).  Draw p0 ~ N(0, I) and raw children r_c = p0 + 0.3 N(0, I).  Put
  the first C-1 children and the parent mean(r) on the dyadic grid 2^-6, then
  set the last child to C*parent - (sum of the others), which stays on the
  grid.  Redraw a parent block if any entry reaches |x| >= 4.  Every entry is
  then k/64 with |k| < 256, exact in bf16 and fp32, and the mean constraint
  holds exactly in any binary floating point format.
* Cluster ids: a (parent, slot) pair, slot uniform over {parent, child 0 ..
  child C-1}; the parent is uniform or Zipf-weighted, (j+1)^-s.  With a token
  grid, one id per 8x8 patch of the row-major grid; without, one id per key.
* Keys: codeword of the cluster id + N(0, 0.1^2) noise.  Queries, values:
  N(0, 1).  Everything is rounded to the workload dtype (round to nearest
  even), stored as float32 arrays whose values are exact in that dtype.

Optional ``checker`` (the tests pass one built on the oracle): the generator
asks it how far each key's assignment and each query tile's top-P choice is
from a tie and redraws the key noise / the tile's queries until the margin is
at least ``margin``.  The generator itself never evaluates those quantities.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

GRID_STEP = 1.0 / 64.0
CODEBOOK_BOUND = 4.0

# sub-stream role ids for SeedSequence spawn keys
_ROLE_CODEBOOK, _ROLE_IDS, _ROLE_KEYS, _ROLE_VALUES, _ROLE_QUERIES, _ROLE_REDRAW_K, _ROLE_REDRAW_Q = range(7)


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  ``P`` may be a tuple for a refinement sweep."""

    name: str
    B: int
    H: int
    N: int
    d: int
    M0: int
    C: int
    P: int
    block_q: int
    dtype: str  # "f32" or "bf16"
    grid: Optional[int]  # side of the square token grid (row-major), None = no spatial structure
    parents: str  # "uniform" or "zipf"
    seed: int
    zipf_s: float = 1.2
    patch: int = 8
    sweep_P: Sequence[int] = ()

    @property
    def Mt(self) -> int:
        return self.M0 * (1 + self.C)

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def tiles(self) -> int:
        return (self.N + self.block_q - 1) // self.block_q

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # tiny single head, fp32, one cluster draw per key
    "tiny": Config("tiny", B=1, H=1, N=1024, d=64, M0=16, C=4, P=4, block_q=64,
                   dtype="f32", grid=None, parents="uniform", seed=1000),
    # M0=64, C=8, P=16 on a 64x64 token grid (SD1.5 level-0 self-attention size)
    "grid64": Config("grid64", B=1, H=12, N=4096, d=64, M0=64, C=8, P=16, block_q=64,
                     dtype="bf16", grid=64, parents="uniform", seed=1001),
    # the headline workload: 128x128 grid, 16 heads, batch 2, Zipf occupancy
    "grid128": Config("grid128", B=2, H=16, N=16384, d=64, M0=64, C=8, P=16, block_q=128,
                      dtype="bf16", grid=128, parents="zipf", seed=1002),
    # large parent codebook at d=128 on a 256x256 grid
    "grid256": Config("grid256", B=1, H=8, N=65536, d=128, M0=256, C=8, P=32, block_q=128,
                      dtype="bf16", grid=256, parents="zipf", seed=1003),
    # flat codebook of 256 codewords (no children, plain VQ attention) at the headline shape
    "flat256": Config("flat256", B=2, H=16, N=16384, d=64, M0=256, C=0, P=0, block_q=128,
                      dtype="bf16", grid=128, parents="zipf", seed=1005),
    # flat codebook of 512 codewords at the headline shape (Tab. 2's largest flat VQ row)
    "flat512": Config("flat512", B=2, H=16, N=16384, d=64, M0=512, C=0, P=0, block_q=128,
                      dtype="bf16", grid=128, parents="zipf", seed=1006),
    # refinement-budget sweep on the 128x128 grid, one batch
    "sweep": Config("sweep", B=1, H=16, N=16384, d=64, M0=64, C=8, P=16, block_q=128,
                    dtype="bf16", grid=128, parents="zipf", seed=1004, sweep_P=(0, 4, 16, 64)),
}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the workload dtype; returns float32 holding exactly representable values."""
    f = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return f
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype}")
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key))))


def _snap(x: np.ndarray) -> np.ndarray:
    return np.round(x / GRID_STEP) * GRID_STEP


def make_codebook(seed: int, H: int, M0: int, C: int, d: int, child_sigma: float = 0.3) -> np.ndarray:
    """Per-head codebook [H, M0*(1+C), d] (float32, entries k/64, |k| < 256)."""
    Mt = M0 * (1 + C)
    cb = np.zeros((H, Mt, d), dtype=np.float64)
    for h in range(H):
        rng = _rng(seed, _ROLE_CODEBOOK, h)
        for m in range(M0):
            while True:
                p0 = rng.standard_normal(d)
                if C == 0:
                    parent = _snap(p0)
                    kids = np.zeros((0, d))
                else:
                    raw = p0[None, :] + child_sigma * rng.standard_normal((C, d))
                    parent = _snap(raw.mean(axis=0))
                    kids = _snap(raw)
                    kids[C - 1] = C * parent - kids[: C - 1].sum(axis=0)
                if np.all(np.abs(parent) < CODEBOOK_BOUND) and np.all(np.abs(kids) < CODEBOOK_BOUND):
                    break
            cb[h, m] = parent
            if C:
                cb[h, M0 + m * C: M0 + (m + 1) * C] = kids
    return cb.astype(np.float32)


def _cluster_rows(cfg: Config, bh: int) -> np.ndarray:
    """Generating codeword row of every token of one (batch, head)."""
    rng = _rng(cfg.seed, _ROLE_IDS, bh)
    M0, C = cfg.M0, cfg.C
    if cfg.parents == "uniform":
        pw = np.full(M0, 1.0 / M0)
    elif cfg.parents == "zipf":
        pw = (np.arange(M0) + 1.0) ** (-cfg.zipf_s)
        pw /= pw.sum()
    else:
        raise ValueError(cfg.parents)
    if cfg.grid is None:
        n_draw = cfg.N
    else:
        if cfg.grid * cfg.grid != cfg.N or cfg.grid % cfg.patch:
            raise ValueError("grid must be square with side a multiple of the patch")
        n_draw = (cfg.grid // cfg.patch) ** 2
    par = rng.choice(M0, size=n_draw, p=pw)
    slot = rng.integers(0, C + 1, size=n_draw)
    rows = np.where(slot == 0, par, M0 + par * C + (slot - 1)).astype(np.int32)
    if cfg.grid is None:
        return rows
    G, p = cfg.grid, cfg.patch
    y, x = np.divmod(np.arange(cfg.N), G)
    return rows[(y // p) * (G // p) + (x // p)]


def make(cfg: Config, seed: Optional[int] = None, checker=None, margin: float = 1e-4) -> dict:
    """Draw one workload.  Returns float32 arrays Q, K, V [BH, N, d], codebook
    [H, Mt, d], the generating row of every key, and redraw counts."""
    seed = cfg.seed if seed is None else seed
    cfg = cfg.replace(seed=seed)
    BH, N, d = cfg.BH, cfg.N, cfg.d
    cb = make_codebook(seed, cfg.H, cfg.M0, cfg.C, d)
    rows = np.zeros((BH, N), dtype=np.int32)
    K = np.empty((BH, N, d), dtype=np.float32)
    V = np.empty((BH, N, d), dtype=np.float32)
    Q = np.empty((BH, N, d), dtype=np.float32)
    for bh in range(BH):
        h = bh % cfg.H
        rows[bh] = _cluster_rows(cfg, bh)
        rk = _rng(seed, _ROLE_KEYS, bh)
        K[bh] = round_to_dtype(cb[h][rows[bh]].astype(np.float64) + 0.1 * rk.standard_normal((N, d)), cfg.dtype)
        V[bh] = round_to_dtype(_rng(seed, _ROLE_VALUES, bh).standard_normal((N, d)), cfg.dtype)
        Q[bh] = round_to_dtype(_rng(seed, _ROLE_QUERIES, bh).standard_normal((N, d)), cfg.dtype)
    redraw_keys = 0
    redraw_tiles = 0
    if checker is not None:
        for attempt in range(1, 101):
            mg = checker.key_margins(cfg, K, cb)
            bad = np.argwhere(mg < margin)
            if bad.size == 0:
                break
            redraw_keys += len(bad)
            for bh, j in bad:
                rr = _rng(seed, _ROLE_REDRAW_K, int(bh), int(j), attempt)
                base = cb[bh % cfg.H][rows[bh, j]].astype(np.float64)
                K[bh, j] = round_to_dtype(base + 0.1 * rr.standard_normal(d), cfg.dtype)
        else:
            raise RuntimeError("could not draw keys clear of assignment ties")
        Ps = [p for p in (cfg.sweep_P or (cfg.P,)) if 0 < p < cfg.M0]
        if Ps:
            for attempt in range(1, 101):
                tm = np.full((BH, cfg.tiles), np.inf)
                for P in Ps:
                    tm = np.minimum(tm, checker.tile_margins(cfg.replace(P=P), Q, K, cb))
                bad = np.argwhere(tm < margin)
                if bad.size == 0:
                    break
                redraw_tiles += len(bad)
                for bh, t in bad:
                    i0, i1 = t * cfg.block_q, min(N, (t + 1) * cfg.block_q)
                    rr = _rng(seed, _ROLE_REDRAW_Q, int(bh), int(t), attempt)
                    Q[bh, i0:i1] = round_to_dtype(rr.standard_normal((i1 - i0, d)), cfg.dtype)
            else:
                raise RuntimeError("could not draw query tiles clear of top-P ties")
    return {
        "cfg": cfg, "Q": Q, "K": K, "V": V, "codebook": cb, "true_rows": rows,
        "redraw_keys": redraw_keys, "redraw_tiles": redraw_tiles,
    }
