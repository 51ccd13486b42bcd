"""CPU oracle for the AVQ-Attention forward pass (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and nothing
here imports the HIP library.  The arithmetic lives in ``avq_oracle.c`` (plain
loops, double precision throughout, decisions included); this file only
marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "avq_oracle.c")
LIB = os.path.join(_HERE, "libavq_oracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over independent heads)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or LIB
    if path is None and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(SRC)):
        build()
    lib = ctypes.CDLL(p)
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    P = ctypes.c_void_p
    lib.avqo_assign.argtypes = [i32] * 6 + [P, P, P, P]
    lib.avqo_aggregate.argtypes = [i32] * 6 + [P, P, P, P, P]
    lib.avqo_importance.argtypes = [i32] * 6 + [P, P, P, i32, dbl, P]
    lib.avqo_importance_tiled_f64.argtypes = [i32] * 6 + [P, P, P, i32, dbl, i32, P]
    lib.avqo_select.argtypes = [i64, i32, i32, P, P]
    for f in (lib.avqo_attention_alg2, lib.avqo_attention_substituted):
        f.argtypes = [i32] * 6 + [P, P, P, P, P, i32, i32, dbl, P]
    lib.avqo_attention_quantized_keys.argtypes = [i32] * 6 + [P, P, P, P, P, P, i32, i32, dbl, P]
    lib.avqo_exact_attention.argtypes = [i32, i32, i32, P, P, P, dbl, i32, i32, P]
    lib.avqo_key_margins.argtypes = [i32] * 6 + [P, P, P]
    lib.avqo_tile_margin.argtypes = [i32, i32, i32, P, P, P, i32, dbl]
    lib.avqo_tile_margin.restype = dbl
    lib.avqo_tile_margins.argtypes = [i32] * 6 + [P, P, P, i32, i32, dbl, P]
    lib.avqo_codebook_update_f64.argtypes = [i32] * 5 + [P, P, dbl, P, P, P]
    if path is None:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc: int):
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")


class Oracle:
    """Numpy-facing wrapper.  Shapes: K, V, Q [B*H, N, d]; codebook [H, Mt, d]."""

    def __init__(self, B: int, H: int, N: int, d: int, M0: int, C: int, lib=None):
        self.B, self.H, self.N, self.d, self.M0, self.C = B, H, N, d, M0, C
        self.Mt = M0 * (1 + C)
        self.lib = lib or load()

    @classmethod
    def for_cfg(cls, cfg, lib=None) -> "Oracle":
        return cls(cfg.B, cfg.H, cfg.N, cfg.d, cfg.M0, cfg.C, lib=lib)

    @property
    def dims(self):
        return (self.B, self.H, self.N, self.d, self.M0, self.C)

    def tiles(self, bq: int) -> int:
        return (self.N + bq - 1) // bq

    # Sec. 4.2, Alg. 1
    def assign(self, K, codebook):
        K, cb = _f64(K), _f64(codebook)
        BH = self.B * self.H
        parent = np.zeros((BH, self.N), np.int32)
        row = np.zeros((BH, self.N), np.int32)
        _ok(self.lib.avqo_assign(*self.dims, _p(K), _p(cb), _p(parent), _p(row)))
        return parent, row

    # Eq. 3
    def aggregate(self, V, parent, row):
        V, parent, row = _f64(V), _i32(parent), _i32(row)
        BH = self.B * self.H
        vsum = np.zeros((BH, self.Mt, self.d), np.float64)
        counts = np.zeros((BH, self.Mt), np.int32)
        _ok(self.lib.avqo_aggregate(*self.dims, _p(V), _p(parent), _p(row), _p(vsum), _p(counts)))
        return vsum, counts

    # Eq. 7, in double
    def importance(self, Q, codebook, counts, bq: int, scale: float):
        Q, cb, counts = _f64(Q), _f64(codebook), _i32(counts)
        w = np.zeros((self.B * self.H, self.tiles(bq), self.M0), np.float64)
        _ok(self.lib.avqo_importance(*self.dims, _p(Q), _p(cb), _p(counts), bq, scale, _p(w)))
        return w

    def importance_tiled_f64(self, Q, codebook, counts, bq: int, scale: float, tile: int):
        """App. B (Eq. 13-14): importance with the approximate denominator over
        codeword tiles of ``tile`` parents."""
        Q, cb, counts = _f64(Q), _f64(codebook), _i32(counts)
        w = np.zeros((self.B * self.H, self.tiles(bq), self.M0), np.float64)
        _ok(self.lib.avqo_importance_tiled_f64(*self.dims, _p(Q), _p(cb), _p(counts), bq, scale, tile, _p(w)))
        return w

    # Alg. 2, the top-P parent choice (on double importances)
    def select(self, w, P: int):
        w = _f64(w)
        R = int(np.prod(w.shape[:-1]))
        sel = np.zeros(w.shape[:-1] + (P,), np.int32)
        _ok(self.lib.avqo_select(R, self.M0, P, _p(w), _p(sel)))
        return sel

    def _attn(self, fn, Q, codebook, vsum, counts, sel, P, bq, scale):
        Q, cb, vsum, counts, sel = _f64(Q), _f64(codebook), _f64(vsum), _i32(counts), _i32(sel)
        Y = np.zeros((self.B * self.H, self.N, self.d), np.float64)
        _ok(fn(*self.dims, _p(Q), _p(cb), _p(vsum), _p(counts), _p(sel), P, bq, scale, _p(Y)))
        return Y

    # O3: Alg. 2 as written
    def attention_alg2(self, Q, codebook, vsum, counts, sel, P, bq, scale):
        return self._attn(self.lib.avqo_attention_alg2, Q, codebook, vsum, counts, sel, P, bq, scale)

    # O2: Eq. 4 over the substituted codebook (Sec. C)
    def attention_substituted(self, Q, codebook, vsum, counts, sel, P, bq, scale):
        return self._attn(self.lib.avqo_attention_substituted, Q, codebook, vsum, counts, sel, P, bq, scale)

    # O1: quantized-key attention by brute force
    def attention_quantized_keys(self, Q, V, codebook, parent, row, sel, P, bq, scale):
        Q, V, cb = _f64(Q), _f64(V), _f64(codebook)
        parent, row, sel = _i32(parent), _i32(row), _i32(sel)
        Y = np.zeros((self.B * self.H, self.N, self.d), np.float64)
        _ok(self.lib.avqo_attention_quantized_keys(*self.dims, _p(Q), _p(V), _p(cb), _p(parent), _p(row),
                                                   _p(sel), P, bq, scale, _p(Y)))
        return Y

    # Eq. 1
    def exact_attention(self, Q, K, V, scale, i0: int = 0, i1: Optional[int] = None):
        i1 = self.N if i1 is None else i1
        Q, K, V = _f64(Q), _f64(K), _f64(V)
        BH = self.B * self.H
        Y = np.zeros((BH, i1 - i0, self.d), np.float64)
        _ok(self.lib.avqo_exact_attention(BH, self.N, self.d, _p(Q), _p(K), _p(V), scale, i0, i1, _p(Y)))
        return Y

    def key_margins(self, K, codebook):
        K, cb = _f64(K), _f64(codebook)
        m = np.zeros((self.B * self.H, self.N), np.float64)
        _ok(self.lib.avqo_key_margins(*self.dims, _p(K), _p(cb), _p(m)))
        return m

    def tile_margins(self, Q, codebook, counts, P: int, bq: int, scale: float):
        Q, cb, counts = _f64(Q), _f64(codebook), _i32(counts)
        out = np.full((self.B * self.H, self.tiles(bq)), np.inf)
        _ok(self.lib.avqo_tile_margins(*self.dims, _p(Q), _p(cb), _p(counts), bq, P, scale, _p(out)))
        return out

    # App. A, Eq. 11-12 (training): EMA statistics and constrained positions
    def codebook_update(self, ksum, counts, decay: float, S, Nm, codebook):
        """One update step from the batch's per-codeword key sums and counts
        (``aggregate`` with the keys as values).  Returns new (S [H, Mt, d],
        N [H, Mt], codebook [H, Mt, d]) in double; the inputs are not changed."""
        ksum, counts = _f64(ksum), _i32(counts)
        S, Nm, cb = _f64(S).copy(), _f64(Nm).copy(), _f64(codebook).copy()
        _ok(self.lib.avqo_codebook_update_f64(self.B, self.H, self.d, self.M0, self.C, _p(ksum), _p(counts),
                                              float(decay), _p(S), _p(Nm), _p(cb)))
        return S, Nm, cb

    # Sec. 4.3 and Fig. 3: query tiles taken along a token order
    def ordered(self, Q, order):
        """The queries in tile order: tile t holds the queries of rows
        order[t*bq ...].  Returns (an Oracle over the ordered queries, the
        ordered queries [BH, n, d], the rows they came from [n]).  Entries of
        ``order`` outside [0, N) are empty positions and must all follow the
        valid ones (the valid positions then tile like a shorter query array);
        a row named twice is rejected.  The per-tile steps (importance,
        selection, output) take the ordered queries unchanged: a tile is a set
        of queries, whatever rows they sit on."""
        order = np.asarray(order, dtype=np.int64).reshape(-1)
        if order.size != self.N:
            raise ValueError("the order names one row per position (N entries)")
        valid = (order >= 0) & (order < self.N)
        n = int(valid.sum())
        if not valid[:n].all():
            raise ValueError("empty positions must follow the valid ones")
        rows = order[:n]
        if np.unique(rows).size != n:
            raise ValueError("a row is named twice")
        Qo = np.asarray(Q)[:, rows]
        return Oracle(self.B, self.H, n, self.d, self.M0, self.C, lib=self.lib), Qo, rows

    def scatter_rows(self, Yo, rows):
        """Outputs in tile order back to the rows of their queries; rows that
        no position names are NaN."""
        Y = np.full((self.B * self.H, self.N, self.d), np.nan)
        Y[:, rows] = Yo
        return Y

    # the whole forward pass in one call: discrete results + all three output forms
    def forward(self, Q, K, V, codebook, P: int, bq: int, scale: float, forms=("substituted",)):
        parent, row = self.assign(K, codebook)
        vsum, counts = self.aggregate(V, parent, row)
        w = self.importance(Q, codebook, counts, bq, scale)
        sel = self.select(w, P)
        out = {"parent": parent, "row": row, "vsum": vsum, "counts": counts, "importance": w, "sel": sel}
        if "substituted" in forms:
            out["Y"] = self.attention_substituted(Q, codebook, vsum, counts, sel, P, bq, scale)
        if "alg2" in forms:
            out["Y_alg2"] = self.attention_alg2(Q, codebook, vsum, counts, sel, P, bq, scale)
        if "quantized_keys" in forms:
            out["Y_qk"] = self.attention_quantized_keys(Q, V, codebook, parent, row, sel, P, bq, scale)
        return out


class MarginChecker:
    """Tie-distance callbacks for ``gen.make`` built on the oracle (double precision)."""

    def __init__(self, lib=None):
        self.lib = lib or load()

    def key_margins(self, cfg, K, cb):
        return Oracle.for_cfg(cfg, self.lib).key_margins(K, cb)

    def tile_margins(self, cfg, Q, K, cb):
        o = Oracle.for_cfg(cfg, self.lib)
        parent, row = o.assign(K, cb)
        # counts only: aggregate a one-column zero value array
        o1 = Oracle(cfg.B, cfg.H, cfg.N, 1, cfg.M0, cfg.C, lib=self.lib)
        _, counts = o1.aggregate(np.zeros((cfg.BH, cfg.N, 1)), parent, row)
        return o.tile_margins(Q, cb, counts, cfg.P, cfg.block_q, cfg.scale)
