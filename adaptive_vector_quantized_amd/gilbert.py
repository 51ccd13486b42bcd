"""Generalized Hilbert ("Gilbert") curve over a W x H token grid: the query
order the pages use so that a query tile of consecutive curve positions is a
compact 2-D region of the image ("AVQ-Attention: Adaptive Vector-Quantized
Attention", Sec. 4.3 and Fig. 3; the curve of ref. [34]).

The recursion in _walk follows, step for step, the "gilbert2d" reference
implementation of the generalized Hilbert curve by Jakub Červený
(github.com/jakubcerveny/gilbert), re-expressed as a Python generator: a
rectangle given by an origin and two axis vectors (a: the major axis, b: the
minor one) is cut in two halves along a when it is long and thin (2w > 3h),
otherwise into three parts (up along b, across along a, down along b back to
the far corner), odd half-lengths nudged so that the pieces keep even lengths
where they can.  That implementation's licence notice:

    BSD 2-Clause License
    Copyright (c) 2018, Jakub Červený
    All rights reserved.
    Redistribution and use in source and binary forms, with or without
    modification, are permitted provided that the following conditions are
    met: 1. Redistributions of source code must retain the above copyright
    notice, this list of conditions and the following disclaimer.
    2. Redistributions in binary form must reproduce the above copyright
    notice, this list of conditions and the following disclaimer in the
    documentation and/or other materials provided with the distribution.
    THIS SOFTWARE IS PROVIDED BY THE COPYRIGHT HOLDERS AND CONTRIBUTORS "AS
    IS" AND ANY EXPRESS OR IMPLIED WARRANTIES, INCLUDING, BUT NOT LIMITED TO,
    THE IMPLIED WARRANTIES OF MERCHANTABILITY AND FITNESS FOR A PARTICULAR
    PURPOSE ARE DISCLAIMED. IN NO EVENT SHALL THE COPYRIGHT HOLDER OR
    CONTRIBUTORS BE LIABLE FOR ANY DIRECT, INDIRECT, INCIDENTAL, SPECIAL,
    EXEMPLARY, OR CONSEQUENTIAL DAMAGES (INCLUDING, BUT NOT LIMITED TO,
    PROCUREMENT OF SUBSTITUTE GOODS OR SERVICES; LOSS OF USE, DATA, OR
    PROFITS; OR BUSINESS INTERRUPTION) HOWEVER CAUSED AND ON ANY THEORY OF
    LIABILITY, WHETHER IN CONTRACT, STRICT LIABILITY, OR TORT (INCLUDING
    NEGLIGENCE OR OTHERWISE) ARISING IN ANY WAY OUT OF THE USE OF THIS
    SOFTWARE, EVEN IF ADVISED OF THE POSSIBILITY OF SUCH DAMAGE.

Consecutive cells are adjacent for every grid whose sides are powers of two
(and for most others).  Host-side utility: the attention call takes the
resulting permutation as an array.
"""
from __future__ import annotations

from typing import Iterator, List, Tuple

import numpy as np


def _sgn(v: int) -> int:
    return (v > 0) - (v < 0)


def _walk(x: int, y: int, ax: int, ay: int, bx: int, by: int) -> Iterator[Tuple[int, int]]:
    w, h = abs(ax + ay), abs(bx + by)     # extent along a and along b
    dax, day = _sgn(ax), _sgn(ay)         # unit step along a
    dbx, dby = _sgn(bx), _sgn(by)         # unit step along b
    if h == 1:                            # a single row: walk along a
        for _ in range(w):
            yield x, y
            x, y = x + dax, y + day
        return
    if w == 1:                            # a single column: walk along b
        for _ in range(h):
            yield x, y
            x, y = x + dbx, y + dby
        return
    ax2, ay2, bx2, by2 = ax // 2, ay // 2, bx // 2, by // 2
    w2, h2 = abs(ax2 + ay2), abs(bx2 + by2)
    if 2 * w > 3 * h:
        # long rectangle: two halves along a, each a full-height rectangle
        if w2 % 2 and w > 2:
            ax2, ay2 = ax2 + dax, ay2 + day
        yield from _walk(x, y, ax2, ay2, bx, by)
        yield from _walk(x + ax2, y + ay2, ax - ax2, ay - ay2, bx, by)
    else:
        # up the first half of b, across the full a, back down to the corner
        if h2 % 2 and h > 2:
            bx2, by2 = bx2 + dbx, by2 + dby
        yield from _walk(x, y, bx2, by2, ax2, ay2)
        yield from _walk(x + bx2, y + by2, ax, ay, bx - bx2, by - by2)
        yield from _walk(x + (ax - dax) + (bx2 - dbx), y + (ay - day) + (by2 - dby),
                         -bx2, -by2, -(ax - ax2), -(ay - ay2))


def curve(width: int, height: int) -> List[Tuple[int, int]]:
    """Cells (x, y) of a width x height grid in curve order, from (0, 0)."""
    if width < 1 or height < 1:
        return []
    if width >= height:
        return list(_walk(0, 0, width, 0, 0, height))
    return list(_walk(0, 0, 0, height, width, 0))


def query_order(width: int, height: int) -> np.ndarray:
    """int32 permutation of the row-major token indices y * width + x: entry
    i is the token at curve position i (the order the attention call visits
    its queries in)."""
    cells = curve(width, height)
    return np.array([y * width + x for x, y in cells], dtype=np.int32)
