"""The query order: the generalized Hilbert ("Gilbert") curve over a token
grid (Sec. 4.3, Fig. 3 of "AVQ-Attention: Adaptive Vector-Quantized
Attention").  Checked against what a space-filling curve must be: a
permutation of the grid whose consecutive cells are neighbours, the Hilbert
curve's nested squares on power-of-two grids, and tiles that are compact 2-D
regions at every tile size (the property the pages use it for).  CPU only."""
import numpy as np
import pytest

from adaptive_vector_quantized_amd import gilbert

SHAPES = [(1, 1), (1, 9), (12, 1), (2, 2), (3, 2), (7, 5), (5, 7), (28, 28), (30, 21), (21, 30), (64, 64),
          (128, 128), (30, 30), (17, 64), (100, 3)]


@pytest.mark.parametrize("W,H", SHAPES)
def test_curve_is_a_path_through_every_cell(W, H):
    c = gilbert.curve(W, H)
    assert len(c) == W * H and len(set(c)) == W * H
    assert all(0 <= x < W and 0 <= y < H for x, y in c)
    steps = np.abs(np.diff(np.array(c), axis=0)).sum(axis=1) if len(c) > 1 else np.zeros(0)
    # neighbours along the curve are neighbours on the grid; on grids of odd
    # length along the long side and even along the short one a single
    # diagonal step cannot be avoided
    diag = int((steps == 2).sum())
    assert np.all(steps >= 1) and np.all(steps <= 2)
    if (W % 2 == 0 and H % 2 == 0) or (W % 2 == 1 and H % 2 == 1) or min(W, H) == 1:
        assert diag == 0, (W, H, diag)
    else:
        assert diag <= 1, (W, H, diag)
    assert c[0] == (0, 0)
    # it ends on the starting edge along the long side (at the far corner
    # unless the long side is odd and the short one even)
    assert c[-1][1] == 0 if W >= H else c[-1][0] == 0
    long_, short = max(W, H), min(W, H)
    if long_ % 2 == 0 or short % 2 == 1:
        assert c[-1] == ((W - 1, 0) if W >= H else (0, H - 1))
    o = gilbert.query_order(W, H)
    assert o.dtype == np.int32 and np.array_equal(np.sort(o), np.arange(W * H))


@pytest.mark.parametrize("side", [8, 64, 128])
def test_power_of_two_grid_is_the_hilbert_curve(side):
    """On a 2^k x 2^k grid every aligned run of 4^j curve positions fills a
    2^j x 2^j square (the Hilbert curve's recursive quadrants)."""
    o = gilbert.query_order(side, side)
    y, x = np.divmod(o, side)
    j = 1
    while 4 ** j <= side * side:
        n = 4 ** j
        xs, ys = x.reshape(-1, n), y.reshape(-1, n)
        assert np.all(xs.max(1) - xs.min(1) == 2 ** j - 1) and np.all(ys.max(1) - ys.min(1) == 2 ** j - 1)
        assert np.all(xs.min(1) % 2 ** j == 0) and np.all(ys.min(1) % 2 ** j == 0)
        j += 1


def _tiles(order, W, bq):
    y, x = np.divmod(order, W)
    return [(x[i:i + bq], y[i:i + bq]) for i in range(0, len(order), bq)]


def _connected(xs, ys):
    cells = set(zip(xs.tolist(), ys.tolist()))
    seen, todo = set(), [next(iter(cells))]
    while todo:
        c = todo.pop()
        if c in seen:
            continue
        seen.add(c)
        for dx, dy in ((1, 0), (-1, 0), (0, 1), (0, -1)):
            n = (c[0] + dx, c[1] + dy)
            if n in cells and n not in seen:
                todo.append(n)
    return len(seen) == len(cells)


@pytest.mark.parametrize("bq,ntiles", [(32, 25), (64, 13), (128, 7)])
def test_fig3_tiles_are_compact(bq, ntiles):
    """Fig. 3: on a 28 x 28 patch grid, tiles of 32, 64 and 128 consecutive
    curve positions (25, 13 and 7 tiles) are connected regions, and their
    bounding boxes are close to those of a square of bq cells and smaller
    than those of raster order's row strips."""
    W = 28
    o = gilbert.query_order(W, W)
    tiles = _tiles(o, W, bq)
    assert len(tiles) == ntiles
    assert all(_connected(xs, ys) for xs, ys in tiles)

    def perimeter(ts):
        return np.mean([2 * (xs.max() - xs.min() + 1 + ys.max() - ys.min() + 1) for xs, ys in ts])
    raster = _tiles(np.arange(W * W), W, bq)
    # a square of n cells has a bounding perimeter of 4 sqrt(n)
    assert perimeter(tiles) < perimeter(raster)
    assert perimeter(tiles[:-1]) <= 1.3 * 4 * np.sqrt(bq)


def test_every_small_grid():
    """Every grid up to 32 x 32: a permutation of the cells, ending on the
    starting edge of the long side, with unit steps except at most one diagonal
    step, which occurs only when the long side is odd and the short one even."""
    for W in range(1, 33):
        for H in range(1, 33):
            c = gilbert.curve(W, H)
            assert len(c) == W * H and len(set(c)) == W * H, (W, H)
            steps = np.abs(np.diff(np.array(c), axis=0)).sum(axis=1) if len(c) > 1 else np.zeros(0)
            diag = int((steps == 2).sum())
            assert (steps >= 1).all() and (steps <= 2).all(), (W, H)
            long_, short = max(W, H), min(W, H)
            assert diag <= (1 if long_ % 2 == 1 and short % 2 == 0 else 0), (W, H, diag)
            assert (c[-1][1] == 0) if W >= H else (c[-1][0] == 0), (W, H)
