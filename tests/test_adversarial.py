"""GPU parity on adversarial inputs ("AVQ-Attention: Adaptive Vector-Quantized
Attention": Alg. 1 and 2, Sec. C Eq. 15-17, Sec. D Eq. 18), through the C
interface, in bf16 and fp32, with sequence lengths that are not a whole number
of query tiles or key chunks:

* every key of a head on one parent (the heaviest contention on one codeword's
  value sum and count);
* every key an exact copy of a child codeword, with P = M0: every key moves, so
  every refined parent keeps no key of its own (n_stay = 0) and Eq. 9 must
  remove every parent contribution; the output is then exact softmax attention
  (Eq. 1), checked against numpy as well as the oracle;
* every key an exact copy of a parent codeword (d_best = 0, no key moves): the
  children are all empty and the output is exact softmax attention for any P.

The last two are not drawn with top-P margins, so the top-P sets are compared
where the double-precision decision is clear and checked for validity
elsewhere.
"""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import check_topp, check_vsum, compare_y, run_gpu, say

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (H, d, M0, C, block_q)
    "small": (2, 64, 16, 4, 64),
    "headline": (2, 64, 64, 8, 128),
}


def _softmax_attention(Q, K, V, scale):
    """Eq. 1 with numpy, per head, in double."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    S = scale * np.matmul(Q, np.swapaxes(K, -1, -2))
    S -= S.max(axis=-1, keepdims=True)
    A = np.exp(S)
    return np.matmul(A, V) / A.sum(axis=-1)[..., None]


def _cfg(shape, dtype, N):
    H, d, M0, C, bq = SHAPES[shape]
    return gen.Config(f"adv-{shape}", B=1, H=H, N=N, d=d, M0=M0, C=C, P=min(16, M0), block_q=bq, dtype=dtype,
                      grid=None, parents="uniform", seed=4242)


def _codeword_keys(cfg, rows_of_head, seed):
    """Keys that are exact copies of the given codebook rows (per head, in a
    shuffled order, repeated to N), with N(0, 1) queries and values."""
    cb = gen.make_codebook(cfg.seed, cfg.H, cfg.M0, cfg.C, cfg.d)
    rng = np.random.default_rng(seed)
    K = np.empty((cfg.BH, cfg.N, cfg.d), np.float32)
    for bh in range(cfg.BH):
        r = np.resize(rng.permutation(rows_of_head), cfg.N)
        K[bh] = cb[bh % cfg.H][r]
    Q = gen.round_to_dtype(rng.standard_normal((cfg.BH, cfg.N, cfg.d)), cfg.dtype)
    V = gen.round_to_dtype(rng.standard_normal((cfg.BH, cfg.N, cfg.d)), cfg.dtype)
    return {"cfg": cfg, "Q": Q, "K": gen.round_to_dtype(K, cfg.dtype), "V": V, "codebook": cb}


def _copy_margin(cb, rows):
    """For keys that are exact copies of the codebook rows `rows` (one head):
    the smallest squared distance from such a key to any other codeword of the
    head, over 1 + |k|^2.  When every key is a copy of a codeword, the nearest
    codeword is the key itself at distance 0 and every decision of Alg. 1 that
    matters is clear by this much."""
    C2 = np.asarray(cb, np.float64)
    worst = np.inf
    for r in rows:
        d2 = ((C2 - C2[r]) ** 2).sum(-1)
        d2[r] = np.inf
        worst = min(worst, d2.min() / (1.0 + (C2[r] ** 2).sum()))
    return worst


def _check_against_oracle(data, P, expect_rows=None, copies_of=None):
    """Assignments, counts and value sums exact / within the summation bound;
    importances within 1e-5 * |tile|; top-P equal where decisive and valid
    everywhere; Y against the substituted-codebook form.  Returns (GPU Y,
    oracle Y).  copies_of: the codebook rows the keys are exact copies of (the
    assignment's margin is then the distance to the next codeword)."""
    cfg = data["cfg"]
    bq = cfg.block_q
    o = oracle.Oracle.for_cfg(cfg)
    if copies_of is None:
        margin = o.key_margins(data["K"], data["codebook"]).min()
    else:
        margin = min(_copy_margin(data["codebook"][h], copies_of) for h in range(cfg.H))
    assert margin >= 1e-4, "every assignment must be clear of ties"
    g = run_gpu(data, P)
    parent, row = o.assign(data["K"], data["codebook"])
    if expect_rows is not None:
        assert np.array_equal(row, expect_rows)
    assert np.array_equal(g["row"], row), f"assignments differ at {np.argwhere(g['row'] != row)[:5]}"
    vsum, counts = o.aggregate(data["V"], parent, row)
    assert np.array_equal(g["counts"], counts), "counts differ"
    vabs, _ = o.aggregate(np.abs(data["V"].astype(np.float64)), parent, row)
    check_vsum(g["vsum"], vsum, vabs, counts)
    w = o.importance(data["Q"], data["codebook"], counts, bq, cfg.scale)
    werr = np.abs(g["importance"].astype(np.float64) - w).max()
    say(f"  importance max|err| = {werr:.3e}")
    assert werr <= 1e-5 * bq
    if P > 0:
        srt = -np.sort(-w, axis=-1)
        if P < cfg.M0:
            margin = (srt[..., P - 1] - srt[..., P]) / np.maximum(srt[..., P - 1], 1.0)
            decisive = (margin >= 1e-4) | ((srt[..., P - 1] == 0.0) & (srt[..., P] == 0.0))
        else:
            decisive = np.ones(srt.shape[:-1], bool)
        sel = o.select(w, P)
        say(f"  decisive tiles {decisive.mean() * 100:.1f}%")
        assert np.array_equal(g["sel"][decisive], sel[decisive])
        check_topp(g["sel"], g["importance"], w, P, cfg.name)
        sel = g["sel"]
    else:
        sel = np.zeros((cfg.BH, cfg.tiles, 0), np.int32)
    Y = o.attention_substituted(data["Q"], data["codebook"], vsum, counts, sel, P, bq, cfg.scale)
    compare_y(g["Y"], Y, cfg.dtype, f"{cfg.name} P={P}")
    return g["Y"], Y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,N", [("small", 2048 + 64 + 5), ("headline", 16384 + 37)])
def test_one_parent(dtype, shape, N):
    """Every key of every head drawn at parent 0's cell (the parent or one of
    its children, plus noise): all keys update one parent row and its C child
    rows, from every workgroup of the head at once."""
    cfg = _cfg(shape, dtype, N).replace(parents="zipf", zipf_s=80.0, H=3)
    say(f"[adversarial] all keys on one parent: {cfg.name} N{N} {dtype}")
    data = gen.make(cfg, checker=oracle.MarginChecker())
    o = oracle.Oracle.for_cfg(cfg)
    parent, _ = o.assign(data["K"], data["codebook"])
    assert (parent == 0).all(), "the case needs every key on parent 0"
    _check_against_oracle(data, cfg.P)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ["small", "headline"])
def test_keys_are_children(dtype, shape):
    """Every key an exact copy of a child codeword (each child at least twice,
    N ragged), P = M0: every key moves, every refined parent's residual count
    is zero, and the output is exact softmax attention (Eq. 1)."""
    H, d, M0, C, bq = SHAPES[shape]
    N = 2 * M0 * C + 37
    cfg = _cfg(shape, dtype, N)
    say(f"[adversarial] keys = children, P = M0: {cfg.name} N{N} {dtype}")
    data = _codeword_keys(cfg, np.arange(M0, M0 * (1 + C)), seed=7)
    cb = data["codebook"]
    expect = np.array([[int(np.flatnonzero((cb[bh % H] == k).all(-1))[0]) for k in data["K"][bh]]
                       for bh in range(cfg.BH)])
    assert (expect >= M0).all()
    gY, oY = _check_against_oracle(data, M0, expect_rows=expect, copies_of=np.arange(M0, M0 * (1 + C)))
    ref = _softmax_attention(data["Q"], data["K"], data["V"], cfg.scale)
    np.testing.assert_allclose(oY, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
    compare_y(gY, ref, dtype, f"{cfg.name} against numpy softmax attention")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", ["small", "headline"])
def test_keys_are_parents(dtype, shape):
    """Every key an exact copy of a parent codeword (d_best = 0; N ragged): no
    key moves, every child is empty, and for any P the output is exact softmax
    attention (Eq. 1)."""
    H, d, M0, C, bq = SHAPES[shape]
    N = 3 * M0 + 5
    cfg = _cfg(shape, dtype, N)
    data = _codeword_keys(cfg, np.arange(M0), seed=8)
    expect = np.array([[int(np.flatnonzero((data["codebook"][bh % H][:M0] == k).all(-1))[0]) for k in data["K"][bh]]
                       for bh in range(cfg.BH)])
    ref = _softmax_attention(data["Q"], data["K"], data["V"], cfg.scale)
    for P in (0, min(4, M0), M0):
        say(f"[adversarial] keys = parents: {cfg.name} N{N} {dtype} P={P}")
        gY, oY = _check_against_oracle(data, P, expect_rows=expect, copies_of=np.arange(M0))
        np.testing.assert_allclose(oY, ref, rtol=0, atol=1e-10 * np.abs(ref).max())
        compare_y(gY, ref, dtype, f"{cfg.name} P={P} against numpy softmax attention")
