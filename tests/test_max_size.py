"""Sizes past 2^31 elements per tensor, checked through a property that holds
at any size, so that the oracle only has to run the small case.

A block of n tokens from the generator, repeated R times along the sequence,
is the input.  The assignment of a key depends only on the key and the
codebook (Alg. 1, "AVQ-Attention: Adaptive Vector-Quantized Attention",
Sec. 4.2), so every key's assignment is its copy's in the block, every count
is R times the block's (Eq. 3) and every value sum R times the block's (up
to float32 rounding).  With R a power of two, R times a count is exact in
float32, and the importances of Eq. 7 (sums of A_ij n_j / Z_i, where R cancels)
and the output (Eq. 6 with Eq. 9: value sums over counts, where R cancels up to
the value sums' rounding) of every query tile equal those of the tile at the
same position in the block, when n is a whole number of tiles.  So the large
run is compared, on every key, codeword and tile, with the oracle's result for
the block: assignments, counts and top-P sets bit for bit, importances within
1e-5 * |tile|, Y within the bf16 bar, value sums within the float32 summation
bound of the R n terms.

The repeated block makes Q, K and V 3 * 2^30 elements (6.4 GB each in bf16)
on the pipelined kernel's path and 2^32 elements (8.6 GB each) on the two-pass
path with 256 parents at d = 128: every per-head, per-key and per-query offset
passes both 2^31 elements and 2^32 bytes.
"""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import U32, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,over,R", [
    # bf16, d 64, 64 parents (Zipf), C 8, P 16, 128-query tiles: the pipelined kernel
    ("grid64", dict(H=3, block_q=128, parents="zipf"), 4096),
    # bf16, d 128, 256 parents, C 8, P 32: parents from L2, the exact second pass
    ("grid256", dict(H=2, N=1024, grid=32), 16384),
])
def test_repeated_block_past_2_31(name, over, R):
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS[name].replace(**over)
    n, bq, P, BH, d = cfg.N, cfg.block_q, cfg.P, cfg.BH, cfg.d
    assert n % bq == 0 and R & (R - 1) == 0
    T = n // bq
    N = n * R
    say(f"[max size] block B{cfg.B} H{cfg.H} N{n} d{d} M0{cfg.M0} C{cfg.C} P{P} bq{bq} {cfg.dtype}, "
        f"repeated {R} times: N {N}, {BH * N * d} elements per tensor")
    data = gen.make(cfg, checker=oracle.MarginChecker())
    o = oracle.Oracle.for_cfg(cfg)
    parent, row = o.assign(data["K"], data["codebook"])
    vsum, counts = o.aggregate(data["V"], parent, row)
    vabs, _ = o.aggregate(np.abs(data["V"].astype(np.float64)), parent, row)
    w = o.importance(data["Q"], data["codebook"], counts, bq, cfg.scale)
    sel = o.select(w, P)
    Ys = o.attention_substituted(data["Q"], data["codebook"], vsum, counts, sel, P, bq, cfg.scale)

    def big(a):
        return to_device(a, cfg.dtype, cfg.B, cfg.H).repeat(1, 1, R, 1).contiguous()

    K, V, Q = big(data["K"]), big(data["V"]), big(data["Q"])
    assert K.shape == (cfg.B, cfg.H, N, d)
    cb = torch.from_numpy(data["codebook"]).to(torch.bfloat16).contiguous().cuda()
    g_vsum, g_counts, g_assign = _lib.assign_aggregate(K, V, cb, cfg.C, want_assign=True)
    del K, V
    Y, g_sel, g_imp = _lib.attention_fwd(Q, cb, g_vsum, g_counts, cfg.C, P, bq, cfg.scale, want_topp=True,
                                         want_importance=True)
    torch.cuda.synchronize()
    del Q
    dev = Y.device

    # every key: its copy's assignment in the block
    row_t = torch.from_numpy(row.astype(np.int32)).to(dev).view(BH, 1, n)
    assert torch.equal(g_assign.view(BH, R, n), row_t.expand(BH, R, n)), "assignments differ"
    # counts R times the block's, exactly
    assert np.array_equal(g_counts.cpu().numpy().reshape(BH, -1), R * counts), "counts differ"
    # value sums: R n terms per codeword's block share, float32 in any order
    gv = g_vsum.cpu().numpy().reshape(BH, cfg.Mt, d).astype(np.float64)
    nn = (R * counts).astype(np.float64)[..., None]
    gamma = nn * U32 / np.maximum(1.0 - nn * U32, 1e-300)
    err = np.abs(gv - R * vsum)
    assert (err <= gamma * R * vabs + 1e-30).all(), "value sums outside the float32 summation bound"
    say(f"  value sums: max |err| / (R sum|v|) = {(err / (R * vabs + 1e-30)).max():.2e}")
    # every tile: the block tile's top-P set, importances and output
    sel_t = torch.from_numpy(sel.astype(np.int32)).to(dev).view(BH, 1, T, P)
    assert torch.equal(g_sel.view(BH, R, T, P), sel_t.expand(BH, R, T, P)), "top-P differs"
    w_t = torch.from_numpy(w).to(dev).view(BH, 1, T, cfg.M0)
    werr = float((g_imp.view(BH, R, T, cfg.M0).double() - w_t).abs().max())
    say(f"  importance max|err| = {werr:.3e}")
    assert werr <= 1e-5 * bq
    scale = float(np.abs(Ys).max())
    ys_t = torch.from_numpy(Ys).to(dev).view(BH, 1, n, d)
    Yv = Y.view(BH, R, n, d)
    yerr = 0.0
    step = max(1, (1 << 28) // (n * d))  # compare about 2^28 elements at a time
    for bh in range(BH):
        for r0 in range(0, R, step):
            yerr = max(yerr, float((Yv[bh, r0:r0 + step].double() - ys_t[bh]).abs().max()))
    say(f"  Y: max|err|/max|Y| = {yerr / scale:.3e} (tol 2e-3)")
    assert yerr <= 2e-3 * scale
    del Y, Yv, g_assign, g_sel, g_imp, g_vsum, g_counts
    torch.cuda.empty_cache()
