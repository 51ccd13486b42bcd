"""avq_attention_prepare + avq_attention_fwd_prepared (the attention call split
into the value-operand preparation and the attention kernel) against
avq_attention_fwd, through the C interface: the two halves run the same
kernels on the same operands and are deterministic, so the outputs agree bit
for bit.  Several query batches attended to one preparation (the aggregates of
Eq. 3 depend on the keys only, "AVQ-Attention: Adaptive Vector-Quantized
Attention", Sec. 4.2-4.3) must each agree with their own avq_attention_fwd.
avq_assign_aggregate_accum adds a batch's aggregates to what the buffers hold
(Eq. 3's sums over the union of the batches), and the prepared attention call
can zero-fill the buffers it no longer reads, so that a loop of accumulate,
prepare and attend needs no fill launch."""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import say, to_device

pytestmark = pytest.mark.gpu


def _setup(cfg):
    import torch
    from adaptive_vector_quantized_amd import _lib
    data = gen.make(cfg, checker=oracle.MarginChecker())
    K, V, Q = (to_device(data[k], cfg.dtype, cfg.B, cfg.H) for k in ("K", "V", "Q"))
    cb = torch.from_numpy(data["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    vsum, counts, _ = _lib.assign_aggregate(K, V, cb, cfg.C)
    return Q, cb, vsum, counts


def _same(a, b, what):
    if a is None:
        assert b is None, what
        return
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), f"{what} differs"


@pytest.mark.parametrize("name,over", [
    ("grid64", {}),                                                          # bf16, d 64, 64 parents, P 16
    ("grid64", dict(P=0)),                                                   # plain VQ attention
    ("grid64", dict(d=128, M0=256, H=2, N=2048 + 5, grid=None, dtype="f32", P=32)),  # tiled parents, fp32
    ("grid64", dict(M0=128, H=3, N=1500, grid=None, P=8, block_q=32)),       # two parent tiles, bf16
    ("grid64", dict(C=0, P=0, H=2, N=777, grid=None)),                       # flat codebook
])
def test_prepared_equals_fwd(name, over):
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS[name].replace(**over)
    P = cfg.P
    say(f"[prepared] B{cfg.B} H{cfg.H} N{cfg.N} d{cfg.d} M0{cfg.M0} C{cfg.C} P{P} bq{cfg.block_q} {cfg.dtype}")
    Q, cb, vsum, counts = _setup(cfg)
    ref = _lib.attention_fwd(Q, cb, vsum, counts, cfg.C, P, cfg.block_q, cfg.scale, want_topp=P > 0,
                             want_importance=True)
    ws = torch.full((_lib.workspace_size(cfg.B, cfg.H, cfg.d, cfg.M0, cfg.C, Q.dtype),), 0xFF, dtype=torch.uint8,
                    device=Q.device)
    ws = _lib.attention_prepare(vsum, counts, cfg.C, Q.dtype, workspace=ws)
    Y = torch.full_like(ref[0], float("nan"))
    got = _lib.attention_fwd_prepared(Q, cb, ws, cfg.C, P, cfg.block_q, cfg.scale, want_topp=P > 0,
                                      want_importance=True, Y=Y)
    torch.cuda.synchronize()
    for a, b, what in zip(ref, got, ("Y", "top-P", "importance")):
        _same(a, b, what)


def test_one_preparation_many_batches():
    """One preparation, three query batches (different queries, the third on
    another stream after the preparation completed), each bit for bit equal to
    avq_attention_fwd on its own queries."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS["grid64"].replace(H=4, N=3000 + 11, grid=None)
    say(f"[prepared] one preparation, three query batches: H{cfg.H} N{cfg.N} {cfg.dtype}")
    Q, cb, vsum, counts = _setup(cfg)
    ws = _lib.attention_prepare(vsum, counts, cfg.C, Q.dtype)
    rng = np.random.default_rng(99)
    Qs = [Q] + [to_device(gen.round_to_dtype(rng.standard_normal((cfg.BH, cfg.N, cfg.d)), cfg.dtype), cfg.dtype,
                          cfg.B, cfg.H) for _ in range(2)]
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for i, q in enumerate(Qs):
        ref = _lib.attention_fwd(q, cb, vsum, counts, cfg.C, cfg.P, cfg.block_q, cfg.scale, want_topp=True,
                                 want_importance=True)
        if i == 2:
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                got = _lib.attention_fwd_prepared(q, cb, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                                  want_topp=True, want_importance=True)
            side.synchronize()
        else:
            got = _lib.attention_fwd_prepared(q, cb, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                              want_topp=True, want_importance=True)
        torch.cuda.synchronize()
        for a, b, what in zip(ref, got, ("Y", "top-P", "importance")):
            _same(a, b, f"batch {i} {what}")


def _keys_values(cfg, seed):
    import torch
    data = gen.make(cfg, seed=seed, checker=oracle.MarginChecker())
    return data, (to_device(data[k], cfg.dtype, cfg.B, cfg.H) for k in ("K", "V", "Q"))


@pytest.mark.parametrize("name,over", [
    ("grid64", dict(H=4, N=3000 + 11, grid=None)),                                    # pipelined kernel
    ("grid64", dict(d=128, M0=256, H=2, N=2048 + 5, grid=None, P=32)),                 # two-pass, split maximum
    ("grid64", dict(C=0, P=0, M0=512, H=2, N=1500, grid=None)),                        # flat, staged values
    ("grid64", dict(dtype="f32", H=2, N=1024 + 3, grid=None, P=8)),                    # fp32
])
def test_accumulate_and_clear(name, over):
    """Two batches accumulated into one set of buffers equal one call over both
    (counts exactly, value sums within the float32 summation bound of the two
    terms); the accumulate -> prepare -> attend(clear) loop gives the outputs of
    avq_assign_aggregate + avq_attention_fwd on every step and leaves the
    buffers zero."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS[name].replace(**over)
    say(f"[accumulate] H{cfg.H} N{cfg.N} d{cfg.d} M0{cfg.M0} C{cfg.C} P{cfg.P} {cfg.dtype}")
    da, (Ka, Va, Qa) = _keys_values(cfg, 11)
    db, (Kb, Vb, Qb) = _keys_values(cfg, 12)
    cb = torch.from_numpy(da["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    # accumulation: A then B on zeroed buffers == the sums of the two separate calls
    va, ca, _ = _lib.assign_aggregate(Ka, Va, cb, cfg.C)
    vb, cbn, _ = _lib.assign_aggregate(Kb, Vb, cb, cfg.C)
    vsum = torch.zeros_like(va)
    counts = torch.zeros_like(ca)
    _lib.assign_aggregate_accum(Ka, Va, cb, cfg.C, vsum=vsum, counts=counts)
    _lib.assign_aggregate_accum(Kb, Vb, cb, cfg.C, vsum=vsum, counts=counts)
    torch.cuda.synchronize()
    assert torch.equal(counts, ca + cbn), "accumulated counts differ"
    va_abs, _, _ = _lib.assign_aggregate(Ka, Va.abs(), cb, cfg.C)
    vb_abs, _, _ = _lib.assign_aggregate(Kb, Vb.abs(), cb, cfg.C)
    n = (ca + cbn).double()[..., None]
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    err = (vsum.double() - (va.double() + vb.double())).abs()
    assert bool((err <= 2 * gamma * (va_abs.double() + vb_abs.double()) + 1e-30).all()), "accumulated sums"
    # the loop: accumulate into zero buffers, prepare, attend and clear
    vsum.zero_()
    counts.zero_()
    ws = torch.empty((_lib.workspace_size(cfg.B, cfg.H, cfg.d, cfg.M0, cfg.C, Qa.dtype),), dtype=torch.uint8,
                     device=Qa.device)
    for (K, V, Q) in ((Ka, Va, Qa), (Kb, Vb, Qb), (Ka, Va, Qa)):
        v1, c1, _ = _lib.assign_aggregate(K, V, cb, cfg.C)
        Y1, t1, i1 = _lib.attention_fwd(Q, cb, v1, c1, cfg.C, cfg.P, cfg.block_q, cfg.scale, want_topp=cfg.P > 0,
                                        want_importance=True)
        _lib.assign_aggregate_accum(K, V, cb, cfg.C, vsum=vsum, counts=counts)
        torch.cuda.synchronize()
        assert torch.equal(counts, c1), "counts of the step"
        _lib.attention_prepare(vsum, counts, cfg.C, Q.dtype, workspace=ws)
        Y2, t2, i2 = _lib.attention_fwd_prepared(Q, cb, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                                 want_topp=cfg.P > 0, want_importance=True, clear_vsum=vsum,
                                                 clear_counts=counts)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(vsum)) == 0 and int(torch.count_nonzero(counts)) == 0, "buffers not cleared"
        assert (t1 is None and t2 is None) or torch.equal(t1, t2), "top-P of the step"
        # the value sums of two calls may round differently (float atomics in
        # any order): Y and the importances agree to that rounding
        scale = float(Y1.abs().max())
        assert float((Y1 - Y2).abs().max()) <= 1e-5 * scale, "Y of the step"
        assert float((i1 - i2).abs().max()) <= 1e-5 * cfg.block_q, "importance of the step"
    # no queries: the call only clears
    vsum.fill_(1.0)
    counts.fill_(3)
    Q0 = Qa[:, :, :0].contiguous()
    _lib.attention_fwd_prepared(Q0, cb, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale, clear_vsum=vsum,
                                clear_counts=counts)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(vsum)) == 0 and int(torch.count_nonzero(counts)) == 0, "N = 0 did not clear"
