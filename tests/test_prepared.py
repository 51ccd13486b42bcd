"""avq_attention_prepare + avq_attention_fwd_prepared (the attention call split
into the value-operand preparation and the attention kernel) against
avq_attention_fwd, through the C interface: the two halves run the same
kernels on the same operands and are deterministic, so the outputs agree bit
for bit.  Several query batches attended to one preparation (the aggregates of
Eq. 3 depend on the keys only, "AVQ-Attention: Adaptive Vector-Quantized
Attention", Sec. 4.2-4.3) must each agree with their own avq_attention_fwd."""
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
    ws = _lib.attention_prepare(vsum, cfg.C, Q.dtype, workspace=ws)
    Y = torch.full_like(ref[0], float("nan"))
    got = _lib.attention_fwd_prepared(Q, cb, counts, ws, cfg.C, P, cfg.block_q, cfg.scale, want_topp=P > 0,
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
    ws = _lib.attention_prepare(vsum, cfg.C, Q.dtype)
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
                got = _lib.attention_fwd_prepared(q, cb, counts, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                                  want_topp=True, want_importance=True)
            side.synchronize()
        else:
            got = _lib.attention_fwd_prepared(q, cb, counts, ws, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                              want_topp=True, want_importance=True)
        torch.cuda.synchronize()
        for a, b, what in zip(ref, got, ("Y", "top-P", "importance")):
            _same(a, b, f"batch {i} {what}")
