"""Sequences without tokens (N = 0) through the C interface on the GPU.

Alg. 1 with no keys leaves every value sum and count at its first step's
zero ("AVQ-Attention: Adaptive Vector-Quantized Attention", Sec. 4.2, the
precompute kernel): the zeroing calls clear buffers that held anything, the
accumulating call adds nothing, and the attention calls have no query tile to
produce (Alg. 2 runs once per tile)."""
import numpy as np
import pytest

from adaptive_vector_quantized_amd import gen
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_assign_without_keys(dtype):
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS["tiny"].replace(B=2, H=3, dtype=dtype)
    say(f"[empty] assignment calls with N = 0, B{cfg.B} H{cfg.H} M0{cfg.M0} C{cfg.C} {dtype}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    K = torch.zeros((cfg.B, cfg.H, 0, cfg.d), dtype=dt, device=dev)
    cb = torch.from_numpy(gen.make_codebook(cfg.seed, cfg.H, cfg.M0, cfg.C, cfg.d)).to(dt).contiguous().to(dev)
    shape_v, shape_c = (cfg.B, cfg.H, cfg.Mt, cfg.d), (cfg.B, cfg.H, cfg.Mt)
    vsum = torch.full(shape_v, 7.0, device=dev)
    counts = torch.full(shape_c, 5, dtype=torch.int32, device=dev)
    _lib.assign_aggregate(K, K, cb, cfg.C, vsum=vsum, counts=counts)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(vsum)) == 0 and int(torch.count_nonzero(counts)) == 0
    vsum.fill_(7.0)
    counts.fill_(5)
    ksum = torch.full(shape_v, 3.0, device=dev)
    _lib.assign_aggregate_kv(K, K, cb, cfg.C, vsum=vsum, counts=counts, ksum=ksum)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(vsum)) == 0 and int(torch.count_nonzero(counts)) == 0
    assert int(torch.count_nonzero(ksum)) == 0
    # the accumulating call adds nothing to what the buffers hold
    vsum.fill_(7.0)
    counts.fill_(5)
    _lib.assign_aggregate_accum(K, K, cb, cfg.C, vsum=vsum, counts=counts)
    torch.cuda.synchronize()
    assert bool((vsum == 7.0).all()) and bool((counts == 5).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_without_queries(dtype):
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS["tiny"].replace(B=2, H=3, dtype=dtype)
    say(f"[empty] attention calls with N = 0, {dtype}")
    data = gen.make(cfg)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda")
    t4 = lambda a: torch.from_numpy(a).to(dt).reshape(cfg.B, cfg.H, cfg.N, cfg.d).contiguous().to(dev)
    K, V = t4(data["K"]), t4(data["V"])
    cb = torch.from_numpy(data["codebook"]).to(dt).contiguous().to(dev)
    vsum, counts, _ = _lib.assign_aggregate(K, V, cb, cfg.C)
    Q0 = torch.zeros((cfg.B, cfg.H, 0, cfg.d), dtype=dt, device=dev)
    for kw in (dict(), dict(approx_denominator=True)):
        Y, topp, imp = _lib.attention_fwd(Q0, cb, vsum, counts, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                          want_topp=True, want_importance=True, **kw)
        torch.cuda.synchronize()
        assert tuple(Y.shape) == (cfg.B, cfg.H, 0, cfg.d)
        assert topp.numel() == 0 and imp.numel() == 0
    order = torch.zeros((0,), dtype=torch.int32, device=dev)
    Y, _, _ = _lib.attention_fwd(Q0, cb, vsum, counts, cfg.C, cfg.P, cfg.block_q, cfg.scale, query_order=order)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (cfg.B, cfg.H, 0, cfg.d)
    assert np.isfinite(vsum.cpu().numpy()).all()
