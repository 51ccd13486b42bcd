"""avq_attention_fwd_noalloc (the attention call whose operands live in the
library's static device scratch instead of a caller workspace) against
avq_attention_fwd, through the C interface, on two calls in a row: the second
with a smaller input, so that it runs over scratch the first call left
behind.  Both calls share their kernels and are deterministic, so the outputs
must agree bit for bit."""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import say, to_device

pytestmark = pytest.mark.gpu


def _both(cfg, P):
    import torch
    from adaptive_vector_quantized_amd import _lib
    data = gen.make(cfg, checker=oracle.MarginChecker())
    K, V, Q = (to_device(data[k], cfg.dtype, cfg.B, cfg.H) for k in ("K", "V", "Q"))
    cb = torch.from_numpy(data["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    vsum, counts, _ = _lib.assign_aggregate(K, V, cb, cfg.C)
    Y1, topp1, imp1 = _lib.attention_fwd(Q, cb, vsum, counts, cfg.C, P, cfg.block_q, cfg.scale,
                                         want_topp=P > 0, want_importance=True)
    T = cfg.tiles
    Y2 = torch.full_like(Y1, float("nan"))
    topp2 = torch.full((cfg.B, cfg.H, T, P), -1, dtype=torch.int32, device=Q.device) if P > 0 else None
    imp2 = torch.full((cfg.B, cfg.H, T, cfg.M0), float("nan"), dtype=torch.float32, device=Q.device)
    _lib.attention_fwd_noalloc(Q, cb, vsum, counts, cfg.C, P, cfg.block_q, cfg.scale, Y=Y2, topp=topp2,
                               importance=imp2)
    torch.cuda.synchronize()
    return (Y1, topp1, imp1), (Y2, topp2, imp2)


def _check(cfg, P):
    say(f"[no-alloc] B{cfg.B} H{cfg.H} N{cfg.N} d{cfg.d} M0{cfg.M0} C{cfg.C} P{P} {cfg.dtype}")
    (Y1, t1, i1), (Y2, t2, i2) = _both(cfg, P)
    assert np.array_equal(Y1.cpu().numpy(), Y2.cpu().numpy()), "Y differs"
    assert np.array_equal(i1.cpu().numpy(), i2.cpu().numpy()), "importance differs"
    if P > 0:
        assert np.array_equal(t1.cpu().numpy(), t2.cpu().numpy()), "top-P differs"


def test_noalloc_two_calls():
    """A 64x64-grid workload (12 heads), then a smaller one (2 heads, a ragged
    N, a different codebook size) reusing the scratch."""
    big = gen.CONFIGS["grid64"]
    _check(big, big.P)
    small = gen.CONFIGS["grid64"].replace(H=2, N=1000 + 37, grid=None, M0=32, P=8, seed=77)
    _check(small, small.P)


def test_noalloc_d128_fp32_then_flat():
    """d = 128 with 256 parents in fp32 (the scratch's largest use here), then a
    smaller flat-codebook call (P = 0)."""
    _check(gen.CONFIGS["grid64"].replace(d=128, M0=256, H=2, N=2048 + 5, grid=None, dtype="f32", P=32), 32)
    _check(gen.CONFIGS["grid64"].replace(M0=64, C=0, P=0, H=1, N=300, grid=None), 0)
