"""GPU parity of the codebook update step (App. A, Eq. 11-12) through the C
interface: avq_codebook_update against the oracle on the same seeded inputs,
and the whole step from the keys (the aggregation call with V = K, then the
update) against the oracle's assignment, aggregation and update.

Bar: the float32 update against the double oracle within 1e-6 of each head's
largest magnitude for S, N and the positions (a handful of roundings of
quantities of that size; a wrong term is off by O(1)); the step from the keys
within a bound carried over from the float32 summation bound of the key sums
(gamma_n * sum |k| per codeword, as for the value sums of the forward pass)."""
import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import U32, check_vsum, say, to_device

pytestmark = pytest.mark.gpu


def _case(seed, B, H, d, M0, C, zero_child=(), zero_parent=(), tiny=()):
    """Seeded random state and batch statistics, float32 values."""
    rng = np.random.default_rng(seed)
    Mt = M0 * (1 + C)
    f = np.float32
    S = (rng.standard_normal((H, Mt, d)) * 3.0).astype(f)
    Nm = rng.uniform(0.5, 20.0, (H, Mt)).astype(f)
    cb = rng.standard_normal((H, Mt, d)).astype(f)
    counts = rng.integers(0, 9, (B, H, Mt)).astype(np.int32)
    ksum = (rng.standard_normal((B, H, Mt, d)) * counts[..., None]).astype(f)
    for h, x in list(zero_child) + list(zero_parent):
        Nm[h, x] = 0.0
        S[h, x] = 0.0
        counts[:, h, x] = 0
        ksum[:, h, x] = 0.0
    for h, x in tiny:
        Nm[h, x] = 1e-30
        S[h, x] = 1e-30 * cb[h, x]
        counts[:, h, x] = 0
        ksum[:, h, x] = 0.0
    return dict(B=B, H=H, d=d, M0=M0, C=C, S=S, Nm=Nm, cb=cb, counts=counts, ksum=ksum)


def _gpu_update(c, decay):
    import torch
    from adaptive_vector_quantized_amd import _lib
    dev = torch.device("cuda:0")
    S = torch.from_numpy(c["S"].copy()).to(dev)
    Nm = torch.from_numpy(c["Nm"].copy()).to(dev)
    cb = torch.from_numpy(c["cb"].copy()).to(dev)
    ksum = torch.from_numpy(c["ksum"]).to(dev)
    counts = torch.from_numpy(c["counts"]).to(dev)
    _lib.codebook_update(ksum, counts, S, Nm, cb, c["C"], decay)
    torch.cuda.synchronize()
    return S.cpu().numpy(), Nm.cpu().numpy(), cb.cpu().numpy()


def _close(name, g, o, per_head_scale, rel):
    err = np.abs(g.astype(np.float64) - o)
    tol = rel * per_head_scale.reshape((-1,) + (1,) * (o.ndim - 1))
    say(f"  {name}: max err / head scale = {(err / tol).max() * rel:.2e} (tol {rel:g})")
    assert (err <= tol).all(), f"{name} differs at {np.argwhere(err > tol)[:5]}"


CASES = {
    "d64 C8": dict(B=2, H=3, d=64, M0=5, C=8),
    "d128 C16": dict(B=3, H=2, d=128, M0=4, C=16),
    "d40 C3": dict(B=1, H=2, d=40, M0=7, C=3),
    "flat": dict(B=2, H=2, d=64, M0=9, C=0),
    "no batch": dict(B=0, H=2, d=64, M0=3, C=4),
    "massless": dict(B=2, H=2, d=64, M0=3, C=4, zero_child=[(0, 3 + 1), (1, 3 + 4 * 2), (1, 3 + 4 * 2 + 3)],
                     zero_parent=[(1, 1)]),
    "all children massless": dict(B=2, H=1, d=64, M0=2, C=4, zero_child=[(0, 2 + c) for c in range(4)]),
    "tiny masses": dict(B=2, H=2, d=64, M0=3, C=4, tiny=[(0, 3 + 2), (1, 3 + 4)]),
}


@pytest.mark.parametrize("decay", [0.99, 0.0, 1.0])
@pytest.mark.parametrize("name", sorted(CASES))
def test_update_unit(name, decay):
    c = _case(sum(map(ord, name)), **CASES[name])
    say(f"[update] {name} decay {decay}")
    gS, gN, gcb = _gpu_update(c, decay)
    o = oracle.Oracle(max(c["B"], 1), c["H"], 1, c["d"], c["M0"], c["C"])
    o.B = c["B"]
    ks = c["ksum"].reshape(-1, c["ksum"].shape[2], c["d"])
    ct = c["counts"].reshape(-1, c["counts"].shape[2])
    # the C interface takes the decay as a float: the oracle gets that value
    oS, oN, ocb = o.codebook_update(ks, ct, float(np.float32(decay)), c["S"], c["Nm"], c["cb"])
    H = c["H"]
    _close("S", gS, oS, np.abs(oS).reshape(H, -1).max(1) + 1e-30, 1e-6)
    _close("N", gN, oN, np.abs(oN).reshape(H, -1).max(1) + 1e-30, 1e-6)
    _close("codebook", gcb, ocb, np.abs(ocb).reshape(H, -1).max(1), 1e-6)


@pytest.mark.parametrize("fused", [False, True])
def test_update_from_keys_grid64(fused):
    """The whole step from the keys of the 64x64-grid workload (bf16 keys,
    M0 = 64, C = 8, 4 heads, batch 2), from a state of one key at every
    codeword's position: the key sums from the aggregation call with V = K, or
    (fused) from avq_assign_aggregate_kv next to the value sums, then the
    update."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS["grid64"].replace(B=2, H=4)
    data = gen.make(cfg, checker=oracle.MarginChecker())
    decay = 0.99
    say(f"[update] from keys {cfg.name} B{cfg.B} H{cfg.H} N{cfg.N} M0{cfg.M0} C{cfg.C}")
    cb32 = data["codebook"].astype(np.float32)
    S0 = cb32.copy()                      # N = 1: one key at each position
    N0 = np.ones((cfg.H, cfg.Mt), np.float32)
    dev = torch.device("cuda:0")
    K = torch.from_numpy(data["K"]).to(torch.bfloat16).reshape(cfg.B, cfg.H, cfg.N, cfg.d).contiguous().to(dev)
    S, Nm, cb = (torch.from_numpy(a.copy()).to(dev) for a in (S0, N0, cb32))
    if fused:
        V = torch.from_numpy(data["V"]).to(torch.bfloat16).reshape(K.shape).contiguous().to(dev)
        _, counts_g, _, ksum_g = _lib.assign_aggregate_kv(K, V, cb.to(torch.bfloat16).contiguous(), cfg.C)
        _lib.codebook_update(ksum_g, counts_g, S, Nm, cb, cfg.C, decay)
    else:
        _lib.update_codebook(K, cb, S, Nm, cfg.C, decay)
    torch.cuda.synchronize()
    gS, gN, gcb = S.cpu().numpy(), Nm.cpu().numpy(), cb.cpu().numpy()
    o = oracle.Oracle.for_cfg(cfg)
    parent, row = o.assign(data["K"], data["codebook"])
    ksum, counts = o.aggregate(data["K"], parent, row)
    kabs, _ = o.aggregate(np.abs(data["K"].astype(np.float64)), parent, row)
    oS, oN, ocb = o.codebook_update(ksum, counts, float(np.float32(decay)), S0, N0, cb32)
    assert (np.abs(gN - oN) <= 4 * U32 * (np.abs(oN) + 1.0)).all()
    # the key sums carry the float32 summation bound gamma_n sum |k| into S,
    # and S / N into the means; the projection adds at most its residual's error
    n = counts.astype(np.float64)
    gamma = n * U32 / np.maximum(1.0 - n * U32, 1e-300)
    ks_err = (gamma[..., None] * kabs).reshape(cfg.B, cfg.H, cfg.Mt, cfg.d).sum(0) * (1 - decay)
    arith = 8 * U32 * (np.abs(oS) + np.abs(S0))
    s_err = ks_err + arith
    err_S = np.abs(gS - oS)
    say(f"  S: max err {err_S.max():.3e}, max bound {s_err.max():.3e}")
    assert (err_S <= s_err).all()
    mean_err = s_err / np.maximum(oN, 1e-30)[..., None] + 8 * U32 * np.abs(ocb)
    M0, C = cfg.M0, cfg.C
    bound = mean_err.copy()
    for p in range(M0):
        kids = slice(M0 + p * C, M0 + (p + 1) * C)
        delta_err = mean_err[:, kids].sum(1) + C * mean_err[:, p] + 8 * U32 * C * np.abs(ocb[:, kids]).max(1)
        bound[:, kids] = mean_err[:, kids] + delta_err[:, None]
    err = np.abs(gcb - ocb)
    say(f"  codebook: max err {err.max():.3e}, max bound {bound.max():.3e}, max|C| {np.abs(ocb).max():.2f}")
    assert (err <= bound).all(), f"positions differ at {np.argwhere(err > bound)[:5]}"
    # the constraint holds on the GPU's positions to float rounding
    kids_mean = gcb[:, M0:].reshape(cfg.H, M0, C, cfg.d).mean(2, dtype=np.float64)
    cerr = np.abs(kids_mean - gcb[:, :M0]).max()
    say(f"  constraint: max|mean(children) - parent| = {cerr:.2e}")
    assert cerr <= 64 * U32 * np.abs(gcb).max()


@pytest.mark.parametrize("name,over", [("tiny", {}), ("grid64", {}), ("grid64", dict(d=128, H=2)),
                                       ("grid64", dict(M0=256, C=0, P=0)), ("tiny", dict(N=1000, C=16))])
def test_assign_aggregate_kv(name, over):
    """avq_assign_aggregate_kv: assignments and counts exact, value sums and
    key sums within the float32 summation bound of the oracle's sums."""
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS[name].replace(**over)
    data = gen.make(cfg, checker=oracle.MarginChecker())
    say(f"[kv] {cfg.name} {over} B{cfg.B} H{cfg.H} N{cfg.N} d{cfg.d} M0{cfg.M0} C{cfg.C} {cfg.dtype}")
    import torch
    K = to_device(data["K"], cfg.dtype, cfg.B, cfg.H)
    V = to_device(data["V"], cfg.dtype, cfg.B, cfg.H)
    cb = torch.from_numpy(data["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    vsum, counts, assign, ksum = _lib.assign_aggregate_kv(K, V, cb, cfg.C, want_assign=True)
    torch.cuda.synchronize()
    o = oracle.Oracle.for_cfg(cfg)
    parent, row = o.assign(data["K"], data["codebook"])
    assert np.array_equal(assign.cpu().numpy().reshape(cfg.BH, cfg.N), row)
    ov, oc = o.aggregate(data["V"], parent, row)
    ok, _ = o.aggregate(data["K"], parent, row)
    assert np.array_equal(counts.cpu().numpy().reshape(cfg.BH, cfg.Mt), oc)
    vabs, _ = o.aggregate(np.abs(data["V"].astype(np.float64)), parent, row)
    kabs, _ = o.aggregate(np.abs(data["K"].astype(np.float64)), parent, row)
    check_vsum(vsum.cpu().numpy().reshape(cfg.BH, cfg.Mt, cfg.d), ov, vabs, oc)
    check_vsum(ksum.cpu().numpy().reshape(cfg.BH, cfg.Mt, cfg.d), ok, kabs, oc)



def test_update_from_keys_d128_fused():
    """The fused key sums at d = 128 with 256 parents (the assign kernel's
    shared parent buffer), then the update, against the oracle."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = gen.CONFIGS["grid64"].replace(B=1, H=2, d=128, M0=256, N=2048 + 64 + 5, grid=None)
    data = gen.make(cfg, checker=oracle.MarginChecker())
    decay = 0.9
    say(f"[update] from keys d128 M0 256 fused")
    cb32 = data["codebook"].astype(np.float32)
    S0, N0 = cb32.copy(), np.ones((cfg.H, cfg.Mt), np.float32)
    dev = torch.device("cuda:0")
    K = torch.from_numpy(data["K"]).to(torch.bfloat16).reshape(cfg.B, cfg.H, cfg.N, cfg.d).contiguous().to(dev)
    V = torch.from_numpy(data["V"]).to(torch.bfloat16).reshape(K.shape).contiguous().to(dev)
    S, Nm, cb = (torch.from_numpy(a.copy()).to(dev) for a in (S0, N0, cb32))
    _, counts_g, _, ksum_g = _lib.assign_aggregate_kv(K, V, cb.to(torch.bfloat16).contiguous(), cfg.C)
    _lib.codebook_update(ksum_g, counts_g, S, Nm, cb, cfg.C, decay)
    torch.cuda.synchronize()
    o = oracle.Oracle.for_cfg(cfg)
    parent, row = o.assign(data["K"], data["codebook"])
    ksum, counts = o.aggregate(data["K"], parent, row)
    assert np.array_equal(counts_g.cpu().numpy().reshape(cfg.BH, cfg.Mt), counts)
    oS, oN, ocb = o.codebook_update(ksum, counts, float(np.float32(decay)), S0, N0, cb32)
    scale = np.abs(ocb).max()
    err = np.abs(cb.cpu().numpy() - ocb).max() / scale
    say(f"  codebook max err / max|C| = {err:.2e}")
    assert err <= 1e-5
    assert np.abs(Nm.cpu().numpy() - oN).max() <= 4 * U32 * (np.abs(oN).max() + 1.0)
