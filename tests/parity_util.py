"""Helpers shared by the GPU parity tests: run the HIP path through the C
interface and the oracle on the same generator arrays, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from adaptive_vector_quantized_amd import gen

U32 = 2.0 ** -24  # unit roundoff of float32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray, dtype: str, B: int, H: int):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    t = t.reshape((B, H) + tuple(a.shape[1:])) if a.shape[0] == B * H else t
    return t.contiguous().cuda()


def run_gpu(data: dict, P: int, want_assign=True, want_topp=True, want_importance=True, bq=None,
            approx=False, order=None, y_fill=None, scale=None):
    """Both kernels through the C interface; returns numpy arrays shaped like the oracle's."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = data["cfg"]
    B, H = cfg.B, cfg.H
    bq = bq or cfg.block_q
    K = to_device(data["K"], cfg.dtype, B, H)
    V = to_device(data["V"], cfg.dtype, B, H)
    Q = to_device(data["Q"], cfg.dtype, B, H)
    cb = torch.from_numpy(data["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    vsum, counts, assign = _lib.assign_aggregate(K, V, cb, cfg.C, want_assign=want_assign)
    qo = None if order is None else torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda()
    Y = None
    if y_fill is not None:
        Y = torch.full((B, H, cfg.N, cfg.d), float(y_fill), dtype=torch.float32, device=Q.device)
    Y, topp, imp = _lib.attention_fwd(Q, cb, vsum, counts, cfg.C, P, bq, cfg.scale if scale is None else scale,
                                      want_topp=want_topp and P > 0, want_importance=want_importance,
                                      approx_denominator=approx, query_order=qo, Y=Y)
    torch.cuda.synchronize()
    BH = B * H
    out = {
        "vsum": vsum.cpu().numpy().reshape(BH, cfg.Mt, cfg.d),
        "counts": counts.cpu().numpy().reshape(BH, cfg.Mt),
        "Y": Y.cpu().numpy().reshape(BH, cfg.N, cfg.d),
    }
    if assign is not None:
        out["row"] = assign.cpu().numpy().reshape(BH, cfg.N)
    if topp is not None:
        out["sel"] = topp.cpu().numpy().reshape(BH, -1, P)
    if imp is not None:
        out["importance"] = imp.cpu().numpy().reshape(BH, -1, cfg.M0)
    return out


def y_tolerance(dtype: str) -> float:
    """Max-abs error allowed on the attention output, relative to its max-abs value."""
    return 1e-5 if dtype == "f32" else 2e-3


def check_vsum(g_vsum, o_vsum, o_abs, counts):
    """Float32 sums of n terms in any order: |error| <= gamma_n * sum|v| (the
    standard bound for recursive summation; the oracle sums in double)."""
    n = counts.astype(np.float64)[..., None]
    gamma = n * U32 / np.maximum(1.0 - n * U32, 1e-300)
    err = np.abs(g_vsum.astype(np.float64) - o_vsum)
    bound = gamma * o_abs + 1e-30
    bad = err > bound
    assert not bad.any(), f"value sums outside the float32 summation bound at {np.argwhere(bad)[:5]}"


def compare_y(g_Y, o_Y, dtype: str, where=""):
    scale = np.abs(o_Y).max()
    err = np.abs(g_Y.astype(np.float64) - o_Y).max()
    tol = y_tolerance(dtype)
    say(f"  Y {where}: max|err|/max|Y| = {err / scale:.3e} (tol {tol:g})")
    assert err <= tol * scale, f"Y mismatch {where}: {err / scale:.3e} > {tol:g}"
    return err / scale


def check_topp(g_sel, g_imp, w_ref, P: int, where=""):
    """Top-P sets on tiles whose reference decision is not drawn clear of ties,
    where several sets can be right: (1) the GPU's set is exactly the top-P of
    the GPU's own importances (larger first, equal ones to the lower index),
    and (2) against the double-precision reference importances every chosen
    parent is at least as important as every unchosen one, up to twice the
    largest importance error (if the GPU ranks by its own importances, a pair
    can only swap within that).  Returns the fraction of tiles whose set equals
    the reference's own top-P."""
    R = int(np.prod(w_ref.shape[:-1]))
    M0 = w_ref.shape[-1]
    g_sel = np.asarray(g_sel).reshape(R, P)
    g_imp = np.asarray(g_imp, np.float64).reshape(R, M0)
    w_ref = np.asarray(w_ref, np.float64).reshape(R, M0)
    own = np.sort(np.argsort(-g_imp, axis=-1, kind="stable")[:, :P], axis=-1)
    bad = np.argwhere((own != g_sel).any(-1))
    assert bad.size == 0, f"{where}: GPU set is not the top-P of its own importances at rows {bad[:5].ravel()}"
    chosen = np.zeros((R, M0), bool)
    np.put_along_axis(chosen, g_sel.astype(np.int64), True, axis=-1)
    tol = 2.0 * np.abs(g_imp - w_ref).max() + 1e-12
    lo = np.where(chosen, w_ref, np.inf).min(-1)
    hi = np.where(chosen, -np.inf, w_ref).max(-1)
    viol = np.argwhere(lo < hi - tol)
    assert viol.size == 0, f"{where}: chosen importance below an unchosen one at rows {viol[:5].ravel()}"
    ref = np.sort(np.argsort(-w_ref, axis=-1, kind="stable")[:, :P], axis=-1)
    same = float((ref == g_sel).all(-1).mean())
    say(f"  top-P valid on every tile (tol {tol:.2e}); equal to the reference set on {same * 100:.1f}%")
    return same


def sub_problem(data: dict, bh: int, t: int):
    """Queries of one tile of one (batch, head) as a stand-alone problem for the
    oracle's per-tile steps (importance, selection, output)."""
    cfg = data["cfg"]
    i0, i1 = t * cfg.block_q, min(cfg.N, (t + 1) * cfg.block_q)
    return data["Q"][bh:bh + 1, i0:i1], i0, i1


def run_attention_variants(data: dict, P: int, variants):
    """Kernel 1 once, then kernel 2 once per variant (keyword arguments of
    attention_fwd) on the same value sums and counts: the attention call is
    deterministic, so variants that must agree can be compared bit for bit
    (two runs of kernel 1 may round the value sums differently: they are
    float atomics added in any order)."""
    import torch
    from adaptive_vector_quantized_amd import _lib
    cfg = data["cfg"]
    K = to_device(data["K"], cfg.dtype, cfg.B, cfg.H)
    V = to_device(data["V"], cfg.dtype, cfg.B, cfg.H)
    Q = to_device(data["Q"], cfg.dtype, cfg.B, cfg.H)
    cb = torch.from_numpy(data["codebook"])
    cb = (cb.to(torch.bfloat16) if cfg.dtype == "bf16" else cb).contiguous().cuda()
    vsum, counts, _ = _lib.assign_aggregate(K, V, cb, cfg.C)
    outs = []
    for kw in variants:
        kw = dict(kw)
        if kw.get("query_order") is not None:
            kw["query_order"] = torch.from_numpy(np.ascontiguousarray(kw["query_order"], dtype=np.int32)).cuda()
        Y, topp, imp = _lib.attention_fwd(Q, cb, vsum, counts, cfg.C, P, cfg.block_q, cfg.scale,
                                          want_topp=P > 0, want_importance=True, **kw)
        torch.cuda.synchronize()
        outs.append({"Y": Y.cpu().numpy(), "sel": None if topp is None else topp.cpu().numpy(),
                     "importance": imp.cpu().numpy()})
    return outs
