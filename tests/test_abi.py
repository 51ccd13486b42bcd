"""The C interface on the CPU: the library loads, exports every function
include/avq.h declares, and rejects bad arguments on the host before touching
the GPU (no HIP call is made on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "avq.h")


@pytest.fixture(scope="module")
def L():
    from adaptive_vector_quantized_amd import _lib
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    from adaptive_vector_quantized_amd import _lib
    names = _lib.declared_symbols()
    assert set(names) == {"avq_assign_aggregate", "avq_assign_aggregate_kv", "avq_attention_fwd", "avq_attention_fwd_approx",
                          "avq_attention_fwd_ordered", "avq_attention_workspace_size", "avq_codebook_update",
                          "avq_status_string", "avq_version"}
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (avq_\w+)", out))
    assert exported == set(names)


def test_version_and_strings(L):
    assert L.avq_version() == 100
    for code in range(0, -8, -1):
        assert L.avq_status_string(code)


def _buf(n=64):
    # 16-byte aligned host buffer; never dereferenced on the error paths
    b = ctypes.create_string_buffer(n + 16)
    addr = (ctypes.addressof(b) + 15) & ~15
    return b, ctypes.c_void_p(addr)


def _call_assign(L, kv=False, **kw):
    _, p = _buf()
    a = dict(K=p, V=p, cb=p, B=1, H=1, N=8, d=64, M0=4, C=2, dtype=1, vsum=p, counts=p, assign=None, ksum=p)
    a.update(kw)
    args = [a["K"], a["V"], a["cb"], a["B"], a["H"], a["N"], a["d"], a["M0"], a["C"], a["dtype"], a["vsum"],
            a["counts"], a["assign"]]
    if kv:
        return L.avq_assign_aggregate_kv(*args, a["ksum"], None)
    return L.avq_assign_aggregate(*args, None)


def _call_attn(L, fn="avq_attention_fwd", **kw):
    _, p = _buf()
    a = dict(Q=p, cb=p, vsum=p, counts=p, B=1, H=1, N=8, d=64, M0=4, C=2, dtype=1, P=2, bq=64, scale=0.125,
             Y=p, topp=None, imp=None, ws=p, wsb=1 << 30, order=p, approx=0)
    a.update(kw)
    if fn == "avq_attention_fwd_ordered":
        return L.avq_attention_fwd_ordered(a["Q"], a["cb"], a["vsum"], a["counts"], a["B"], a["H"], a["N"], a["d"],
                                           a["M0"], a["C"], a["dtype"], a["P"], a["bq"], a["scale"], a["order"],
                                           a["approx"], a["Y"], a["topp"], a["imp"], a["ws"], a["wsb"], None)
    return getattr(L, fn)(a["Q"], a["cb"], a["vsum"], a["counts"], a["B"], a["H"], a["N"], a["d"], a["M0"],
                          a["C"], a["dtype"], a["P"], a["bq"], a["scale"], a["Y"], a["topp"], a["imp"],
                          a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kv", [False, True])
def test_assign_validation(L, kv):
    _, p = _buf()
    mis = ctypes.c_void_p(p.value + 4)

    def _assign(L, **kw):  # both entry points validate the same way
        return _call_assign(L, kv, **kw)
    assert _assign(L, dtype=7) == -3
    assert _assign(L, N=-1) == -2
    assert _assign(L, B=-1) == -2
    assert _assign(L, C=-1) == -2
    assert _assign(L, M0=0) == -2
    assert _assign(L, d=96) == -5
    assert _assign(L, M0=513) == -5
    assert _assign(L, C=17) == -5
    assert _assign(L, K=None) == -1
    assert _assign(L, vsum=None) == -1
    assert _assign(L, counts=None) == -1
    assert _assign(L, cb=None) == -1
    assert _assign(L, K=mis) == -4
    assert _assign(L, assign=mis) == -4
    assert _assign(L, B=0) == 0       # no (batch, head): nothing to do, nothing launched
    assert _assign(L, H=0, K=None) == 0
    if kv:
        assert _assign(L, ksum=None) == -1
        assert _assign(L, ksum=mis) == -4


@pytest.mark.parametrize("fn", ["avq_attention_fwd", "avq_attention_fwd_approx", "avq_attention_fwd_ordered"])
def test_attention_validation(L, fn):
    _, p = _buf()
    mis = ctypes.c_void_p(p.value + 8)

    def _attn(L, **kw):  # both entry points validate the same way
        return _call_attn(L, fn=fn, **kw)
    assert _attn(L, P=-1) == -2
    assert _attn(L, P=5) == -2
    assert _attn(L, C=0, P=1) == -2  # a flat codebook has no children to refine with
    assert _attn(L, bq=48) == -5
    assert _attn(L, bq=256) == -5
    assert _attn(L, scale=float("nan")) == -2
    assert _attn(L, scale=float("inf")) == -2
    assert _attn(L, dtype=2) == -3
    assert _attn(L, d=32) == -5
    assert _attn(L, Q=None) == -1
    assert _attn(L, Y=None) == -1
    assert _attn(L, counts=None) == -1
    assert _attn(L, Y=mis) == -4
    assert _attn(L, topp=mis) == -4
    assert _attn(L, scale=0.0) == -2
    assert _attn(L, ws=None) == -1
    assert _attn(L, ws=mis) == -4
    need = L.avq_attention_workspace_size(1, 1, 64, 4, 2, 1)
    assert need > 0
    assert _attn(L, wsb=need - 1) == -7
    assert L.avq_attention_workspace_size(1, 1, 96, 4, 2, 1) == 0   # invalid sizes
    assert _attn(L, N=0) == 0         # no queries: nothing to do
    assert _attn(L, B=0, Q=None) == 0


def test_ordered_validation(L):
    _, p = _buf()

    def _attn(**kw):
        return _call_attn(L, fn="avq_attention_fwd_ordered", **kw)
    assert _attn(order=None) == -1                          # the order is required
    assert _attn(order=ctypes.c_void_p(p.value + 2)) == -4  # int32 entries: 4-byte aligned
    assert _attn(order=ctypes.c_void_p(p.value + 4), approx=1, P=9) == -2  # the rest as avq_attention_fwd
    assert _attn(N=0, order=None) == 0                      # no queries: nothing to do


def test_binding_fails_loudly_without_library(tmp_path):
    """The product path has no fallback: a missing library is an import error."""
    from adaptive_vector_quantized_amd import _lib
    with pytest.raises(ImportError):
        _lib._load(str(tmp_path / "missing.so"))


def test_codebook_update_validation(L):
    _, p = _buf()

    def upd(**kw):
        a = dict(ksum=p, counts=p, B=2, H=1, d=64, M0=4, C=2, decay=0.99, S=p, N=p, cb=p)
        a.update(kw)
        return L.avq_codebook_update(a["ksum"], a["counts"], a["B"], a["H"], a["d"], a["M0"], a["C"], a["decay"],
                                     a["S"], a["N"], a["cb"], None)
    assert upd(decay=-0.1) == -2
    assert upd(decay=1.5) == -2
    assert upd(decay=float("nan")) == -2
    assert upd(d=0) == -2
    assert upd(M0=0) == -2
    assert upd(C=-1) == -2
    assert upd(B=-1) == -2
    assert upd(C=17) == -5
    assert upd(S=None) == -1
    assert upd(N=None) == -1
    assert upd(cb=None) == -1
    assert upd(ksum=None) == -1
    assert upd(counts=ctypes.c_void_p(p.value + 2)) == -4
    assert upd(H=0, S=None) == 0      # no head: nothing to do
