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
    assert set(names) == {"avq_assign_aggregate", "avq_assign_aggregate_kv", "avq_assign_aggregate_accum",
                          "avq_attention_fwd", "avq_attention_fwd_approx",
                          "avq_attention_fwd_ordered", "avq_attention_fwd_noalloc", "avq_attention_prepare",
                          "avq_attention_fwd_prepared", "avq_attention_workspace_size",
                          "avq_codebook_update", "avq_status_string", "avq_version"}
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (avq_\w+)", out))
    assert exported == set(names)


def test_version_and_strings(L):
    assert L.avq_version() == 100
    for code in range(0, -9, -1):
        assert L.avq_status_string(code) != b"unknown status"


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
    if kv == "accum":
        return L.avq_assign_aggregate_accum(*args, None)
    if kv:
        return L.avq_assign_aggregate_kv(*args, a["ksum"], None)
    return L.avq_assign_aggregate(*args, None)


def _call_attn(L, fn="avq_attention_fwd", **kw):
    _, p = _buf()
    a = dict(Q=p, cb=p, vsum=p, counts=p, B=1, H=1, N=8, d=64, M0=4, C=2, dtype=1, P=2, bq=64, scale=0.125,
             Y=p, topp=None, imp=None, ws=p, wsb=1 << 30, order=p, approx=0)
    a.update(kw)
    if fn == "avq_attention_fwd_noalloc":
        return L.avq_attention_fwd_noalloc(a["Q"], a["cb"], a["vsum"], a["counts"], a["B"], a["H"], a["N"], a["d"],
                                           a["M0"], a["C"], a["dtype"], a["P"], a["bq"], a["scale"], a["Y"],
                                           a["topp"], a["imp"], None)
    if fn == "avq_attention_fwd_prepared":
        return L.avq_attention_fwd_prepared(a["Q"], a["cb"], a["B"], a["H"], a["N"], a["d"], a["M0"], a["C"],
                                            a["dtype"], a["P"], a["bq"], a["scale"], a["Y"], a["topp"], a["imp"],
                                            a["ws"], a["wsb"], a.get("cv"), a.get("cc"), None)
    if fn == "avq_attention_fwd_ordered":
        return L.avq_attention_fwd_ordered(a["Q"], a["cb"], a["vsum"], a["counts"], a["B"], a["H"], a["N"], a["d"],
                                           a["M0"], a["C"], a["dtype"], a["P"], a["bq"], a["scale"], a["order"],
                                           a["approx"], a["Y"], a["topp"], a["imp"], a["ws"], a["wsb"], None)
    return getattr(L, fn)(a["Q"], a["cb"], a["vsum"], a["counts"], a["B"], a["H"], a["N"], a["d"], a["M0"],
                          a["C"], a["dtype"], a["P"], a["bq"], a["scale"], a["Y"], a["topp"], a["imp"],
                          a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kv", [False, True, "accum"])
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
    if kv is True:
        assert _assign(L, ksum=None) == -1
        assert _assign(L, ksum=mis) == -4


@pytest.mark.parametrize("fn", ["avq_attention_fwd", "avq_attention_fwd_approx", "avq_attention_fwd_ordered",
                                "avq_attention_fwd_noalloc", "avq_attention_fwd_prepared"])
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
    if fn != "avq_attention_fwd_prepared":  # (the prepared call reads the workspace's copy of the counts)
        assert _attn(L, counts=None) == -1
    else:
        assert _attn(L, cv=mis) == -4
        assert _attn(L, cc=ctypes.c_void_p(p.value + 4)) == -4
    assert _attn(L, Y=mis) == -4
    assert _attn(L, topp=mis) == -4
    assert _attn(L, scale=0.0) == -2
    if fn != "avq_attention_fwd_noalloc":
        assert _attn(L, ws=None) == -1
        assert _attn(L, ws=mis) == -4
        need = L.avq_attention_workspace_size(1, 1, 64, 4, 2, 1)
        assert need > 0
        assert _attn(L, wsb=need - 1) == -7
    else:
        # beyond the static scratch: refused before anything is launched
        need = L.avq_attention_workspace_size(1, 200, 64, 64, 8, 1)
        assert need > (8 << 20)
        assert _attn(L, H=200, M0=64, C=8, P=16, bq=128) == -8
        assert L.avq_attention_workspace_size(1, 110, 64, 64, 8, 1) <= (8 << 20)
    assert L.avq_attention_workspace_size(1, 1, 96, 4, 2, 1) == 0   # invalid sizes
    assert _attn(L, N=0) == 0         # no queries: nothing to do
    assert _attn(L, B=0, Q=None) == 0


def test_prepare_validation(L):
    """avq_attention_prepare checks the sizes, the value sums, the counts and
    the workspace (it reads nothing else)."""
    _, p = _buf()
    mis = ctypes.c_void_p(p.value + 8)

    def _prep(**kw):
        a = dict(vsum=p, counts=p, B=1, H=1, d=64, M0=4, C=2, dtype=1, ws=p, wsb=1 << 30)
        a.update(kw)
        return L.avq_attention_prepare(a["vsum"], a["counts"], a["B"], a["H"], a["d"], a["M0"], a["C"], a["dtype"],
                                       a["ws"], a["wsb"], None)
    assert _prep(dtype=2) == -3
    assert _prep(B=-1) == -2
    assert _prep(M0=0) == -2
    assert _prep(C=-1) == -2
    assert _prep(d=32) == -5
    assert _prep(M0=513) == -5
    assert _prep(vsum=None) == -1
    assert _prep(counts=None) == -1
    assert _prep(ws=None) == -1
    assert _prep(counts=ctypes.c_void_p(p.value + 4)) == -4
    assert _prep(vsum=mis) == -4
    assert _prep(ws=mis) == -4
    need = L.avq_attention_workspace_size(1, 1, 64, 4, 2, 1)
    assert _prep(wsb=need - 1) == -7
    assert _prep(B=0, vsum=None) == 0   # no (batch, head): nothing to do


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


# ---- the Python binding's checks (CPU tensors: every structural mismatch is
# reported before the device check, and a tensor that is not GPU memory is
# refused; nothing reaches the C interface) --------------------------------
def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _assign_inputs(dtype=None):
    import torch
    dt = dtype or torch.bfloat16
    B, H, N, d, M0, C = 1, 2, 40, 64, 4, 2
    Mt = M0 * (1 + C)
    return dict(K=_t((B, H, N, d), dt), V=_t((B, H, N, d), dt), codebook=_t((H, Mt, d), dt), C=C), (B, H, N, d, Mt)


@pytest.mark.parametrize("kv", [False, True])
def test_binding_assign_checks(kv):
    import torch
    from adaptive_vector_quantized_amd import _lib
    fn = _lib.assign_aggregate_kv if kv else _lib.assign_aggregate
    a, (B, H, N, d, Mt) = _assign_inputs()
    cases = [
        (dict(V=_t((B, H, N, d), torch.float32)), TypeError, "V must be torch.bfloat16"),
        (dict(V=_t((B, H, N + 1, d), torch.bfloat16)), ValueError, "V must have shape"),
        (dict(codebook=_t((H, Mt, d), torch.float32)), TypeError, "codebook must be torch.bfloat16"),
        (dict(codebook=_t((H + 1, Mt, d), torch.bfloat16)), ValueError, "codebook must have shape"),
        (dict(codebook=_t((H, Mt + 1, d), torch.bfloat16)), ValueError, "must be M0 * (1 + C)"),
        (dict(C=-1), ValueError, "C must be"),
        (dict(K=_t((B, H, N, d), torch.float16)), TypeError, "unsupported dtype"),
        (dict(K=_t((B, H, d, N), torch.bfloat16).transpose(2, 3)), ValueError, "contiguous"),
        (dict(vsum=_t((B, H, Mt, d), torch.bfloat16)), TypeError, "vsum must be torch.float32"),
        (dict(vsum=_t((B, H, Mt - 1, d), torch.float32)), ValueError, "vsum must have shape"),
        (dict(counts=_t((B, H, Mt), torch.int64)), TypeError, "counts must be torch.int32"),
        (dict(counts=_t((B, H, Mt + 3), torch.int32)), ValueError, "counts must have shape"),
        (dict(assign=_t((B, H, N - 1), torch.int32)), ValueError, "assign must have shape"),
        ({}, ValueError, "must be a GPU tensor"),
    ]
    if kv:
        cases.append((dict(ksum=_t((B, H, Mt, d + 1), torch.float32)), ValueError, "ksum must have shape"))
    for over, exc, msg in cases:
        kw = dict(a, **over)
        with pytest.raises(exc, match=re.escape(msg)):
            fn(kw.pop("K"), kw.pop("V"), kw.pop("codebook"), kw.pop("C"), **kw)


def test_binding_attention_checks():
    import torch
    from adaptive_vector_quantized_amd import _lib
    B, H, N, d, M0, C = 1, 2, 40, 64, 4, 2
    Mt = M0 * (1 + C)
    base = dict(Q=_t((B, H, N, d), torch.bfloat16), codebook=_t((H, Mt, d), torch.bfloat16),
                vsum=_t((B, H, Mt, d), torch.float32), counts=_t((B, H, Mt), torch.int32))
    cases = [
        (dict(codebook=_t((H, Mt, d), torch.float32)), TypeError, "codebook must be torch.bfloat16"),
        (dict(codebook=_t((H, Mt, d + 64), torch.bfloat16)), ValueError, "codebook must have shape"),
        (dict(codebook=_t((H, Mt + 2, d), torch.bfloat16)), ValueError, "must be M0 * (1 + C)"),
        (dict(vsum=_t((B, H, Mt, d), torch.bfloat16)), TypeError, "vsum must be torch.float32"),
        (dict(vsum=_t((B, H + 1, Mt, d), torch.float32)), ValueError, "vsum must have shape"),
        (dict(counts=_t((B, H, Mt), torch.float32)), TypeError, "counts must be torch.int32"),
        (dict(counts=_t((B, H, Mt, 1), torch.int32)), ValueError, "counts must have shape"),
        (dict(Y=_t((B, H, N, d), torch.bfloat16)), TypeError, "Y must be torch.float32"),
        (dict(Y=_t((B, H, N - 1, d), torch.float32)), ValueError, "Y must have shape"),
        (dict(workspace=_t((64,), torch.float32)), TypeError, "workspace must be torch.uint8"),
        (dict(query_order=_t((N,), torch.int64)), TypeError, "query_order must be torch.int32"),
        (dict(query_order=_t((N + 1,), torch.int32)), ValueError, "query_order must have shape"),
        ({}, ValueError, "must be a GPU tensor"),
    ]
    for over, exc, msg in cases:
        kw = dict(base, **over)
        with pytest.raises(exc, match=re.escape(msg)):
            _lib.attention_fwd(kw.pop("Q"), kw.pop("codebook"), kw.pop("vsum"), kw.pop("counts"), C, 2, 64, **kw)


def test_binding_update_checks():
    import torch
    from adaptive_vector_quantized_amd import _lib
    B, H, d, M0, C = 2, 2, 64, 4, 2
    Mt = M0 * (1 + C)
    base = dict(ksum=_t((B, H, Mt, d), torch.float32), counts=_t((B, H, Mt), torch.int32),
                S=_t((H, Mt, d), torch.float32), Nema=_t((H, Mt), torch.float32), codebook=_t((H, Mt, d), torch.float32))
    cases = [
        (dict(ksum=_t((B, H, Mt, d), torch.bfloat16)), TypeError, "ksum must be torch.float32"),
        (dict(counts=_t((B, H, Mt - 1), torch.int32)), ValueError, "counts must have shape"),
        (dict(S=_t((H, Mt, d), torch.bfloat16)), TypeError, "S must be torch.float32"),
        (dict(Nema=_t((H, Mt + 1), torch.float32)), ValueError, "Nema must have shape"),
        (dict(codebook=_t((H, Mt, d), torch.bfloat16)), TypeError, "codebook must be torch.float32"),
        ({}, ValueError, "must be a GPU tensor"),
    ]
    for over, exc, msg in cases:
        kw = dict(base, **over)
        with pytest.raises(exc, match=re.escape(msg)):
            _lib.codebook_update(kw["ksum"], kw["counts"], kw["S"], kw["Nema"], kw["codebook"], C, 0.9)
