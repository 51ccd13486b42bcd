"""ctypes binding of libavq (include/avq.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libavq.so.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libavq.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "avq.h")

AVQ_F32 = 0
AVQ_BF16 = 1
STATUS = {0: "AVQ_OK", -1: "AVQ_ERR_NULL", -2: "AVQ_ERR_SHAPE", -3: "AVQ_ERR_DTYPE", -4: "AVQ_ERR_ALIGN",
          -5: "AVQ_ERR_UNSUPPORTED", -6: "AVQ_ERR_HIP", -7: "AVQ_ERR_WORKSPACE", -8: "AVQ_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 8 << 20  # AVQ_NOALLOC_SCRATCH_BYTES


class AvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib.avq_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{what}: {STATUS.get(status, status)} ({msg})")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libavq.so not found at {path}; build it with __graft_entry__.build() "
                          "or python adaptive_vector_quantized_amd/build.py")
    lib = ctypes.CDLL(path)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.avq_assign_aggregate.argtypes = [P, P, P] + [i32] * 7 + [P, P, P, P]
    lib.avq_assign_aggregate.restype = i32
    lib.avq_assign_aggregate_kv.argtypes = [P, P, P] + [i32] * 7 + [P, P, P, P, P]
    lib.avq_assign_aggregate_kv.restype = i32
    for f in (lib.avq_attention_fwd, lib.avq_attention_fwd_approx):
        f.argtypes = [P, P, P, P] + [i32] * 7 + [i32, i32, f32, P, P, P, P, ctypes.c_size_t, P]
        f.restype = i32
    lib.avq_attention_fwd_ordered.argtypes = [P, P, P, P] + [i32] * 7 + [i32, i32, f32, P, i32, P, P, P, P,
                                                                      ctypes.c_size_t, P]
    lib.avq_attention_fwd_ordered.restype = i32
    lib.avq_attention_fwd_noalloc.argtypes = [P, P, P, P] + [i32] * 7 + [i32, i32, f32, P, P, P, P]
    lib.avq_attention_fwd_noalloc.restype = i32
    lib.avq_assign_aggregate_accum.argtypes = [P, P, P] + [i32] * 7 + [P, P, P, P]
    lib.avq_assign_aggregate_accum.restype = i32
    lib.avq_attention_prepare.argtypes = [P, P] + [i32] * 6 + [P, ctypes.c_size_t, P]
    lib.avq_attention_prepare.restype = i32
    lib.avq_attention_fwd_prepared.argtypes = [P, P] + [i32] * 7 + [i32, i32, f32, P, P, P, P, ctypes.c_size_t,
                                                                  P, P, P]
    lib.avq_attention_fwd_prepared.restype = i32
    lib.avq_codebook_update.argtypes = [P, P] + [i32] * 5 + [f32, P, P, P, P]
    lib.avq_codebook_update.restype = i32
    lib.avq_attention_workspace_size.argtypes = [i32] * 6
    lib.avq_attention_workspace_size.restype = ctypes.c_size_t
    lib.avq_status_string.argtypes = [i32]
    lib.avq_status_string.restype = ctypes.c_char_p
    lib.avq_version.argtypes = []
    lib.avq_version.restype = i32
    return lib


_lib: Optional[ctypes.CDLL] = None
_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def declared_symbols(header: str = HEADER):
    """Names of the functions include/avq.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(avq_\w+)\s*\(", text, flags=re.M)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return AVQ_F32
    if t.dtype == torch.bfloat16:
        return AVQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


# The C interface sees only pointers and sizes, so the binding is where every
# tensor is checked against the sizes it will be read or written with: dtype,
# shape and layout of every tensor first, then (_on_device) that all of them
# are device memory on the device of the call's first tensor.
def _check(t, name: str, shape, dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_device(named):
    """named: (name, tensor or None) pairs; the first tensor's device is the call's."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call runs on {dev}")


def _shape4(t: torch.Tensor, name: str) -> Tuple[int, int, int, int]:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    _dtype_code(t)
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    return tuple(t.shape)


def _codebook_rows(codebook, H: int, d: int, dtype, C: int) -> Tuple[int, int]:
    """(Mt, M0) of a [H, M0 * (1 + C), d] codebook in the activations' dtype."""
    if not isinstance(C, int) or C < 0:
        raise ValueError(f"C must be a non-negative int, got {C!r}")
    if not isinstance(codebook, torch.Tensor) or codebook.dim() != 3:
        raise ValueError("codebook must be an [H, M0 * (1 + C), d] tensor")
    Mt = int(codebook.shape[1])
    _check(codebook, "codebook", (H, Mt, d), dtype)
    if Mt == 0 or Mt % (1 + C):
        raise ValueError(f"codebook rows ({Mt}) must be M0 * (1 + C) with M0 >= 1, C = {C}")
    return Mt, Mt // (1 + C)


def _assign_args(K, V, codebook, C, vsum, counts, assign, ksum, want_assign, with_keys):
    B, H, N, d = _shape4(K, "K")
    dev = K.device
    _check(V, "V", (B, H, N, d), K.dtype)
    Mt, M0 = _codebook_rows(codebook, H, d, K.dtype, C)
    for name, t, shape in (("vsum", vsum, (B, H, Mt, d)), ("counts", counts, (B, H, Mt)),
                           ("assign", assign, (B, H, N)), ("ksum", ksum if with_keys else None, (B, H, Mt, d))):
        if t is not None:
            _check(t, name, shape, torch.int32 if name in ("counts", "assign") else torch.float32)
    _on_device([("K", K), ("V", V), ("codebook", codebook), ("vsum", vsum), ("counts", counts),
                ("assign", assign), ("ksum", ksum if with_keys else None)])
    if vsum is None:
        vsum = torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty((B, H, Mt), dtype=torch.int32, device=dev)
    if want_assign and assign is None:
        assign = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    if with_keys and ksum is None:
        ksum = torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev)
    return (B, H, N, d, M0), vsum, counts, assign, ksum


def assign_aggregate(K: torch.Tensor, V: torch.Tensor, codebook: torch.Tensor, C: int, *,
                     want_assign: bool = False, vsum: Optional[torch.Tensor] = None,
                     counts: Optional[torch.Tensor] = None, assign: Optional[torch.Tensor] = None):
    """Kernel 1.  K, V: [B, H, N, d]; codebook: [H, M0*(1+C), d] (same dtype).
    Returns (vsum [B, H, Mt, d] float32, counts [B, H, Mt] int32, assign [B, H, N] int32 or None)."""
    (B, H, N, d, M0), vsum, counts, assign, _ = _assign_args(K, V, codebook, C, vsum, counts, assign, None,
                                                            want_assign, False)
    rc = _lib.avq_assign_aggregate(_ptr(K), _ptr(V), _ptr(codebook), B, H, N, d, M0, C, _dtype_code(K),
                                   _ptr(vsum), _ptr(counts), _ptr(assign), _stream(K))
    if rc != 0:
        raise AvqError(rc, "avq_assign_aggregate")
    return vsum, counts, assign


def assign_aggregate_accum(K: torch.Tensor, V: torch.Tensor, codebook: torch.Tensor, C: int, *,
                           vsum: torch.Tensor, counts: torch.Tensor, assign: Optional[torch.Tensor] = None):
    """avq_assign_aggregate_accum: kernel 1 adding this batch's value sums and counts to vsum and
    counts (given, [B, H, Mt, d] float32 and [B, H, Mt] int32; no zero fill).  Returns (vsum,
    counts, assign or None)."""
    if vsum is None or counts is None:
        raise ValueError("vsum and counts are accumulated into: both must be given")
    (B, H, N, d, M0), vsum, counts, assign, _ = _assign_args(K, V, codebook, C, vsum, counts, assign, None,
                                                            assign is not None, False)
    rc = _lib.avq_assign_aggregate_accum(_ptr(K), _ptr(V), _ptr(codebook), B, H, N, d, M0, C, _dtype_code(K),
                                         _ptr(vsum), _ptr(counts), _ptr(assign), _stream(K))
    if rc != 0:
        raise AvqError(rc, "avq_assign_aggregate_accum")
    return vsum, counts, assign


def assign_aggregate_kv(K: torch.Tensor, V: torch.Tensor, codebook: torch.Tensor, C: int, *,
                        want_assign: bool = False, vsum: Optional[torch.Tensor] = None,
                        counts: Optional[torch.Tensor] = None, assign: Optional[torch.Tensor] = None,
                        ksum: Optional[torch.Tensor] = None):
    """Kernel 1 with the keys also summed per codeword (for codebook_update), in one pass.
    Returns (vsum, counts, assign or None, ksum [B, H, Mt, d] float32)."""
    (B, H, N, d, M0), vsum, counts, assign, ksum = _assign_args(K, V, codebook, C, vsum, counts, assign, ksum,
                                                               want_assign, True)
    rc = _lib.avq_assign_aggregate_kv(_ptr(K), _ptr(V), _ptr(codebook), B, H, N, d, M0, C, _dtype_code(K),
                                      _ptr(vsum), _ptr(counts), _ptr(assign), _ptr(ksum), _stream(K))
    if rc != 0:
        raise AvqError(rc, "avq_assign_aggregate_kv")
    return vsum, counts, assign, ksum


def workspace_size(B: int, H: int, d: int, M0: int, C: int, dtype: torch.dtype) -> int:
    return int(_lib.avq_attention_workspace_size(B, H, d, M0, C, AVQ_BF16 if dtype == torch.bfloat16 else AVQ_F32))


def attention_fwd(Q: torch.Tensor, codebook: torch.Tensor, vsum: torch.Tensor, counts: torch.Tensor, C: int, P: int,
                  block_q: int, scale: Optional[float] = None, *, want_topp: bool = False,
                  want_importance: bool = False, Y: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, approx_denominator: bool = False,
                  query_order: Optional[torch.Tensor] = None):
    """Kernel 2.  Q: [B, H, N, d]; codebook [H, Mt, d]; vsum/counts from assign_aggregate.
    Returns (Y [B, H, N, d] float32, topp [B, H, T, P] int32 or None, importance [B, H, T, M0] or None).
    ``workspace`` (uint8 device tensor) is allocated here when not given.  ``approx_denominator``
    selects avq_attention_fwd_approx (importances per 64-parent tile, App. B Eq. 13-14).
    ``query_order`` (int32 [N] device tensor, a permutation of the token rows, e.g.
    ``gilbert.query_order``) selects avq_attention_fwd_ordered: tile t holds the
    queries of rows query_order[t*block_q ...]; Y stays in the row order of Q."""
    B, H, N, d = _shape4(Q, "Q")
    dev = Q.device
    Mt, M0 = _codebook_rows(codebook, H, d, Q.dtype, C)
    _check(vsum, "vsum", (B, H, Mt, d), torch.float32)
    _check(counts, "counts", (B, H, Mt), torch.int32)
    if Y is not None:
        _check(Y, "Y", (B, H, N, d), torch.float32)
    if workspace is not None:
        _check(workspace, "workspace", None, torch.uint8)
    if query_order is not None:
        _check(query_order, "query_order", (N,), torch.int32)
    _on_device([("Q", Q), ("codebook", codebook), ("vsum", vsum), ("counts", counts), ("Y", Y),
                ("workspace", workspace), ("query_order", query_order)])
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    T = (N + block_q - 1) // block_q if block_q > 0 else 0
    if Y is None:
        Y = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    topp = torch.empty((B, H, T, P), dtype=torch.int32, device=dev) if want_topp else None
    imp = torch.empty((B, H, T, M0), dtype=torch.float32, device=dev) if want_importance else None
    need = workspace_size(B, H, d, M0, C, Q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel()
    if query_order is not None:
        name = "avq_attention_fwd_ordered"
        rc = _lib.avq_attention_fwd_ordered(_ptr(Q), _ptr(codebook), _ptr(vsum), _ptr(counts), B, H, N, d, M0, C,
                                            _dtype_code(Q), P, block_q, float(scale), _ptr(query_order),
                                            1 if approx_denominator else 0, _ptr(Y), _ptr(topp), _ptr(imp),
                                            _ptr(workspace), ws_bytes, _stream(Q))
    else:
        fn, name = ((_lib.avq_attention_fwd_approx, "avq_attention_fwd_approx") if approx_denominator
                    else (_lib.avq_attention_fwd, "avq_attention_fwd"))
        rc = fn(_ptr(Q), _ptr(codebook), _ptr(vsum), _ptr(counts), B, H, N, d, M0, C,
                _dtype_code(Q), P, block_q, float(scale), _ptr(Y), _ptr(topp), _ptr(imp),
                _ptr(workspace), ws_bytes, _stream(Q))
    if rc != 0:
        raise AvqError(rc, name)
    return Y, topp, imp


def attention_prepare(vsum: torch.Tensor, counts: torch.Tensor, C: int, dtype: torch.dtype, *,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """avq_attention_prepare: the value-sum operands of kernel 2 (Eq. 6 and 9) and a copy of the
    counts for this batch's aggregates, written to ``workspace`` (uint8 device tensor, allocated
    here when not given) and returned for attention_fwd_prepared.  ``dtype`` is the dtype of the
    queries and codebook."""
    if not isinstance(vsum, torch.Tensor) or vsum.dim() != 4:
        raise ValueError("vsum must be a float32 [B, H, Mt, d] tensor")
    B, H, Mt, d = (int(x) for x in vsum.shape)
    _check(vsum, "vsum", (B, H, Mt, d), torch.float32)
    _check(counts, "counts", (B, H, Mt), torch.int32)
    if not isinstance(C, int) or C < 0 or Mt == 0 or Mt % (1 + C):
        raise ValueError(f"codeword rows ({Mt}) must be M0 * (1 + C) with C >= 0, C = {C!r}")
    if dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    M0 = Mt // (1 + C)
    if workspace is not None:
        _check(workspace, "workspace", None, torch.uint8)
    _on_device([("vsum", vsum), ("counts", counts), ("workspace", workspace)])
    need = workspace_size(B, H, d, M0, C, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=vsum.device)
    rc = _lib.avq_attention_prepare(_ptr(vsum), _ptr(counts), B, H, d, M0, C,
                                    AVQ_BF16 if dtype == torch.bfloat16 else AVQ_F32, _ptr(workspace),
                                    workspace.numel(), _stream(vsum))
    if rc != 0:
        raise AvqError(rc, "avq_attention_prepare")
    return workspace


def attention_fwd_prepared(Q: torch.Tensor, codebook: torch.Tensor, workspace: torch.Tensor, C: int, P: int,
                           block_q: int, scale: Optional[float] = None, *, want_topp: bool = False,
                           want_importance: bool = False, Y: Optional[torch.Tensor] = None,
                           topp: Optional[torch.Tensor] = None, importance: Optional[torch.Tensor] = None,
                           clear_vsum: Optional[torch.Tensor] = None, clear_counts: Optional[torch.Tensor] = None):
    """avq_attention_fwd_prepared: the attention kernel alone, on a workspace that attention_prepare
    filled for the same aggregates.  Returns (Y, topp or None, importance or None) like attention_fwd;
    outputs given as tensors are written in place (nothing is allocated then).  ``clear_vsum`` /
    ``clear_counts`` ([B, H, Mt, d] float32 / [B, H, Mt] int32) are zero-filled by the call."""
    B, H, N, d = _shape4(Q, "Q")
    dev = Q.device
    Mt, M0 = _codebook_rows(codebook, H, d, Q.dtype, C)
    T = (N + block_q - 1) // block_q if block_q > 0 else 0
    _check(workspace, "workspace", None, torch.uint8)
    for name, t, shape, dt in (("Y", Y, (B, H, N, d), torch.float32), ("topp", topp, (B, H, T, P), torch.int32),
                               ("importance", importance, (B, H, T, M0), torch.float32),
                               ("clear_vsum", clear_vsum, (B, H, Mt, d), torch.float32),
                               ("clear_counts", clear_counts, (B, H, Mt), torch.int32)):
        if t is not None:
            _check(t, name, shape, dt)
    _on_device([("Q", Q), ("codebook", codebook), ("workspace", workspace), ("Y", Y), ("topp", topp),
                ("importance", importance), ("clear_vsum", clear_vsum), ("clear_counts", clear_counts)])
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if Y is None:
        Y = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    if topp is None and want_topp:
        topp = torch.empty((B, H, T, P), dtype=torch.int32, device=dev)
    if importance is None and want_importance:
        importance = torch.empty((B, H, T, M0), dtype=torch.float32, device=dev)
    rc = _lib.avq_attention_fwd_prepared(_ptr(Q), _ptr(codebook), B, H, N, d, M0, C, _dtype_code(Q), P, block_q,
                                         float(scale), _ptr(Y), _ptr(topp), _ptr(importance), _ptr(workspace),
                                         workspace.numel(), _ptr(clear_vsum), _ptr(clear_counts), _stream(Q))
    if rc != 0:
        raise AvqError(rc, "avq_attention_fwd_prepared")
    return Y, topp, importance


def attention_fwd_noalloc(Q: torch.Tensor, codebook: torch.Tensor, vsum: torch.Tensor, counts: torch.Tensor, C: int,
                          P: int, block_q: int, scale: Optional[float] = None, *, Y: torch.Tensor,
                          topp: Optional[torch.Tensor] = None, importance: Optional[torch.Tensor] = None):
    """avq_attention_fwd_noalloc: kernel 2 with its operands in the library's static scratch (no
    workspace).  Every output is caller-provided (Y [B, H, N, d] float32; topp [B, H, T, P] int32 and
    importance [B, H, T, M0] float32, or None), so this call allocates nothing."""
    B, H, N, d = _shape4(Q, "Q")
    Mt, M0 = _codebook_rows(codebook, H, d, Q.dtype, C)
    T = (N + block_q - 1) // block_q if block_q > 0 else 0
    _check(vsum, "vsum", (B, H, Mt, d), torch.float32)
    _check(counts, "counts", (B, H, Mt), torch.int32)
    _check(Y, "Y", (B, H, N, d), torch.float32)
    if topp is not None:
        _check(topp, "topp", (B, H, T, P), torch.int32)
    if importance is not None:
        _check(importance, "importance", (B, H, T, M0), torch.float32)
    _on_device([("Q", Q), ("codebook", codebook), ("vsum", vsum), ("counts", counts), ("Y", Y), ("topp", topp),
                ("importance", importance)])
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    rc = _lib.avq_attention_fwd_noalloc(_ptr(Q), _ptr(codebook), _ptr(vsum), _ptr(counts), B, H, N, d, M0, C,
                                        _dtype_code(Q), P, block_q, float(scale), _ptr(Y), _ptr(topp),
                                        _ptr(importance), _stream(Q))
    if rc != 0:
        raise AvqError(rc, "avq_attention_fwd_noalloc")
    return Y, topp, importance


def forward(Q, K, V, codebook, C: int, P: int, block_q: int, scale: Optional[float] = None):
    """The whole AVQ-Attention forward pass: kernel 1 then kernel 2 on the current stream."""
    vsum, counts, _ = assign_aggregate(K, V, codebook, C)
    Y, _, _ = attention_fwd(Q, codebook, vsum, counts, C, P, block_q, scale)
    return Y


def codebook_update(ksum: torch.Tensor, counts: torch.Tensor, S: torch.Tensor, Nema: torch.Tensor,
                    codebook: torch.Tensor, C: int, decay: float):
    """Codebook update step (App. A, Eq. 11-12), in place on S [H, Mt, d], Nema [H, Mt] and
    codebook [H, Mt, d] (all float32).  ksum [B, H, Mt, d] float32 and counts [B, H, Mt] int32 are
    this batch's per-codeword key sums and counts: assign_aggregate(K, K, ...)."""
    if not isinstance(ksum, torch.Tensor) or ksum.dim() != 4:
        raise ValueError("ksum must be a float32 [B, H, Mt, d] tensor")
    B, H, Mt, d = (int(x) for x in ksum.shape)
    _check(ksum, "ksum", (B, H, Mt, d), torch.float32)
    if not isinstance(C, int) or C < 0:
        raise ValueError(f"C must be a non-negative int, got {C!r}")
    if Mt == 0 or Mt % (1 + C):
        raise ValueError("codeword rows must be M0 * (1 + C)")
    M0 = Mt // (1 + C)
    _check(counts, "counts", (B, H, Mt), torch.int32)
    for name, t, shape in (("S", S, (H, Mt, d)), ("Nema", Nema, (H, Mt)), ("codebook", codebook, (H, Mt, d))):
        _check(t, name, shape, torch.float32)
    _on_device([("ksum", ksum), ("counts", counts), ("S", S), ("Nema", Nema), ("codebook", codebook)])
    rc = _lib.avq_codebook_update(_ptr(ksum), _ptr(counts), B, H, d, M0, C, float(decay), _ptr(S), _ptr(Nema),
                                  _ptr(codebook), _stream(S))
    if rc != 0:
        raise AvqError(rc, "avq_codebook_update")
    return S, Nema, codebook


def update_codebook(K: torch.Tensor, codebook: torch.Tensor, S: torch.Tensor, Nema: torch.Tensor, C: int,
                    decay: float):
    """One training step of the codebook from the keys K [B, H, N, d]: the keys are assigned and
    summed per codeword against the codebook rounded to K's dtype (assign_aggregate with V = K),
    then codebook_update moves the float32 positions in place.  Returns (S, Nema, codebook)."""
    cb_in = codebook if K.dtype == torch.float32 else codebook.to(K.dtype).contiguous()
    ksum, counts, _ = assign_aggregate(K, K, cb_in, C)
    return codebook_update(ksum, counts, S, Nema, codebook, C, decay)
