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
          -5: "AVQ_ERR_UNSUPPORTED", -6: "AVQ_ERR_HIP", -7: "AVQ_ERR_WORKSPACE"}


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


def _shape4(t: torch.Tensor, name: str) -> Tuple[int, int, int, int]:
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    return tuple(t.shape)


def assign_aggregate(K: torch.Tensor, V: torch.Tensor, codebook: torch.Tensor, C: int, *,
                     want_assign: bool = False, vsum: Optional[torch.Tensor] = None,
                     counts: Optional[torch.Tensor] = None, assign: Optional[torch.Tensor] = None):
    """Kernel 1.  K, V: [B, H, N, d]; codebook: [H, M0*(1+C), d] (same dtype).
    Returns (vsum [B, H, Mt, d] float32, counts [B, H, Mt] int32, assign [B, H, N] int32 or None)."""
    B, H, N, d = _shape4(K, "K")
    if tuple(V.shape) != (B, H, N, d) or V.dtype != K.dtype or not V.is_contiguous():
        raise ValueError("V must match K")
    if codebook.dim() != 3 or codebook.shape[0] != H or codebook.shape[2] != d or not codebook.is_contiguous():
        raise ValueError("codebook must be a contiguous [H, Mt, d] tensor")
    Mt = codebook.shape[1]
    if Mt % (1 + C):
        raise ValueError("codebook rows must be M0 * (1 + C)")
    M0 = Mt // (1 + C)
    dev = K.device
    if vsum is None:
        vsum = torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty((B, H, Mt), dtype=torch.int32, device=dev)
    if want_assign and assign is None:
        assign = torch.empty((B, H, N), dtype=torch.int32, device=dev)
    rc = _lib.avq_assign_aggregate(_ptr(K), _ptr(V), _ptr(codebook), B, H, N, d, M0, C, _dtype_code(K),
                                   _ptr(vsum), _ptr(counts), _ptr(assign), _stream(K))
    if rc != 0:
        raise AvqError(rc, "avq_assign_aggregate")
    return vsum, counts, assign


def assign_aggregate_kv(K: torch.Tensor, V: torch.Tensor, codebook: torch.Tensor, C: int, *,
                        want_assign: bool = False, vsum: Optional[torch.Tensor] = None,
                        counts: Optional[torch.Tensor] = None, assign: Optional[torch.Tensor] = None,
                        ksum: Optional[torch.Tensor] = None):
    """Kernel 1 with the keys also summed per codeword (for codebook_update), in one pass.
    Returns (vsum, counts, assign or None, ksum [B, H, Mt, d] float32)."""
    B, H, N, d = _shape4(K, "K")
    if tuple(V.shape) != (B, H, N, d) or V.dtype != K.dtype or not V.is_contiguous():
        raise ValueError("V must match K")
    if codebook.dim() != 3 or codebook.shape[0] != H or codebook.shape[2] != d or not codebook.is_contiguous():
        raise ValueError("codebook must be a contiguous [H, Mt, d] tensor")
    Mt = codebook.shape[1]
    if Mt % (1 + C):
        raise ValueError("codebook rows must be M0 * (1 + C)")
    M0 = Mt // (1 + C)
    dev = K.device
    if vsum is None:
        vsum = torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev)
    if counts is None:
        counts = torch.empty((B, H, Mt), dtype=torch.int32, device=dev)
    if ksum is None:
        ksum = torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev)
    if want_assign and assign is None:
        assign = torch.empty((B, H, N), dtype=torch.int32, device=dev)
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
    Mt = codebook.shape[1]
    M0 = Mt // (1 + C)
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    dev = Q.device
    T = (N + block_q - 1) // block_q
    if Y is None:
        Y = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    topp = torch.empty((B, H, T, P), dtype=torch.int32, device=dev) if want_topp else None
    imp = torch.empty((B, H, T, M0), dtype=torch.float32, device=dev) if want_importance else None
    need = workspace_size(B, H, d, M0, C, Q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    for name, t in (("vsum", vsum), ("counts", counts)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    ws_bytes = workspace.numel() * workspace.element_size()
    if query_order is not None:
        if (query_order.dtype != torch.int32 or query_order.dim() != 1 or query_order.numel() != N
                or not query_order.is_contiguous() or query_order.device != dev):
            raise ValueError("query_order must be a contiguous int32 [N] tensor on the device of Q")
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
    if ksum.dim() != 4 or ksum.dtype != torch.float32 or not ksum.is_contiguous():
        raise ValueError("ksum must be a contiguous float32 [B, H, Mt, d] tensor")
    B, H, Mt, d = ksum.shape
    if Mt % (1 + C):
        raise ValueError("codeword rows must be M0 * (1 + C)")
    M0 = Mt // (1 + C)
    if tuple(counts.shape) != (B, H, Mt) or counts.dtype != torch.int32 or not counts.is_contiguous():
        raise ValueError("counts must be a contiguous int32 [B, H, Mt] tensor")
    for name, t, shape in (("S", S, (H, Mt, d)), ("Nema", Nema, (H, Mt)), ("codebook", codebook, (H, Mt, d))):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor")
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
