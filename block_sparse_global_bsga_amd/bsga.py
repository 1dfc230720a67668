"""Thin ctypes binding of libbsga (argument marshalling only).

Every computation happens in the HIP kernels behind the C ABI declared in
``include/bsga.h``; this module only checks tensor properties, allocates
outputs and workspaces with torch (device memory is PyTorch's job here), and
passes raw pointers plus torch's current HIP stream.  Importing it raises if
the native library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsga.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libbsga.so not found at {LIB_PATH}; build it with "
        "`python -m block_sparse_global_bsga_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_HIP = range(6)
(OP_PREDICT_MASK, OP_SELECT, OP_SPARSE_ATTN, OP_SPECIAL_DENSE, OP_DENSE_ATTN, OP_LAYER,
 OP_SPECIAL_DENSE_PACKED, OP_PROBE_SELECT, OP_NMSE, OP_BACKWARD,
 OP_PATCH_ROWS_PACKED) = range(11)
MAX_HEADS = 256
MAX_BLOCKS = 4096
SELECT_STATIC_MAX_ROWS = 65536

EXPORTS = [
    "bsga_version", "bsga_status_string", "bsga_num_blocks", "bsga_keep_count",
    "bsga_csr_capacity", "bsga_workspace_bytes", "bsga_predict_mask",
    "bsga_select", "bsga_sparse_attn", "bsga_special_dense", "bsga_dense_attn",
    "bsga_layer", "bsga_packed_kv_bytes", "bsga_pack_kv", "bsga_sparse_attn_packed",
    "bsga_special_dense_packed", "bsga_dense_attn_packed", "bsga_patch_rows_packed",
    "bsga_special_rows_packed", "bsga_redistribute", "bsga_probe_select", "bsga_nmse",
    "bsga_attn_backward", "bsga_select_static", "bsga_layer_train", "bsga_attn_backward_o32",
]


class Shape(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("patches_per_frame", ctypes.c_int32),
                ("special_per_frame", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32)]


_p = ctypes.c_void_p
_sp = ctypes.POINTER(Shape)
_lib.bsga_version.restype = ctypes.c_int
_lib.bsga_status_string.restype = ctypes.c_char_p
_lib.bsga_status_string.argtypes = [ctypes.c_int]
_lib.bsga_num_blocks.argtypes = [_sp, ctypes.POINTER(ctypes.c_int32)]
_lib.bsga_keep_count.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]
_lib.bsga_csr_capacity.argtypes = [_sp, ctypes.POINTER(ctypes.c_int64)]
_lib.bsga_redistribute.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_double), ctypes.c_double,
                                   ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
_lib.bsga_workspace_bytes.argtypes = [_sp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
_lib.bsga_predict_mask.argtypes = [_sp, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_select.argtypes = [_sp, _p, _p, ctypes.c_double, ctypes.c_double, _p, _p,
                             ctypes.c_int64, _p, ctypes.c_size_t, _p]
_lib.bsga_select_static.argtypes = [_sp, _p, _p, ctypes.c_double, ctypes.c_double, _p, _p,
                                    ctypes.c_int64, _p]
_lib.bsga_probe_select.argtypes = [_sp, _p, _p, ctypes.c_int32, _p, _p, _p, ctypes.c_int64, _p,
                                   ctypes.c_size_t, _p]
_lib.bsga_nmse.argtypes = [_sp, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_attn_backward.argtypes = [_sp, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    ctypes.c_size_t, _p]
_lib.bsga_sparse_attn.argtypes = [_sp, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_special_dense.argtypes = [_sp, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_dense_attn.argtypes = [_sp, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_packed_kv_bytes.argtypes = [_sp, ctypes.POINTER(ctypes.c_size_t)]
_lib.bsga_pack_kv.argtypes = [_sp, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_sparse_attn_packed.argtypes = [_sp, _p, _p, ctypes.c_size_t, _p, _p, _p, _p, _p]
_lib.bsga_special_dense_packed.argtypes = [_sp, _p, _p, ctypes.c_size_t, _p, _p, _p,
                                           ctypes.c_size_t, _p]
_lib.bsga_dense_attn_packed.argtypes = [_sp, _p, _p, ctypes.c_size_t, _p, _p, _p]
_lib.bsga_patch_rows_packed.argtypes = [_sp, _p, _p, ctypes.c_size_t, _p, _p, _p, _p, _p,
                                        ctypes.c_size_t, _p]
_lib.bsga_special_rows_packed.argtypes = [_sp, _p, _p, ctypes.c_size_t, _p, _p, _p,
                                          ctypes.c_size_t, _p]
_lib.bsga_layer.argtypes = [_sp, _p, _p, _p, _p, ctypes.c_double, ctypes.c_double, _p, _p, _p,
                            ctypes.c_int64, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_layer_train.argtypes = [_sp, _p, _p, _p, _p, ctypes.c_double, ctypes.c_double, _p, _p,
                                  _p, ctypes.c_int64, _p, _p, _p, _p, ctypes.c_size_t, _p]
_lib.bsga_attn_backward_o32.argtypes = [_sp, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                        ctypes.c_size_t, _p]


class BsgaError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return _lib.bsga_status_string(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != OK:
        raise BsgaError(status, call)


@dataclass(frozen=True)
class LayerShape:
    frames: int
    patches_per_frame: int
    special_per_frame: int
    heads: int
    block: int
    head_dim: int = 64

    def c(self) -> Shape:
        return Shape(self.frames, self.patches_per_frame, self.special_per_frame,
                     self.heads, self.head_dim, self.block)

    @property
    def tokens(self) -> int:
        return self.frames * (self.patches_per_frame + self.special_per_frame)


def version() -> int:
    return _lib.bsga_version()


def num_blocks(shape: LayerShape) -> int:
    out = ctypes.c_int32()
    _check(_lib.bsga_num_blocks(ctypes.byref(shape.c()), ctypes.byref(out)), "bsga_num_blocks")
    return out.value


def keep_count(n_blocks: int, rho: float) -> int:
    out = ctypes.c_int32()
    _check(_lib.bsga_keep_count(n_blocks, rho, ctypes.byref(out)), "bsga_keep_count")
    return out.value


def redistribute(weights: Sequence[float], mean_rho: float, rho_min: float,
                 rho_max: float) -> list:
    """Per-head rho from head weights (bsga_redistribute, host-side)."""
    h = len(weights)
    w = (ctypes.c_double * h)(*[float(x) for x in weights])
    out = (ctypes.c_double * h)()
    _check(_lib.bsga_redistribute(h, w, mean_rho, rho_min, rho_max, out), "bsga_redistribute")
    return list(out)


def csr_capacity(shape: LayerShape) -> int:
    out = ctypes.c_int64()
    _check(_lib.bsga_csr_capacity(ctypes.byref(shape.c()), ctypes.byref(out)), "bsga_csr_capacity")
    return out.value


def workspace_bytes(shape: LayerShape, op: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.bsga_workspace_bytes(ctypes.byref(shape.c()), op, ctypes.byref(out)),
           "bsga_workspace_bytes")
    return out.value


# ----------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _bf16(t: torch.Tensor, name: str, shape: LayerShape) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 bits (bfloat16/int16/uint16), got {t.dtype}")
    if tuple(t.shape) != (shape.heads, shape.tokens, shape.head_dim) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [H][N][64] = "
                         f"{(shape.heads, shape.tokens, shape.head_dim)}, got {tuple(t.shape)}")
    return t


def workspace(shape: LayerShape, op: int, device) -> torch.Tensor:
    n = max(1, workspace_bytes(shape, op))
    return torch.empty(n + 256, dtype=torch.uint8, device=device)


def _ws_ptr(ws: torch.Tensor) -> int:
    return (ws.data_ptr() + 255) & ~255


def _ws_len(ws: torch.Tensor) -> int:
    return ws.numel() - (_ws_ptr(ws) - ws.data_ptr())


def predict_mask(shape: LayerShape, q: torch.Tensor, k: torch.Tensor, *,
                 probs: Optional[torch.Tensor] = None, want_means: bool = False,
                 want_scores: bool = False, ws: Optional[torch.Tensor] = None):
    """Returns probs [H][B][B] float32, or a tuple (probs, then the pooled
    scores S [H][B][B] if want_scores, then Qbar, Kbar [H][B][64] if
    want_means)."""
    _bf16(q, "q", shape), _bf16(k, "k", shape)
    dev = q.device
    B = num_blocks(shape)
    if probs is None:
        probs = torch.empty((shape.heads, B, B), dtype=torch.float32, device=dev)
    scores = torch.empty_like(probs) if want_scores else None
    qbar = kbar = None
    if want_means:
        qbar = torch.empty((shape.heads, B, 64), dtype=torch.float32, device=dev)
        kbar = torch.empty_like(qbar)
    if ws is None:
        ws = workspace(shape, OP_PREDICT_MASK, dev)
    _check(_lib.bsga_predict_mask(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(probs),
                                  _ptr(scores), _ptr(qbar), _ptr(kbar), _ws_ptr(ws), _ws_len(ws),
                                  _stream(dev)),
           "bsga_predict_mask")
    if not (want_means or want_scores):
        return probs
    out = (probs,) + ((scores,) if want_scores else ()) + ((qbar, kbar) if want_means else ())
    return out


def _rho_array(shape: LayerShape, rho_per_head: Optional[Sequence[float]]):
    if rho_per_head is None:
        return None, None
    if len(rho_per_head) != shape.heads:
        raise ValueError("rho_per_head needs one value per head")
    arr = (ctypes.c_double * shape.heads)(*[float(r) for r in rho_per_head])
    return arr, ctypes.cast(arr, ctypes.c_void_p).value


def select(shape: LayerShape, probs: torch.Tensor, rho: float, tau: float,
           rho_per_head: Optional[Sequence[float]] = None, *,
           row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None,
           ws: Optional[torch.Tensor] = None):
    """Returns (row_ptr [H*B+1] int32, col_idx [H*B*B] int32 buffer)."""
    dev = probs.device
    B = num_blocks(shape)
    if probs.dtype != torch.float32 or tuple(probs.shape) != (shape.heads, B, B) \
            or not probs.is_contiguous():
        raise ValueError("probs must be contiguous float32 [H][B][B]")
    if row_ptr is None:
        row_ptr = torch.empty(shape.heads * B + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(csr_capacity(shape), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(shape, OP_SELECT, dev)
    keep, rp = _rho_array(shape, rho_per_head)
    _check(_lib.bsga_select(ctypes.byref(shape.c()), _ptr(probs), rp, float(rho), float(tau),
                            _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ws_ptr(ws),
                            _ws_len(ws), _stream(dev)), "bsga_select")
    del keep
    return row_ptr, col_idx


def select_static(shape: LayerShape, probs: torch.Tensor, rho: float, tau: float,
                  rho_per_head: Optional[Sequence[float]] = None, *,
                  row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None):
    """bsga_select_static: the selection without a workspace (the library's own
    per-GPU scratch).  Returns (row_ptr, col_idx) like select()."""
    dev = probs.device
    B = num_blocks(shape)
    if probs.dtype != torch.float32 or tuple(probs.shape) != (shape.heads, B, B) \
            or not probs.is_contiguous():
        raise ValueError("probs must be contiguous float32 [H][B][B]")
    if row_ptr is None:
        row_ptr = torch.empty(shape.heads * B + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(csr_capacity(shape), dtype=torch.int32, device=dev)
    keep, rp = _rho_array(shape, rho_per_head)
    _check(_lib.bsga_select_static(ctypes.byref(shape.c()), _ptr(probs), rp, float(rho),
                                   float(tau), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                   _stream(dev)), "bsga_select_static")
    del keep
    return row_ptr, col_idx


def probe_select(shape: LayerShape, q: torch.Tensor, k: torch.Tensor, topk: int, *,
                 want_scores: bool = False, row_ptr: Optional[torch.Tensor] = None,
                 col_idx: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Query-probe Top-K block lists.  Returns (row_ptr, col_idx) or, with
    want_scores, (row_ptr, col_idx, scores [H][N_p] float32)."""
    q, k = _bf16(q, "q", shape), _bf16(k, "k", shape)
    dev = q.device
    B = num_blocks(shape)
    n_p = shape.frames * shape.patches_per_frame
    if row_ptr is None:
        row_ptr = torch.empty(shape.heads * B + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(csr_capacity(shape), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(shape, OP_PROBE_SELECT, dev)
    scores = torch.empty((shape.heads, n_p), dtype=torch.float32, device=dev) if want_scores else None
    _check(_lib.bsga_probe_select(ctypes.byref(shape.c()), _ptr(q), _ptr(k), int(topk),
                                  _ptr(scores), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                  _ws_ptr(ws), _ws_len(ws), _stream(dev)), "bsga_probe_select")
    return (row_ptr, col_idx, scores) if want_scores else (row_ptr, col_idx)


def nmse(shape: LayerShape, o_ref: torch.Tensor, o: torch.Tensor, *,
         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head ||o_ref - o||^2 / ||o_ref||^2 (float64 [H] on the device)."""
    o_ref, o = _bf16(o_ref, "o_ref", shape), _bf16(o, "o", shape)
    dev = o.device
    out = torch.empty(shape.heads, dtype=torch.float64, device=dev)
    if ws is None:
        ws = workspace(shape, OP_NMSE, dev)
    _check(_lib.bsga_nmse(ctypes.byref(shape.c()), _ptr(o_ref), _ptr(o), _ptr(out), _ws_ptr(ws),
                          _ws_len(ws), _stream(dev)), "bsga_nmse")
    return out


def attn_backward(shape: LayerShape, q, k, v, o, lse, d_o, row_ptr, col_idx, *,
                  dq=None, dk=None, dv=None, ws: Optional[torch.Tensor] = None):
    """Gradients (dQ, dK, dV) [H][N][64] float32 of the layer's attention for
    the mask (row_ptr, col_idx) that produced o and lse.  o: the bf16 rows
    (bsga_attn_backward), or the float32 rows of layer_train
    (bsga_attn_backward_o32)."""
    o32 = o.dtype == torch.float32
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")) + (() if o32 else ((o, "o"),)):
        _bf16(t, n, shape)
    if o32 and (tuple(o.shape) != (shape.heads, shape.tokens, 64) or not o.is_contiguous()):
        raise ValueError("o (float32) must be a contiguous [H][N][64] tensor")
    dev = q.device
    grads = []
    for g in (dq, dk, dv):
        if g is None:
            g = torch.empty((shape.heads, shape.tokens, 64), dtype=torch.float32, device=dev)
        grads.append(g)
    if ws is None:
        ws = workspace(shape, OP_BACKWARD, dev)
    fn, name = ((_lib.bsga_attn_backward_o32, "bsga_attn_backward_o32") if o32 else
                (_lib.bsga_attn_backward, "bsga_attn_backward"))
    _check(fn(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o),
              _ptr(row_ptr), _ptr(col_idx), *[_ptr(g) for g in grads], _ws_ptr(ws), _ws_len(ws),
              _stream(dev)), name)
    return tuple(grads)


def pooled_specials_shape(shape: LayerShape) -> LayerShape:
    """The ablation without a dense special path: the whole token sequence as
    one run of blocks (special tokens pooled with the patches)."""
    return LayerShape(1, shape.tokens, 0, shape.heads, shape.block)


def _outputs(shape: LayerShape, q: torch.Tensor, o, lse):
    if o is None:
        o = torch.zeros_like(q, dtype=torch.bfloat16)
    if lse is None:
        lse = torch.zeros((shape.heads, shape.tokens), dtype=torch.float32, device=q.device)
    return o, lse


def sparse_attn(shape: LayerShape, q, k, v, row_ptr, col_idx, *, o=None, lse=None, ws=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, n, shape)
    o, lse = _outputs(shape, q, o, lse)
    if ws is None:
        ws = workspace(shape, OP_SPARSE_ATTN, q.device)
    _check(_lib.bsga_sparse_attn(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse), _ws_ptr(ws),
                                 _ws_len(ws), _stream(q.device)), "bsga_sparse_attn")
    return o, lse


def special_dense(shape: LayerShape, q, k, v, o, lse, *, ws=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, n, shape)
    if ws is None:
        ws = workspace(shape, OP_SPECIAL_DENSE, q.device)
    _check(_lib.bsga_special_dense(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), _ws_ptr(ws), _ws_len(ws), _stream(q.device)),
           "bsga_special_dense")
    return o, lse


def dense_attn(shape: LayerShape, q, k, v, *, o=None, lse=None, ws=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, n, shape)
    o, lse = _outputs(shape, q, o, lse)
    if ws is None:
        ws = workspace(shape, OP_DENSE_ATTN, q.device)
    _check(_lib.bsga_dense_attn(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                _ptr(lse), _ws_ptr(ws), _ws_len(ws), _stream(q.device)),
           "bsga_dense_attn")
    return o, lse


def packed_kv_bytes(shape: LayerShape) -> int:
    out = ctypes.c_size_t()
    _check(_lib.bsga_packed_kv_bytes(ctypes.byref(shape.c()), ctypes.byref(out)),
           "bsga_packed_kv_bytes")
    return out.value


def pack_kv(shape: LayerShape, k, v, *, kv: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed K / V^T buffer (uint8 tensor; the packed data start at its
    first 256-byte aligned byte)."""
    _bf16(k, "k", shape), _bf16(v, "v", shape)
    if kv is None:
        kv = torch.empty(packed_kv_bytes(shape) + 256, dtype=torch.uint8, device=k.device)
    _check(_lib.bsga_pack_kv(ctypes.byref(shape.c()), _ptr(k), _ptr(v), _ws_ptr(kv),
                             _ws_len(kv), _stream(k.device)), "bsga_pack_kv")
    return kv


def sparse_attn_packed(shape: LayerShape, q, kv, row_ptr, col_idx, o, lse):
    _bf16(q, "q", shape)
    _check(_lib.bsga_sparse_attn_packed(ctypes.byref(shape.c()), _ptr(q), _ws_ptr(kv), _ws_len(kv),
                                        _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse),
                                        _stream(q.device)), "bsga_sparse_attn_packed")
    return o, lse


def special_dense_packed(shape: LayerShape, q, kv, o, lse, *, ws=None):
    _bf16(q, "q", shape)
    if ws is None:
        ws = workspace(shape, OP_SPECIAL_DENSE_PACKED, q.device)
    _check(_lib.bsga_special_dense_packed(ctypes.byref(shape.c()), _ptr(q), _ws_ptr(kv),
                                          _ws_len(kv), _ptr(o), _ptr(lse), _ws_ptr(ws),
                                          _ws_len(ws), _stream(q.device)),
           "bsga_special_dense_packed")
    return o, lse


def dense_attn_packed(shape: LayerShape, q, kv, o, lse):
    _bf16(q, "q", shape)
    _check(_lib.bsga_dense_attn_packed(ctypes.byref(shape.c()), _ptr(q), _ws_ptr(kv), _ws_len(kv),
                                       _ptr(o), _ptr(lse), _stream(q.device)),
           "bsga_dense_attn_packed")
    return o, lse


def patch_rows_packed(shape: LayerShape, q, kv, row_ptr, col_idx, o, lse, *, ws="auto"):
    """Final patch rows.  ws: a workspace of workspace_bytes(OP_PATCH_ROWS_PACKED)
    (allocated here when "auto"), or None to compute every row in one
    workgroup (no tail splitting)."""
    _bf16(q, "q", shape)
    if isinstance(ws, str):
        ws = workspace(shape, OP_PATCH_ROWS_PACKED, q.device)
    _check(_lib.bsga_patch_rows_packed(ctypes.byref(shape.c()), _ptr(q), _ws_ptr(kv), _ws_len(kv),
                                       _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse),
                                       None if ws is None else _ws_ptr(ws),
                                       0 if ws is None else _ws_len(ws), _stream(q.device)),
           "bsga_patch_rows_packed")
    return o, lse


def special_rows_packed(shape: LayerShape, q, kv, o, lse, *, ws=None):
    _bf16(q, "q", shape)
    if ws is None:
        ws = workspace(shape, OP_SPECIAL_DENSE_PACKED, q.device)
    _check(_lib.bsga_special_rows_packed(ctypes.byref(shape.c()), _ptr(q), _ws_ptr(kv),
                                         _ws_len(kv), _ptr(o), _ptr(lse), _ws_ptr(ws),
                                         _ws_len(ws), _stream(q.device)),
           "bsga_special_rows_packed")
    return o, lse


class LayerBuffers:
    """Outputs and workspace of one layer call, allocated once and reused."""

    def __init__(self, shape: LayerShape, device):
        B = num_blocks(shape)
        self.probs = torch.empty((shape.heads, B, B), dtype=torch.float32, device=device)
        self.row_ptr = torch.empty(shape.heads * B + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(csr_capacity(shape), dtype=torch.int32, device=device)
        self.o = torch.empty((shape.heads, shape.tokens, 64), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((shape.heads, shape.tokens), dtype=torch.float32, device=device)
        self.ws = workspace(shape, OP_LAYER, device)


def layer(shape: LayerShape, q, k, v, rho: float, tau: float,
          rho_per_head: Optional[Sequence[float]] = None, *,
          bufs: Optional[LayerBuffers] = None) -> LayerBuffers:
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, n, shape)
    if bufs is None:
        bufs = LayerBuffers(shape, q.device)
    keep, rp = _rho_array(shape, rho_per_head)
    _check(_lib.bsga_layer(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), rp, float(rho),
                           float(tau), _ptr(bufs.probs), _ptr(bufs.row_ptr), _ptr(bufs.col_idx),
                           bufs.col_idx.numel(), _ptr(bufs.o), _ptr(bufs.lse), _ws_ptr(bufs.ws),
                           _ws_len(bufs.ws), _stream(q.device)), "bsga_layer")
    del keep
    return bufs


def layer_train(shape: LayerShape, q, k, v, rho: float, tau: float,
                rho_per_head: Optional[Sequence[float]] = None, *,
                bufs: Optional[LayerBuffers] = None, o32: Optional[torch.Tensor] = None):
    """bsga_layer_train: the layer with P as a float16 pair hi + lo in the P V
    products and the final rows also as float32.  Returns (bufs, o32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, n, shape)
    if bufs is None:
        bufs = LayerBuffers(shape, q.device)
    if o32 is None:
        o32 = torch.empty((shape.heads, shape.tokens, 64), dtype=torch.float32, device=q.device)
    keep, rp = _rho_array(shape, rho_per_head)
    _check(_lib.bsga_layer_train(ctypes.byref(shape.c()), _ptr(q), _ptr(k), _ptr(v), rp,
                                 float(rho), float(tau), _ptr(bufs.probs), _ptr(bufs.row_ptr),
                                 _ptr(bufs.col_idx), bufs.col_idx.numel(), _ptr(bufs.o),
                                 _ptr(bufs.lse), _ptr(o32), _ws_ptr(bufs.ws), _ws_len(bufs.ws),
                                 _stream(q.device)), "bsga_layer_train")
    del keep
    return bufs, o32
