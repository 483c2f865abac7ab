"""Thin ctypes binding of libgdn.so (``include/gdn.h``) for torch tensors.

Argument marshalling only: every step of the path runs in the library's gfx950
kernels.  Functions carry the C entry points' names.  Tensors must be contiguous and
on one HIP device; the call is enqueued on ``stream`` (default: torch's current
stream on that device) and returns without synchronising.  If the library is not
built the first call raises -- there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

GDN_CHUNK = 64
GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP = 0, 1, 2, 3
GDN_F32, GDN_BF16 = 0, 1
_STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARGUMENT", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_HIP"}


class GdnShape(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), message))
        self.status = status


_lock = threading.Lock()
_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

SIGNATURES = {
    "gdn_chunk_prefill_workspace_size": (_sz, [ctypes.POINTER(GdnShape), _i32, _i64]),
    "gdn_recurrent_decode": (ctypes.c_int, [ctypes.POINTER(GdnShape), _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _i32, _vp, _vp, _vp]),
    "gdn_chunk_prefill": (ctypes.c_int, [ctypes.POINTER(GdnShape), _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _vp,
                                         _sz, _vp]),
    "gdn_mixed_step": (ctypes.c_int, [ctypes.POINTER(GdnShape), _i32, _vp, _vp, _i32, _i64, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                      _i64, _vp, _sz, _vp]),
    "gdn_recurrent_verify": (ctypes.c_int, [ctypes.POINTER(GdnShape), _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _i32, _vp, _vp, _vp]),
    "gdn_last_error": (ctypes.c_char_p, []),
}


def library(path: str = LIB_PATH):
    """Load libgdn.so once and declare its entry points."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build()" % path)
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype, fn.argtypes = res, args
            _lib = lib
    return _lib


def gdn_last_error() -> str:
    return library().gdn_last_error().decode()


def _check(status: int) -> None:
    if status != GDN_OK:
        raise GdnError(status, gdn_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise ValueError("q/k/v/o must be bfloat16 or float32, got %s" % t.dtype)


def make_shape(num_k_heads, num_v_heads, d_k, d_v, dtype: int, scale: float) -> GdnShape:
    return GdnShape(int(num_k_heads), int(num_v_heads), int(d_k), int(d_v), int(dtype), float(scale))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, device=None, ndim=None):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))


def _heads(q, k, v, g, beta, o, rows):
    _need(q, "q", ndim=3)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device, got %s" % dev)
    _need(k, "k", dtype=q.dtype, device=dev, ndim=3)
    _need(v, "v", dtype=q.dtype, device=dev, ndim=3)
    _need(o, "o", dtype=q.dtype, device=dev, ndim=3)
    _need(g, "g", dtype=torch.float32, device=dev, ndim=2)
    _need(beta, "beta", dtype=torch.float32, device=dev, ndim=2)
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if T != rows or k.shape != q.shape or v.shape[0] != T or o.shape != v.shape \
            or g.shape != (T, H_v) or beta.shape != (T, H_v):
        raise ValueError("inconsistent shapes: q %s k %s v %s o %s g %s beta %s (rows %d)" % (
            tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(o.shape), tuple(g.shape),
            tuple(beta.shape), rows))
    return dev, H_k, H_v, d_k, d_v


def _pool(state_pool, dev, H_v, d_k, d_v):
    _need(state_pool, "state_pool", dtype=torch.float32, device=dev, ndim=4)
    if tuple(state_pool.shape[1:]) != (H_v, d_k, d_v):
        raise ValueError("state_pool must be [num_slots, %d, %d, %d], got %s" % (
            H_v, d_k, d_v, tuple(state_pool.shape)))
    return state_pool.shape[0]


def _index(t, name, n, dev, optional=False):
    if t is None and optional:
        return
    _need(t, name, dtype=torch.int32, device=dev, ndim=1)
    if t.shape[0] != n:
        raise ValueError("%s must have %d entries, got %d" % (name, n, t.shape[0]))


def gdn_chunk_prefill_workspace_size(num_k_heads, num_v_heads, d_k, d_v, dtype: int, num_seqs: int,
                                     total_tokens: int) -> int:
    shape = make_shape(num_k_heads, num_v_heads, d_k, d_v, dtype, 1.0)
    return int(library().gdn_chunk_prefill_workspace_size(ctypes.byref(shape), int(num_seqs),
                                                          int(total_tokens)))


def export_offsets(lengths: Sequence[int], start_pos: Optional[Sequence[int]], export_grid: int):
    """Exclusive prefix sum of each sequence's number of grid points in (s, s + L]."""
    offs = [0]
    for i, L in enumerate(lengths):
        s = 0 if start_pos is None else int(start_pos[i])
        n = 0 if export_grid <= 0 else (s + int(L)) // export_grid - s // export_grid
        offs.append(offs[-1] + n)
    return offs


def gdn_recurrent_decode(q, k, v, g, beta, o, state_pool, slot_in, slot_out, *, scale: float,
                         stream=None) -> None:
    """Packed single-token decode of q.shape[0] cached rows (see include/gdn.h)."""
    B = q.shape[0]
    dev, H_k, H_v, d_k, d_v = _heads(q, k, v, g, beta, o, B)
    num_slots = _pool(state_pool, dev, H_v, d_k, d_v)
    _index(slot_in, "slot_in", B, dev)
    _index(slot_out, "slot_out", B, dev)
    shape = make_shape(H_k, H_v, d_k, d_v, _dtype_code(q), scale)
    with torch.cuda.device(dev):
        _check(library().gdn_recurrent_decode(
            ctypes.byref(shape), B, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
            _ptr(state_pool), num_slots, _ptr(slot_in), _ptr(slot_out), _stream(dev, stream)))


def gdn_recurrent_verify(q, k, v, g, beta, o, state_pool, slot_in, token_slots, *, scale: float,
                         tokens_per_row: int, stream=None) -> None:
    """Multi-token verify rows: len(slot_in) rows of tokens_per_row tokens each, the
    state after every token written to its token slot (see include/gdn.h)."""
    B = slot_in.shape[0]
    n = B * int(tokens_per_row)
    dev, H_k, H_v, d_k, d_v = _heads(q, k, v, g, beta, o, n)
    num_slots = _pool(state_pool, dev, H_v, d_k, d_v)
    _index(slot_in, "slot_in", B, dev)
    _index(token_slots, "token_slots", n, dev)
    shape = make_shape(H_k, H_v, d_k, d_v, _dtype_code(q), scale)
    with torch.cuda.device(dev):
        _check(library().gdn_recurrent_verify(
            ctypes.byref(shape), B, int(tokens_per_row), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
            _ptr(state_pool), num_slots, _ptr(slot_in), _ptr(token_slots), _stream(dev, stream)))


def _prefill_common(dev, num_seqs, cu_seqlens, init_slot, final_slot, start_pos, export_grid,
                    export_states, export_offsets_t, export_slots, workspace, H_v, d_k, d_v):
    _index(cu_seqlens, "cu_seqlens", num_seqs + 1, dev)
    _index(init_slot, "init_slot", num_seqs, dev)
    _index(final_slot, "final_slot", num_seqs, dev)
    _index(start_pos, "start_pos", num_seqs, dev, optional=True)
    n_exp = 0
    if export_grid:
        _index(export_offsets_t, "export_offsets", num_seqs + 1, dev)
        if export_slots is not None:
            _need(export_slots, "export_slots", dtype=torch.int32, device=dev, ndim=1)
            n_exp = export_slots.shape[0]
        elif export_states is not None:
            _need(export_states, "export_states", dtype=torch.float32, device=dev, ndim=4)
            if tuple(export_states.shape[1:]) != (H_v, d_k, d_v):
                raise ValueError("export_states must be [E, %d, %d, %d]" % (H_v, d_k, d_v))
            n_exp = export_states.shape[0]
    if workspace is None:            # the library reports an error if the call needs one
        return n_exp, 0
    _need(workspace, "workspace", device=dev)
    return n_exp, workspace.numel() * workspace.element_size()


def _prefill_call(entry, q, k, v, g, beta, o, cu_seqlens, state_pool, init_slot, final_slot, scale, workspace,
                  start_pos, export_grid, export_states, export_offsets, export_slots, stream):
    T = q.shape[0]
    dev, H_k, H_v, d_k, d_v = _heads(q, k, v, g, beta, o, T)
    num_slots = _pool(state_pool, dev, H_v, d_k, d_v)
    N = cu_seqlens.shape[0] - 1
    n_exp, ws_bytes = _prefill_common(dev, N, cu_seqlens, init_slot, final_slot, start_pos, export_grid,
                                      export_states, export_offsets, export_slots, workspace, H_v, d_k, d_v)
    shape = make_shape(H_k, H_v, d_k, d_v, _dtype_code(q), scale)
    with torch.cuda.device(dev):
        _check(getattr(library(), entry)(
            ctypes.byref(shape), N, T, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(o), _ptr(state_pool), num_slots, _ptr(init_slot), _ptr(final_slot), _ptr(start_pos),
            int(export_grid), _ptr(export_states), _ptr(export_offsets), _ptr(export_slots), n_exp,
            _ptr(workspace), ws_bytes, _stream(dev, stream)))


def gdn_chunk_prefill(q, k, v, g, beta, o, cu_seqlens, state_pool, init_slot, final_slot, *,
                      scale: float, workspace=None, start_pos=None, export_grid: int = 0,
                      export_states=None, export_offsets=None, export_slots=None, stream=None) -> None:
    """Chunked prefill over len(cu_seqlens) - 1 packed sequences (see include/gdn.h).
    Exports go to export_states, or straight into state_pool slots when export_slots
    (one int32 slot per export) is given."""
    _prefill_call("gdn_chunk_prefill", q, k, v, g, beta, o, cu_seqlens, state_pool, init_slot, final_slot,
                  scale, workspace, start_pos, export_grid, export_states, export_offsets, export_slots, stream)


def gdn_mixed_step(q, k, v, g, beta, o, state_pool, slot_in, slot_out, cu_seqlens_prefill, init_slot,
                   final_slot, *, scale: float, workspace=None, start_pos=None, export_grid: int = 0,
                   export_states=None, export_offsets=None, export_slots=None, stream=None) -> None:
    """One mixed step: rows [0, len(slot_in)) decode, the rest prefill (see include/gdn.h)."""
    T = q.shape[0]
    dev, H_k, H_v, d_k, d_v = _heads(q, k, v, g, beta, o, T)
    num_slots = _pool(state_pool, dev, H_v, d_k, d_v)
    B = slot_in.shape[0]
    _index(slot_in, "slot_in", B, dev)
    _index(slot_out, "slot_out", B, dev)
    N = cu_seqlens_prefill.shape[0] - 1
    n_exp, ws_bytes = _prefill_common(dev, N, cu_seqlens_prefill, init_slot, final_slot, start_pos,
                                      export_grid, export_states, export_offsets, export_slots, workspace,
                                      H_v, d_k, d_v)
    shape = make_shape(H_k, H_v, d_k, d_v, _dtype_code(q), scale)
    with torch.cuda.device(dev):
        _check(library().gdn_mixed_step(
            ctypes.byref(shape), B, _ptr(slot_in), _ptr(slot_out), N, T - B, _ptr(cu_seqlens_prefill),
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o), _ptr(state_pool), num_slots,
            _ptr(init_slot), _ptr(final_slot), _ptr(start_pos), int(export_grid), _ptr(export_states),
            _ptr(export_offsets), _ptr(export_slots), n_exp, _ptr(workspace), ws_bytes, _stream(dev, stream)))


def alloc_workspace(H_v: int, dtype: torch.dtype, num_seqs: int, total_tokens: int, device) -> torch.Tensor:
    """A uint8 device buffer of the size gdn_chunk_prefill needs (torch allocates it;
    at least 256 bytes so that it always has a valid address)."""
    code = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    n = gdn_chunk_prefill_workspace_size(1, H_v, 64, 64, code, num_seqs, total_tokens)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
