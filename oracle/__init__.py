"""Oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

A plain sequential fp64 CPU evaluation of the recurrence (``gdn_oracle.c``), loaded
through ctypes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package.  It shares no code with the GPU library, and
the GPU library never imports it.

Every function takes numpy arrays already widened to float64 from the exact values
the GPU receives (bf16 or fp32), so the oracle itself rounds nothing.

Parity pins (see ``tests/test_oracle_pins.py``): brute-force dense transition
matrices, an exact-rational evaluation, closed forms for the pure-decay and
exact-recall special cases, an independent fp64 chunked (WY/UT) evaluation, and a
hand-worked example under ``tests/golden/``.  The conventions that the pages leave
open and that no pin can fix -- the output scale, the GQA head map and the state
layout -- are "parity unpinned": oracle and GPU share them by definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lock = threading.Lock()
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle (gcc, -O2, OpenMP, no fast-math) into a shared library."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def open_library(path: str):
    """Load an oracle shared library and declare its entry points."""
    lib = ctypes.CDLL(path)
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p,
        _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_double, _f64p, ctypes.c_int,
        _i32p, _i32p, _i32p, ctypes.c_int, _f64p, _i32p, _f64p, _f64p]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        _f64p, _f64p, _f64p, _f64p, _f64p, ctypes.c_double, _f64p, ctypes.c_int,
        _i32p, _i32p, _f64p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            _lib = open_library(_LIB_PATH)
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def export_counts(lengths, start_pos, export_grid):
    """Number of grid positions p (p % export_grid == 0) with start < p <= start + len."""
    lengths = np.asarray(lengths, dtype=np.int64)
    start = np.zeros_like(lengths) if start_pos is None else np.asarray(start_pos, dtype=np.int64)
    if export_grid <= 0:
        return np.zeros_like(lengths)
    return (start + lengths) // export_grid - start // export_grid


def prefill(q, k, v, g, beta, cu_seqlens, *, scale, pool=None, init_slot=None,
            final_slot=None, start_pos=None, export_grid=0, initial_states=None, lib=None):
    """Sequential fp64 prefill.

    q, k: [T, H_k, d_k]; v: [T, H_v, d_v]; g, beta: [T, H_v]; cu_seqlens: [N+1].
    Either ``pool`` (+ ``init_slot``/``final_slot``, updated in place) or
    ``initial_states`` [N, H_v, d_k, d_v] (None = zeros) supplies the start states.

    Returns (o [T, H_v, d_v], finals [N, H_v, d_k, d_v], exports [E, H_v, d_k, d_v],
    export_offsets [N+1]).  ``lib`` selects another build of the oracle (tests only).
    """
    lib = lib or _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = _i32(cu_seqlens)
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    N = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, H_v) and beta.shape == (T, H_v)
    if initial_states is not None:
        assert pool is None
        pool = _f64(initial_states).copy()
        init_slot = np.arange(N, dtype=np.int32)
        final_slot = None
    if pool is not None:
        assert pool.dtype == np.float64 and pool.flags.c_contiguous
        num_slots = pool.shape[0]
    else:
        num_slots = 0
    init_slot = None if init_slot is None else _i32(init_slot)
    final_slot = None if final_slot is None else _i32(final_slot)
    sp = None if start_pos is None else _i32(start_pos)
    lengths = np.diff(cu.astype(np.int64))
    counts = export_counts(lengths, sp, export_grid)
    offsets = np.zeros(N + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    n_exp = int(offsets[-1])
    exports = np.zeros((max(n_exp, 1), H_v, d_k, d_v), dtype=np.float64)
    o = np.zeros((T, H_v, d_v), dtype=np.float64)
    finals = np.zeros((N, H_v, d_k, d_v), dtype=np.float64)
    st = lib.oracle_prefill(H_k, H_v, d_k, d_v, N, _p(cu, _i32p), _p(q, _f64p), _p(k, _f64p),
                            _p(v, _f64p), _p(g, _f64p), _p(beta, _f64p), float(scale),
                            _p(pool, _f64p), num_slots, _p(init_slot, _i32p),
                            _p(final_slot, _i32p), _p(sp, _i32p), int(export_grid),
                            _p(exports, _f64p) if export_grid > 0 else None,
                            _p(offsets, _i32p) if export_grid > 0 else None,
                            _p(o, _f64p), _p(finals, _f64p))
    if st != 0:
        raise ValueError("oracle_prefill rejected its arguments (status %d)" % st)
    return o, finals, exports[:n_exp], offsets


def decode(q, k, v, g, beta, pool, slot_in, slot_out, *, scale, lib=None):
    """Sequential fp64 single-token decode; ``pool`` (float64) is updated in place.

    q, k: [B, H_k, d_k]; v: [B, H_v, d_v]; g, beta: [B, H_v]; returns o [B, H_v, d_v].
    """
    lib = lib or _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    assert pool.dtype == np.float64 and pool.flags.c_contiguous
    B, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    si, so = _i32(slot_in), _i32(slot_out)
    o = np.zeros((B, H_v, d_v), dtype=np.float64)
    st = lib.oracle_decode(H_k, H_v, d_k, d_v, B, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                           _p(g, _f64p), _p(beta, _f64p), float(scale), _p(pool, _f64p),
                           pool.shape[0], _p(si, _i32p), _p(so, _i32p), _p(o, _f64p))
    if st != 0:
        raise ValueError("oracle_decode rejected its arguments (status %d)" % st)
    return o
