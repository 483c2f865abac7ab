"""The C ABI without a GPU: the library loads, exports every symbol that
include/gdn.h declares, sizes the workspace, and rejects bad host arguments with a
clear message before anything is enqueued.

Every call here is built to fail host validation: besides the argument under test,
each one carries a second invalid argument that validation checks later (a NULL
slot_out for decode, a NULL init_slot for prefill), so no call can ever reach a
kernel launch, on a machine with or without a GPU."""
import ctypes
import os
import re

import pytest

from gated_deltanet_rule_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libgdn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"gdn_chunk_prefill_workspace_size", "gdn_recurrent_decode", "gdn_chunk_prefill",
                          "gdn_mixed_step", "gdn_recurrent_verify", "gdn_last_error"}
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(B.SIGNATURES) == set(names)


def test_workspace_size():
    """The prefill keeps every intermediate in LDS and registers: no scratch needed."""
    lib = B.library()
    s = B.make_shape(16, 32, 128, 128, B.GDN_BF16, 0.1)
    assert lib.gdn_chunk_prefill_workspace_size(ctypes.byref(s), 16, 16 * 8192) == 0
    bad = B.make_shape(3, 32, 128, 128, B.GDN_BF16, 0.1)
    assert lib.gdn_chunk_prefill_workspace_size(ctypes.byref(bad), 16, 1000) == 0


FAKE = 0x100000           # a 16-byte aligned stand-in address that is never dereferenced


def _decode(shape=None, num_rows=4, q=FAKE, num_slots=8, slot_out=None):
    lib = B.library()
    shape = shape or B.make_shape(2, 4, 64, 64, B.GDN_BF16, 0.125)
    st = lib.gdn_recurrent_decode(ctypes.byref(shape), num_rows, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  num_slots, FAKE, slot_out, None)
    return st, B.gdn_last_error()


def _prefill(shape=None, num_seqs=2, total_tokens=100, export_grid=0, q=FAKE, cu=FAKE, ws_bytes=0,
             num_export=0, init_slot=None, export_offsets=FAKE, export_slots=None):
    # guard: init_slot is NULL unless a test passes one, and validation rejects that
    # after every check the tests below exercise
    lib = B.library()
    shape = shape or B.make_shape(2, 4, 64, 64, B.GDN_BF16, 0.125)
    st = lib.gdn_chunk_prefill(ctypes.byref(shape), num_seqs, total_tokens, cu, q, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, 8, init_slot, FAKE, None, export_grid, FAKE, export_offsets,
                               export_slots, num_export, FAKE, ws_bytes, None)
    return st, B.gdn_last_error()


@pytest.mark.parametrize("shape,needle,code", [
    (B.make_shape(3, 4, 64, 64, B.GDN_BF16, 0.1), "multiple of num_k_heads", B.GDN_ERR_UNSUPPORTED),
    (B.make_shape(2, 4, 96, 64, B.GDN_BF16, 0.1), "64 or 128", B.GDN_ERR_UNSUPPORTED),
    (B.make_shape(2, 4, 64, 256, B.GDN_BF16, 0.1), "64 or 128", B.GDN_ERR_UNSUPPORTED),
    (B.make_shape(2, 4, 64, 64, 7, 0.1), "dtype 7", B.GDN_ERR_UNSUPPORTED),
    (B.make_shape(0, 4, 64, 64, B.GDN_BF16, 0.1), "positive", B.GDN_ERR_INVALID_ARGUMENT),
    (B.make_shape(2, 4, 64, 64, B.GDN_BF16, float("nan")), "scale", B.GDN_ERR_INVALID_ARGUMENT),
])
def test_bad_shapes(shape, needle, code):
    for st, msg in (_decode(shape=shape), _prefill(shape=shape)):
        assert st == code and needle in msg, (st, msg)


def test_decode_validation():
    st, msg = _decode(num_rows=-1)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "num_rows -1" in msg
    st, msg = _decode(num_slots=-2)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "num_slots -2" in msg
    st, msg = _decode(q=None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "q is NULL" in msg
    st, msg = _decode(q=FAKE + 4)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "16-byte aligned" in msg
    st, msg = _decode()
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "slot_out is NULL" in msg
    # zero rows is a no-op, whatever the pointers
    st, msg = _decode(num_rows=0, q=None)
    assert st == B.GDN_OK and msg == ""


def test_prefill_validation():
    st, msg = _prefill(export_grid=1056)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "1056" in msg and "chunk size 64" in msg
    st, msg = _prefill(export_grid=-64)
    assert st == B.GDN_ERR_INVALID_ARGUMENT
    st, msg = _prefill(num_seqs=-1)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "num_seqs -1" in msg
    st, msg = _prefill(total_tokens=-5)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "total_tokens -5" in msg
    st, msg = _prefill(cu=None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "cu_seqlens is NULL" in msg
    # q is checked after init_slot; the guard here is a NULL export_offsets, checked after q
    st, msg = _prefill(q=FAKE + 8, init_slot=FAKE, export_grid=64, export_offsets=None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "q (" in msg and "aligned" in msg
    st, msg = _prefill(init_slot=FAKE, export_grid=64, export_offsets=None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "export_offsets is NULL" in msg
    st, msg = _prefill(num_export=-1, export_grid=64)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "num_export_states" in msg
    st, msg = _prefill(init_slot=FAKE, export_grid=64, num_export=4, export_slots=FAKE + 2)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "export_slots" in msg
    st, msg = _prefill(export_grid=1088)          # lcm(64, 1088) = 1088 is accepted; the NULL init_slot is not
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "init_slot is NULL" in msg
    st, msg = _prefill(num_seqs=0, q=None, cu=None)   # no sequences: a no-op
    assert st == B.GDN_OK


def test_mixed_step_validation():
    lib = B.library()
    shape = B.make_shape(2, 4, 64, 64, B.GDN_BF16, 0.125)
    # decode part checked first: slot_out NULL
    st = lib.gdn_mixed_step(ctypes.byref(shape), 3, FAKE, None, 1, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, 8, FAKE, FAKE, None, 0, None, None, None, 0, FAKE, 0, None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "slot_out is NULL" in B.gdn_last_error()
    # prefill part: export grid off the chunk grid (init_slot NULL as the guard)
    st = lib.gdn_mixed_step(ctypes.byref(shape), 3, FAKE, FAKE, 1, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, 8, None, FAKE, None, 100, FAKE, FAKE, None, 1, FAKE, 0, None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "export_grid 100" in B.gdn_last_error()
    # prefill part: a NULL init_slot
    st = lib.gdn_mixed_step(ctypes.byref(shape), 3, FAKE, FAKE, 1, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            FAKE, FAKE, 8, None, FAKE, None, 0, None, None, None, 0, FAKE, 0, None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "init_slot is NULL" in B.gdn_last_error()


def test_verify_validation():
    lib = B.library()
    shape = B.make_shape(2, 4, 64, 64, B.GDN_BF16, 0.125)
    st = lib.gdn_recurrent_verify(ctypes.byref(shape), 3, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE,
                                  FAKE, None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "tokens_per_row 0" in B.gdn_last_error()
    st = lib.gdn_recurrent_verify(ctypes.byref(shape), 3, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE,
                                  None, None)
    assert st == B.GDN_ERR_INVALID_ARGUMENT and "is NULL" in B.gdn_last_error()
    st = lib.gdn_recurrent_verify(ctypes.byref(shape), 0, 4, None, None, None, None, None, None, None, 0, None,
                                  None, None)
    assert st == B.GDN_OK                          # no rows: a no-op


def test_binding_checks_tensors_before_calling():
    import torch
    q = torch.zeros(2, 1, 64)
    with pytest.raises(ValueError):
        B.gdn_recurrent_decode(q, q, q, torch.zeros(2, 1), torch.zeros(2, 1), q, torch.zeros(1, 1, 64, 64),
                               torch.zeros(2, dtype=torch.int32), torch.zeros(2, dtype=torch.int32), scale=1.0)
    assert B.export_offsets([100, 64, 0, 1200], [0, 64, 5, 1000], 64) == [0, 1, 2, 2, 21]
