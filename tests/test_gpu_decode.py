"""Decode on the GPU: parity with the fp64 oracle, bitwise batch invariance, slot
semantics and determinism ("[Model] Enable batch-invariant mixed decode and prefill
for Qwen GDN", sections "How" and "Results": a cached row's output and updated state
do not depend on the batch it runs in)."""
import numpy as np
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import TOL, assert_close, decode_reference, to_device

pytestmark = pytest.mark.gpu


def _decode(d, rows=None, slot_in=None, slot_out=None, w=None):
    idx = slice(None) if rows is None else torch.as_tensor(rows, device="cuda", dtype=torch.long)
    q, k, v, g, b = (d[x][idx].contiguous() for x in ("q", "k", "v", "g", "beta"))
    si = d["slot_in"][idx].contiguous() if slot_in is None else torch.as_tensor(slot_in, dtype=torch.int32, device="cuda")
    so = si.clone() if slot_out is None else torch.as_tensor(slot_out, dtype=torch.int32, device="cuda")
    o = torch.empty_like(v)
    binding.gdn_recurrent_decode(q, k, v, g, b, o, d["pool"], si, so, scale=w.scale)
    return o


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", [("bf16", 128, 128, 16, 32), ("f32", 128, 128, 16, 32),
                                               ("bf16", 64, 64, 2, 4), ("f32", 64, 128, 1, 3),
                                               ("bf16", 128, 64, 4, 4)])
def test_decode_parity(dtype, dk, dv, hk, hv):
    """Every row, every head, output and updated state, within the dtype's bound."""
    if (dtype, dk, dv, hk, hv) == ("bf16", 128, 128, 16, 32):
        w = W.config(1)                              # the standard decode batch, B = 64
    else:
        w = W.make_workload("dec", seed=7, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype,
                            num_decode_rows=37, num_slots=96)
    d = to_device(w)
    o = _decode(d, w=w)
    torch.cuda.synchronize()
    ref_o, ref_s = decode_reference(w)
    atol, rtol = TOL[dtype]
    assert_close("o", o.float().cpu().numpy(), ref_o, atol, rtol)
    assert_close("state", d["pool"][torch.from_numpy(w.slot_out).long().cuda()].cpu().numpy(), ref_s, atol, rtol)
    # slots that no row names are bitwise untouched
    untouched = np.setdiff1d(np.arange(w.pool.shape[0]), w.slot_out)
    assert torch.equal(d["pool"][torch.from_numpy(untouched).long().cuda()].cpu(),
                       torch.from_numpy(w.pool[untouched]))


def test_decode_batch_invariance():
    """The same rows alone, in batches of 2, 3, 7, 64 and 255, at different positions
    and from different slots: outputs and states bitwise identical."""
    w = W.make_workload("bi", seed=11, H_k=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                        num_decode_rows=255, num_slots=520)
    d = to_device(w)
    pool0 = d["pool"].clone()
    probe = [0, 17, 254]
    alone_o, alone_s = {}, {}
    for r in probe:
        d["pool"].copy_(pool0)
        o = _decode(d, rows=[r], w=w)
        alone_o[r] = o[0].clone()
        alone_s[r] = d["pool"][int(w.slot_out[r])].clone()
    rng = np.random.default_rng(5)
    for size in (2, 3, 7, 64, 255):
        others = [x for x in rng.permutation(255) if x not in probe][:size - len(probe)] if size > 3 else []
        rows = list(probe[:size]) + others
        rng.shuffle(rows)
        d["pool"].copy_(pool0)
        o = _decode(d, rows=rows, w=w)
        for pos, r in enumerate(rows):
            if r in alone_o:
                assert torch.equal(o[pos], alone_o[r]), (size, r)
                assert torch.equal(d["pool"][int(w.slot_out[r])], alone_s[r]), (size, r)
    # the same row read from another slot and written to a third gives the same bits
    d["pool"].copy_(pool0)
    src, dst = 300, 301
    d["pool"][src] = pool0[int(w.slot_in[17])]
    o = _decode(d, rows=[17], slot_in=[src], slot_out=[dst], w=w)
    assert torch.equal(o[0], alone_o[17])
    assert torch.equal(d["pool"][dst], alone_s[17])
    assert torch.equal(d["pool"][src], pool0[int(w.slot_in[17])])


def test_decode_padding_and_slots():
    """slot_in outside [0, num_slots) is padding: zero output, no state touched;
    slot_out outside the range computes the output but writes no state."""
    w = W.make_workload("pad", seed=12, H_k=2, H_v=4, d_k=64, d_v=64, dtype="bf16", num_decode_rows=6,
                        num_slots=16)
    d = to_device(w)
    pool0 = d["pool"].clone()
    si = np.array([3, -1, 5, 16, 7, 9], dtype=np.int32)
    so = np.array([3, 2, 11, 4, -1, 1 << 20], dtype=np.int32)
    o = _decode(d, slot_in=si, slot_out=so, w=w)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 0) and torch.all(o[3] == 0)
    changed = {3, 11}
    for s in range(16):
        if s not in changed:
            assert torch.equal(d["pool"][s], pool0[s]), s
    w2 = W.make_workload("pad", seed=12, H_k=2, H_v=4, d_k=64, d_v=64, dtype="bf16", num_decode_rows=6,
                         num_slots=16)
    w2.slot_in = np.array([3, -1, 5, -1, 7, 9], dtype=np.int32)
    ref_o, ref_s = decode_reference(w2)
    atol, rtol = TOL["bf16"]
    for r in (0, 2, 4, 5):
        assert_close("o row %d" % r, o[r].float().cpu().numpy(), ref_o[r], atol, rtol)
    assert_close("state 3", d["pool"][3].cpu().numpy(), ref_s[0], atol, rtol)
    assert_close("state 11", d["pool"][11].cpu().numpy(), ref_s[2], atol, rtol)


def test_decode_deterministic():
    w = W.make_workload("det", seed=13, H_k=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                        num_decode_rows=64, num_slots=128)
    d = to_device(w)
    pool0 = d["pool"].clone()
    first_o = first_pool = None
    for _ in range(20):
        d["pool"].copy_(pool0)
        o = _decode(d, w=w)
        if first_o is None:
            first_o, first_pool = o.clone(), d["pool"].clone()
        else:
            assert torch.equal(o, first_o) and torch.equal(d["pool"], first_pool)


def test_decode_zero_rows():
    w = W.make_workload("z", seed=1, H_k=1, H_v=1, d_k=64, d_v=64, dtype="bf16", num_decode_rows=1, num_slots=8)
    d = to_device(w)
    pool0 = d["pool"].clone()
    e = torch.empty(0, 1, 64, dtype=torch.bfloat16, device="cuda")
    binding.gdn_recurrent_decode(e, e, e, torch.empty(0, 1, device="cuda"), torch.empty(0, 1, device="cuda"),
                                 e.clone(), d["pool"], torch.empty(0, dtype=torch.int32, device="cuda"),
                                 torch.empty(0, dtype=torch.int32, device="cuda"), scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(d["pool"], pool0)


def test_decode_exact_recall():
    """g = 0, beta = 1, a basis key as key and query, zero state: the row stores v and
    reads it back bit-exactly (every product is 0 or 1)."""
    w = W.make_workload("rec", seed=14, H_k=1, H_v=1, d_k=64, d_v=64, dtype="bf16", num_decode_rows=1,
                        num_slots=4)
    d = to_device(w)
    d["pool"].zero_()
    k = torch.zeros(1, 1, 64, dtype=torch.bfloat16, device="cuda")
    k[0, 0, 5] = 1
    g = torch.zeros(1, 1, device="cuda")
    b = torch.ones(1, 1, device="cuda")
    o = torch.empty_like(d["v"])
    si = torch.tensor([1], dtype=torch.int32, device="cuda")
    binding.gdn_recurrent_decode(k, k, d["v"], g, b, o, d["pool"], si, si, scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(o, d["v"])
    assert torch.equal(d["pool"][1, 0, 5], d["v"][0, 0].float())
