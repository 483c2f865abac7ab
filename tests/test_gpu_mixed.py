"""The mixed step on the GPU ("[Model] Enable batch-invariant mixed decode and prefill
for Qwen GDN", sections "How" and "Results": cached decode rows at the front of a
mixed step take the same packed decode path as a decode-only step, so their output
and updated state are bitwise equal with atol = rtol = 0)."""
import numpy as np
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import TOL, assert_close, check_prefill, decode_reference, prefill_reference, to_device

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


def _mixed(w, d, pool, o, export=False):
    N, T = w.num_seqs, w.prefill_tokens
    ws = binding.alloc_workspace(w.H_v, d["q"].dtype, N, T, "cuda")
    kw = {}
    if export and w.export_grid:
        offs = binding.export_offsets(w.lengths, None, w.export_grid)
        kw = dict(export_grid=w.export_grid, export_offsets=_i32(offs),
                  export_states=torch.full((max(offs[-1], 1), w.H_v, w.d_k, w.d_v), float("nan"), device="cuda"))
    binding.gdn_mixed_step(d["q"], d["k"], d["v"], d["g"], d["beta"], o, pool, d["slot_in"], d["slot_out"],
                           d["cu"], d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws, **kw)
    return kw.get("export_states")


def test_mixed_step_decode_rows_bitwise_equal_decode_only():
    """The mixed step of 32 cached rows ahead of prefills of 116, 321, 1059 and 2000
    tokens: its decode rows equal a decode-only call bitwise, its prefills equal a
    prefill-only call bitwise, and both match the oracle."""
    w = W.config(3)
    d = to_device(w)
    B = w.num_decode_rows
    pool0 = d["pool"].clone()

    o_mixed = torch.empty_like(d["v"])
    _mixed(w, d, d["pool"], o_mixed)
    torch.cuda.synchronize()
    pool_mixed = d["pool"].clone()

    # decode-only on the same rows, from the same cache
    pool_dec = pool0.clone()
    o_dec = torch.empty_like(d["v"][:B])
    binding.gdn_recurrent_decode(d["q"][:B], d["k"][:B], d["v"][:B], d["g"][:B], d["beta"][:B], o_dec, pool_dec,
                                 d["slot_in"], d["slot_out"], scale=w.scale)
    # prefill-only on the rest
    pool_pre = pool0.clone()
    o_pre = torch.empty_like(d["v"][B:])
    ws = binding.alloc_workspace(w.H_v, torch.bfloat16, w.num_seqs, w.prefill_tokens, "cuda")
    binding.gdn_chunk_prefill(d["q"][B:], d["k"][B:], d["v"][B:], d["g"][B:], d["beta"][B:], o_pre, d["cu"],
                              pool_pre, d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws)
    torch.cuda.synchronize()

    assert torch.equal(o_mixed[:B], o_dec)
    dec_slots = torch.from_numpy(w.slot_out).long().cuda()
    assert torch.equal(pool_mixed[dec_slots], pool_dec[dec_slots])
    assert torch.equal(o_mixed[B:], o_pre)
    fin = torch.from_numpy(w.final_slot).long().cuda()
    assert torch.equal(pool_mixed[fin], pool_pre[fin])
    # slots named by neither part are untouched
    named = set(int(x) for x in w.slot_out) | set(int(x) for x in w.final_slot)
    rest = torch.tensor([s for s in range(w.pool.shape[0]) if s not in named], device="cuda")
    assert torch.equal(pool_mixed[rest], pool0[rest])

    # and against the oracle: every decode row, every prefill chain (one oracle call)
    atol, rtol = TOL["bf16"]
    ref_o, ref_s = decode_reference(w)
    assert_close("decode o", o_mixed[:B].float().cpu().numpy(), ref_o, atol, rtol)
    assert_close("decode states", pool_mixed[dec_slots].cpu().numpy(), ref_s, atol, rtol)
    check_prefill(w, prefill_reference(w), o_mixed[B:], pool_mixed, tag="prefill ")


@pytest.mark.parametrize("decode_rows,lengths", [(0, [70, 5]), (9, []), (5, [0, 64, 1])])
def test_mixed_step_edges(decode_rows, lengths):
    """No decode rows, no prefills, and zero-length prefills all route correctly."""
    w = W.make_workload("edge", seed=31, H_k=2, H_v=4, d_k=64, d_v=64, dtype="bf16", num_decode_rows=decode_rows,
                        lengths=lengths, num_slots=40)
    d = to_device(w)
    o = torch.empty_like(d["v"])
    _mixed(w, d, d["pool"], o)
    torch.cuda.synchronize()
    atol, rtol = TOL["bf16"]
    B = decode_rows
    if B:
        ref_o, ref_s = decode_reference(w)
        assert_close("decode o", o[:B].float().cpu().numpy(), ref_o, atol, rtol)
        assert_close("decode states", d["pool"][torch.from_numpy(w.slot_out).long().cuda()].cpu().numpy(), ref_s,
                     atol, rtol)
    if lengths:
        check_prefill(w, prefill_reference(w), o[B:], d["pool"])


def test_mixed_step_with_exports_and_resume_from_cache():
    """Cached decode rows ahead of a prefill that resumes from a cached state at an
    absolute start position and exports on the 1088 grid."""
    w = W.make_workload("mx", seed=32, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16", num_decode_rows=7,
                        lengths=[1500, 300], num_slots=40, prefill_init="slots", start_pos=[1088, 0],
                        export_grid=1088)
    d = to_device(w)
    o = torch.empty_like(d["v"])
    N, T = w.num_seqs, w.prefill_tokens
    ws = binding.alloc_workspace(w.H_v, torch.bfloat16, N, T, "cuda")
    offs = binding.export_offsets(w.lengths, list(w.start_pos), 1088)
    exp_states = torch.full((max(offs[-1], 1), w.H_v, w.d_k, w.d_v), float("nan"), device="cuda")
    binding.gdn_mixed_step(d["q"], d["k"], d["v"], d["g"], d["beta"], o, d["pool"], d["slot_in"], d["slot_out"],
                           d["cu"], d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws,
                           start_pos=d["start_pos"], export_grid=1088, export_offsets=_i32(offs),
                           export_states=exp_states)
    torch.cuda.synchronize()
    assert offs == [0, 1, 1]          # 1088 + 1500 crosses 2176 once; 300 tokens from 0 cross nothing
    check_prefill(w, prefill_reference(w), o[w.num_decode_rows:], d["pool"], exp_states)


def test_mixed_step_on_a_side_stream():
    """A call enqueues on the stream it is given: the mixed step issued on a side
    stream (inputs made ready by an event, results read after the stream is synchronised)
    equals the same step on the default stream bitwise."""
    w = W.make_workload("side", seed=31, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16", num_decode_rows=5,
                        lengths=[130, 64, 7], num_slots=24, export_grid=64)
    d = to_device(w)
    pool0 = d["pool"].clone()
    o_ref = torch.empty_like(d["v"])
    exp_ref = _mixed(w, d, d["pool"], o_ref, export=True)
    torch.cuda.synchronize()
    pool_ref = d["pool"].clone()

    d["pool"].copy_(pool0)
    o_side = torch.full_like(d["v"], float("nan"))
    ready = torch.cuda.Event()
    ready.record()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        side.wait_event(ready)
        exp_side = _mixed(w, d, d["pool"], o_side, export=True)
    side.synchronize()
    assert torch.equal(o_side, o_ref)
    assert torch.equal(d["pool"], pool_ref)
    assert torch.equal(exp_side, exp_ref)
