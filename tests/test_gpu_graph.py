"""The hot path under HIP-graph capture.

A serving loop replays decode as one captured graph and steps that contain prefills as
piecewise graphs, over static buffers sized for the largest decode batch ("[V1][Hybrid]
GatedDeltaNet Automatic Prefix Caching", sections "TODOs" and "Test Result", and its
review comments on the decode graph buffers).  Every entry point here only enqueues
kernels on the caller's stream (no allocation, no synchronisation, no memset), so a call
can be captured once over static buffers and replayed with new contents; padding rows
(slot -1) let one decode graph serve any smaller batch.  Each test replays several times,
with eager work and synchronisations between replays, and checks every replay bitwise
against the same call made eagerly, and one replay against the oracle."""
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import TOL, assert_close, decode_reference, prefill_reference, to_device

pytestmark = pytest.mark.gpu


def _fill(dst: dict, src: dict):
    for name, t in src.items():
        if t is not None and name in dst:
            dst[name].copy_(t)


def test_decode_graph_replays_match_eager():
    """A decode graph captured for 64 rows, replayed for batches of 64, 40 and 17 live
    rows (the rest padding rows with slot -1), each replay bitwise equal to the eager
    call on the same inputs."""
    B = 64
    base = W.config(1)
    static = to_device(base)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        binding.gdn_recurrent_decode(static["q"], static["k"], static["v"], static["g"], static["beta"],
                                     static["o"], static["pool"], static["slot_in"], static["slot_out"],
                                     scale=base.scale)
    torch.cuda.synchronize()
    atol, rtol = TOL["bf16"]
    for rep, live in enumerate((64, 40, 17)):
        w = W.make_workload("graph%d" % rep, seed=2000 + rep, H_k=16, H_v=32, d_k=128, d_v=128, dtype="bf16",
                            num_decode_rows=B, num_slots=256)
        w.slot_in[live:] = -1
        w.slot_out[live:] = -1
        d = to_device(w)
        _fill(static, d)
        eager_pool = d["pool"].clone()
        eager_o = torch.empty_like(d["o"])
        binding.gdn_recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], eager_o, eager_pool,
                                     d["slot_in"], d["slot_out"], scale=w.scale)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(static["o"], eager_o), "replay %d: o differs from the eager call" % rep
        assert torch.equal(static["pool"], eager_pool), "replay %d: states differ from the eager call" % rep
        assert torch.all(static["o"][live:] == 0)
        if rep == 0:
            ref_o, ref_s = decode_reference(w)
            assert_close("graph decode o", static["o"].float().cpu().numpy(), ref_o, atol, rtol)
            slots = torch.from_numpy(w.slot_out).long().cuda()
            assert_close("graph decode states", static["pool"][slots].cpu().numpy(), ref_s, atol, rtol)


def test_mixed_step_graph_replays_match_eager():
    """A mixed step (8 decode rows ahead of 3 prefills, 600 prefill tokens in all) captured
    once and replayed with new values and a different split of the 600 tokens between the
    sequences (cu_seqlens is a device tensor, so the same graph serves any split)."""
    def workload(seed, lengths):
        return W.make_workload("mg%d" % seed, seed=seed, H_k=4, H_v=8, d_k=128, d_v=128, dtype="bf16",
                               num_decode_rows=8, lengths=lengths, num_slots=40, prefill_init="slots",
                               start_pos=[64, 0, 1088], export_grid=64)
    base = workload(3000, [200, 300, 100])
    static = to_device(base)
    offs = binding.export_offsets(base.lengths, list(base.start_pos), 64)
    cap = 16
    exp_static = torch.zeros((cap, base.H_v, base.d_k, base.d_v), device="cuda")
    offs_static = torch.zeros(len(offs), dtype=torch.int32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    kw = dict(scale=base.scale, start_pos=static["start_pos"], export_grid=64, export_states=exp_static,
              export_offsets=offs_static)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        binding.gdn_mixed_step(static["q"], static["k"], static["v"], static["g"], static["beta"], static["o"],
                               static["pool"], static["slot_in"], static["slot_out"], static["cu"],
                               static["init_slot"], static["final_slot"], **kw)
    torch.cuda.synchronize()
    atol, rtol = TOL["bf16"]
    for rep, lengths in enumerate(([200, 300, 100], [64, 500, 36], [599, 1, 0])):
        w = workload(3001 + rep, lengths)
        d = to_device(w)
        _fill(static, d)
        o_ = binding.export_offsets(w.lengths, list(w.start_pos), 64)
        offs_static.copy_(torch.tensor(o_, dtype=torch.int32))
        exp_static.zero_()
        eager_pool = d["pool"].clone()
        eager_o = torch.empty_like(d["o"])
        eager_exp = torch.zeros_like(exp_static)
        binding.gdn_mixed_step(d["q"], d["k"], d["v"], d["g"], d["beta"], eager_o, eager_pool, d["slot_in"],
                               d["slot_out"], d["cu"], d["init_slot"], d["final_slot"], scale=w.scale,
                               start_pos=d["start_pos"], export_grid=64, export_states=eager_exp,
                               export_offsets=offs_static)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(static["o"], eager_o), "replay %d: o differs from the eager call" % rep
        assert torch.equal(static["pool"], eager_pool), "replay %d: states differ from the eager call" % rep
        assert torch.equal(exp_static, eager_exp), "replay %d: exports differ from the eager call" % rep
        if rep == 1:
            ref = prefill_reference(w)
            cu = w.cu_seqlens() + w.num_decode_rows
            for i in range(w.num_seqs):
                for h in range(w.H_v):
                    ro, rf, rexp = ref[(i, h)]
                    assert_close("graph o %d/%d" % (i, h), static["o"][cu[i]:cu[i + 1], h].float().cpu().numpy(),
                                 ro, atol, rtol)
                    assert_close("graph final %d/%d" % (i, h),
                                 static["pool"][int(w.final_slot[i]), h].cpu().numpy(), rf, atol, rtol)
                    got = exp_static[o_[i]:o_[i + 1], h].cpu().numpy()
                    assert_close("graph exports %d/%d" % (i, h), got, rexp, atol, rtol)
