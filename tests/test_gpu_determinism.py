"""Run-to-run determinism on the GPU: the same call on the same inputs gives bitwise the
same outputs, final states and exported states every time.

A sequence's results may not depend on timing ("[Model] Enable batch-invariant mixed
decode and prefill for Qwen GDN", section "Why": the results must not change with how
a step is scheduled; "[WIP][Kernel] Enable GDN batch-invariant prefix caching",
section "Purpose": a resumed request reproduces the same states).  The gates here are
scaled down (weak decay), so that a difference anywhere in a sequence would survive
to its final state instead of being decayed away."""
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import to_device

pytestmark = pytest.mark.gpu

REPEATS = 3


def _i32(a):
    return torch.as_tensor(a, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("dtype,H_k,H_v,d_k,d_v", [("bf16", 16, 32, 128, 128),   # two value heads per group
                                                   ("bf16", 4, 4, 128, 64),      # one value head per group
                                                   ("bf16", 2, 4, 64, 128),
                                                   ("bf16", 3, 3, 64, 64),
                                                   ("f32", 2, 4, 64, 128)])
def test_prefill_repeats_are_bitwise_identical(dtype, H_k, H_v, d_k, d_v):
    w = W.make_workload("det", seed=61, H_k=H_k, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype,
                        lengths=[2048, 1000, 77, 640], num_slots=16, export_grid=64)
    w.g *= 0.05
    d = to_device(w)
    offs = binding.export_offsets(w.lengths, None, 64)
    runs = []
    for _ in range(REPEATS):
        pool = d["pool"].clone()
        o = torch.empty_like(d["o"])
        exp = torch.zeros((offs[-1], H_v, d_k, d_v), device="cuda")
        binding.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], o, d["cu"], pool, d["init_slot"],
                                  d["final_slot"], scale=w.scale, export_grid=64, export_states=exp,
                                  export_offsets=_i32(offs))
        torch.cuda.synchronize()
        runs.append((o, pool, exp))
    o0, p0, e0 = runs[0]
    for r, (o, p, e) in enumerate(runs[1:], 1):
        assert torch.equal(o, o0), "run %d: outputs differ from run 0" % r
        assert torch.equal(p, p0), "run %d: final states differ from run 0" % r
        assert torch.equal(e, e0), "run %d: exported states differ from run 0" % r


def test_decode_and_verify_repeats_are_bitwise_identical():
    w = W.make_workload("detd", seed=62, H_k=16, H_v=32, d_k=128, d_v=128, dtype="bf16", num_decode_rows=96,
                        num_slots=256)
    d = to_device(w)
    outs = []
    for _ in range(REPEATS):
        pool = d["pool"].clone()
        o = torch.empty_like(d["o"])
        binding.gdn_recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], o, pool, d["slot_in"],
                                     d["slot_out"], scale=w.scale)
        pool_v = d["pool"].clone()
        o_v = torch.empty_like(d["o"])
        slot_in = torch.arange(0, 96, 3, dtype=torch.int32, device="cuda")          # 32 rows of 3 tokens
        token_slots = torch.arange(128, 224, dtype=torch.int32, device="cuda")   # disjoint from slot_in
        binding.gdn_recurrent_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], o_v, pool_v, slot_in, token_slots,
                                     scale=w.scale, tokens_per_row=3)
        torch.cuda.synchronize()
        outs.append((o, pool, o_v, pool_v))
    for r, run in enumerate(outs[1:], 1):
        for name, x, x0 in zip(("decode o", "decode states", "verify o", "verify states"), run, outs[0]):
            assert torch.equal(x, x0), "run %d: %s differ from run 0" % (r, name)
