"""Chunked prefill on the GPU: parity with the fp64 oracle on every output row, final
state and export (one oracle call per workload, full-size workloads included),
exported states on the grid,
resume from an exported state, per-sequence batch invariance, slot semantics and
determinism.

Pages: "[V1][Hybrid] GatedDeltaNet Automatic Prefix Caching", section "Purpose"
(intermediate chunk states as one flat stream); "[WIP][Kernel] Enable GDN
batch-invariant prefix caching", sections "Purpose" and "Test Result" (one
lcm(64, block) grid; a 1100-token prefix resumes from 1088, a 200-token one from 0;
a hit at batch size 1 and N is bitwise identical)."""
import numpy as np
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import check_prefill, prefill_reference, run_prefill, to_device

pytestmark = pytest.mark.gpu


def test_prefill_single_sequence_fp32():
    """The single-sequence fp32 case (T = 256, d = 64) at 1e-5."""
    w = W.config(0)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", [("bf16", 128, 128, 2, 4), ("f32", 64, 64, 1, 2),
                                               ("bf16", 64, 128, 1, 1), ("f32", 128, 64, 2, 2),
                                               ("bf16", 64, 64, 3, 6),
                                               # the remaining bf16 kernel shapes: two value
                                               # heads per workgroup (even group size) or one
                                               # (odd: 1 or 3 value heads per key head)
                                               ("bf16", 128, 64, 2, 4), ("bf16", 128, 64, 1, 3),
                                               ("bf16", 128, 128, 3, 3), ("bf16", 64, 64, 2, 2),
                                               ("bf16", 64, 128, 2, 4)])
def test_prefill_varlen_ragged(dtype, dk, dv, hk, hv):
    """Ragged lengths (1, 63, 64, 65, 130, 200, 0), initial states from slots,
    start positions on and off the 64 grid, exports every 64 tokens; every
    instantiation of the bf16 kernel (d_k, d_v in {64, 128}, one or two value heads
    per workgroup)."""
    lengths = [1, 63, 64, 65, 130, 200, 0]
    starts = [0, 64, 5, 1000, 128, 33, 7]
    w = W.make_workload("rag", seed=21, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=lengths,
                        num_slots=32, prefill_init="slots", start_pos=starts, export_grid=64)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)


@pytest.mark.parametrize("dtype,dk,dv,hk,hv,key_mix,gate_scale,beta_shift", [
    ("bf16", 128, 128, 2, 4, 3.0, 0.01, 2.0),   # keys with cosine near 0.9, almost no decay, beta near 0.85
    ("bf16", 128, 128, 2, 4, 3.0, 0.0, 3.0),    # no decay at all, beta near 0.95
    ("bf16", 64, 64, 2, 4, 3.0, 0.01, 2.0),
    ("bf16", 128, 128, 2, 4, 1.0, 0.1, 0.0),    # cosine near 0.5, slow decay
    # the other bf16 kernel shapes: d_k != d_v, one value head per workgroup (odd group)
    ("bf16", 128, 64, 2, 4, 3.0, 0.0, 3.0),
    ("bf16", 64, 128, 2, 4, 3.0, 0.0, 3.0),
    ("bf16", 128, 128, 1, 3, 3.0, 0.0, 3.0),
    ("bf16", 64, 64, 1, 3, 3.0, 0.01, 2.0),
    ("f32", 128, 128, 2, 4, 3.0, 0.01, 2.0),
    ("f32", 64, 64, 2, 4, 3.0, 0.0, 3.0)])
def test_prefill_stress_inputs(dtype, dk, dv, hk, hv, key_mix, gate_scale, beta_shift):
    """Inputs that make the in-chunk triangular system ill-conditioned: highly
    correlated keys (so K K^T is near rank one and I + A has large off-diagonal
    entries), gates near zero (nothing in D damps them) and beta near one.  The
    split-precision solve must still meet the same per-element bound as on the
    standard inputs, for outputs, final states and every export."""
    lengths = [700, 64, 1, 333, 129]
    w = W.make_workload("stress", seed=28, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=lengths,
                        num_slots=24, prefill_init="slots", export_grid=64, key_mix=key_mix,
                        gate_scale=gate_scale, beta_shift=beta_shift)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)


def test_prefill_canaries():
    """Slots no sequence names stay bitwise unchanged, rows past the packed tokens of o
    and export rows past the last grid point are never written."""
    lengths = [100, 1, 257]
    w = W.make_workload("can", seed=22, H_k=2, H_v=4, d_k=64, d_v=64, dtype="bf16", lengths=lengths,
                        num_slots=20, export_grid=64)
    d = to_device(w)
    T = w.total_tokens
    pool0 = d["pool"].clone()
    big_o = torch.full((T + 9, 4, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    d["o"] = big_o[:T]
    ws = binding.alloc_workspace(4, torch.bfloat16, 3, T, "cuda")
    offs = binding.export_offsets(lengths, None, 64)
    exp_offs = torch.tensor(offs, dtype=torch.int32, device="cuda")
    exp_states = torch.full((offs[-1] + 3, 4, 64, 64), float("nan"), device="cuda")
    binding.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["o"], d["cu"], d["pool"],
                              d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws, export_grid=64,
                              export_states=exp_states, export_offsets=exp_offs)
    torch.cuda.synchronize()
    assert torch.isnan(big_o[T:].float()).all()
    assert not torch.isnan(big_o[:T].float()).any()
    assert torch.isnan(exp_states[offs[-1]:]).all()
    assert not torch.isnan(exp_states[:offs[-1]]).any()
    named = set(int(x) for x in w.final_slot)
    for s in range(20):
        if s not in named:
            assert torch.equal(d["pool"][s], pool0[s]), s


def test_prefill_export_capacity_bound():
    """An export buffer smaller than the stream: the kernels drop what does not fit."""
    lengths = [300]
    w = W.make_workload("cap", seed=23, H_k=1, H_v=2, d_k=64, d_v=64, dtype="bf16", lengths=lengths,
                        num_slots=4, export_grid=64)
    d = to_device(w)
    ws = binding.alloc_workspace(2, torch.bfloat16, 1, 300, "cuda")
    exp_offs = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    storage = torch.full((4, 2, 64, 64), float("nan"), device="cuda")
    binding.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["o"], d["cu"], d["pool"],
                              d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws, export_grid=64,
                              export_states=storage[:2], export_offsets=exp_offs)
    torch.cuda.synchronize()
    assert not torch.isnan(storage[:2]).any() and torch.isnan(storage[2:]).all()


def test_prefill_batch_invariance():
    """A sequence alone and at several positions of a varlen batch: bitwise equal
    outputs, final states and exports."""
    base = W.make_workload("bi", seed=24, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16",
                           lengths=[333, 64, 1000, 17, 512], num_slots=16, export_grid=64)
    dbase = to_device(base)
    exp_all, _ = run_prefill(base, dbase)
    cu = base.cu_seqlens()
    offs = binding.export_offsets(base.lengths, None, 64)
    for i in (0, 2, 3):
        a, b = int(cu[i]), int(cu[i + 1])
        solo = W.make_workload("bi1", seed=24, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16",
                               lengths=[b - a], num_slots=16, export_grid=64)
        for name in ("q", "k", "v", "g", "beta"):
            setattr(solo, name, getattr(base, name)[a:b].copy())
        solo.final_slot = np.array([3], dtype=np.int32)
        dsolo = to_device(solo)
        exp_solo, _ = run_prefill(solo, dsolo)
        torch.cuda.synchronize()
        assert torch.equal(dsolo["o"], dbase["o"][a:b]), i
        assert torch.equal(dsolo["pool"][3], dbase["pool"][int(base.final_slot[i])]), i
        n_i = offs[i + 1] - offs[i]
        assert torch.equal(exp_solo[:n_i], exp_all[offs[i]:offs[i + 1]]), i


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64),
                                         ("f32", 128, 128), ("f32", 64, 64)])
def test_prefill_launch_shapes_are_bitwise_equal(dtype, dk, dv):
    """With two value heads per key head the bf16 kernel gives each workgroup both
    heads when the call has enough (sequence, key head) pairs to fill the compute
    units, one head with 32-column strips when its (sequence, value head) chains
    outnumber the compute units, one head with 16-column strips when they do not, and
    (d_v 128) half a head's strips when the chains are at most half the compute units.
    The same sequences alone (half heads at d_v 128, else 16-column strips), in a batch
    of as many chains as compute units (16-column strips), in a middling batch
    (32-column strips, one head) and inside a batch that fills the GPU (two heads per
    workgroup) give bitwise equal outputs, final states and exports.  The fp32 kernel
    has one head per workgroup and the two strip widths, chosen the same way."""
    H_k, H_v = 16, 32
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = -(-cus // H_k)                               # sequences for a full launch of head pairs
    rng = np.random.default_rng(33)
    lengths = [int(x) for x in rng.integers(1, 400, size=n)]
    lengths[0], lengths[-1] = 333, 130
    base = W.make_workload("shape", seed=33, H_k=H_k, H_v=H_v, d_k=dk, d_v=dv, dtype=dtype, lengths=lengths,
                           num_slots=2 * n + 4, prefill_init="slots", export_grid=64)
    dbase = to_device(base)
    exp_all, _ = run_prefill(base, dbase)
    cu = base.cu_seqlens()
    offs = binding.export_offsets(base.lengths, None, 64)
    for i in (0, n // 2, n - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        solo = W.make_workload("shape1", seed=33, H_k=H_k, H_v=H_v, d_k=dk, d_v=dv, dtype=dtype, lengths=[b - a],
                               num_slots=2 * n + 4, export_grid=64)
        for name in ("q", "k", "v", "g", "beta"):
            setattr(solo, name, getattr(base, name)[a:b].copy())
        solo.pool = base.pool
        solo.init_slot = base.init_slot[i:i + 1].copy()
        solo.final_slot = np.array([2 * n + 3], dtype=np.int32)
        dsolo = to_device(solo)
        exp_solo, _ = run_prefill(solo, dsolo)
        torch.cuda.synchronize()
        assert torch.equal(dsolo["o"], dbase["o"][a:b]), i
        assert torch.equal(dsolo["pool"][2 * n + 3], dbase["pool"][int(base.final_slot[i])]), i
        n_i = offs[i + 1] - offs[i]
        assert torch.equal(exp_solo[:n_i], exp_all[offs[i]:offs[i + 1]]), i
    # the first m sequences: as many chains as compute units (16-column strips), then
    # more chains than compute units and fewer head pairs (32-column strips)
    m16, m = cus // H_v, cus // H_v + 1
    assert cus < 2 * m16 * H_v <= 2 * cus
    assert m * H_v > cus and m * H_k < cus and m < n
    for tag, mm in (("shape16", m16), ("shape2", m)):
        mid = W.make_workload(tag, seed=33, H_k=H_k, H_v=H_v, d_k=dk, d_v=dv, dtype=dtype, lengths=lengths[:mm],
                              num_slots=2 * n + 4, export_grid=64)
        b = int(cu[mm])
        for name in ("q", "k", "v", "g", "beta"):
            setattr(mid, name, getattr(base, name)[:b].copy())
        mid.pool = base.pool
        mid.init_slot = base.init_slot[:mm].copy()
        mid.final_slot = base.final_slot[:mm].copy()
        dmid = to_device(mid)
        exp_mid, _ = run_prefill(mid, dmid)
        torch.cuda.synchronize()
        assert torch.equal(dmid["o"], dbase["o"][:b]), tag
        fin = torch.as_tensor(mid.final_slot, device=dmid["pool"].device).long()
        assert torch.equal(dmid["pool"][fin], dbase["pool"][fin]), tag
        assert torch.equal(exp_mid[:offs[mm]], exp_all[:offs[mm]]), tag
    # and the full batch against the oracle
    check_prefill(base, prefill_reference(base), dbase["o"], dbase["pool"], exp_all)


def test_prefill_deterministic():
    w = W.make_workload("det", seed=25, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16",
                        lengths=[700, 129, 64], num_slots=16, export_grid=128)
    d = to_device(w)
    first = None
    for _ in range(10):
        exp_states, _ = run_prefill(w, d)
        snap = (d["o"].clone(), d["pool"].clone(), exp_states.clone())
        if first is None:
            first = snap
        else:
            assert all(torch.equal(x, y) for x, y in zip(snap, first))


def test_prefill_cfg2_full():
    """The varlen batch (8 sequences, lengths in [64, 4096], 16/32 heads, d = 128,
    bf16, exports every 64 tokens) at full size: every output row, final state and
    export of every (sequence, value head) chain against one oracle call."""
    w = W.config(2, fill_pool=False)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)


def test_prefill_cfg4_full_and_resume():
    """Long prefill (16 x 8192, export grid 1088 = lcm(64, 1088)) at full size: every
    chain against one oracle call, then a resume from the exported state at 4352 =
    4 x 1088 reproduces the rest of the run bitwise."""
    w = W.config(4, fill_pool=False)
    d = to_device(w)
    exp_states, exp_offs = run_prefill(w, d)
    torch.cuda.synchronize()
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)
    full_o, full_pool = d["o"].clone(), d["pool"].clone()
    # resume every sequence at 4352 from its 4th exported state (index 3)
    cut = 4352
    N = w.num_seqs
    offs = binding.export_offsets(w.lengths, None, w.export_grid)
    assert offs[1] - offs[0] == 7
    pool = torch.zeros_like(d["pool"])
    init = torch.arange(16, 32, dtype=torch.int32, device="cuda")
    for i in range(N):
        pool[16 + i] = exp_states[offs[i] + 3]
    cu = w.cu_seqlens()
    idx = np.concatenate([np.arange(cu[i] + cut, cu[i + 1]) for i in range(N)])
    ti = torch.from_numpy(idx).long().cuda()
    sub = {x: d[x][ti].contiguous() for x in ("q", "k", "v", "g", "beta")}
    o2 = torch.empty_like(sub["v"])
    L2 = 8192 - cut
    cu2 = torch.arange(0, N + 1, dtype=torch.int32, device="cuda") * L2
    final = torch.arange(0, 16, dtype=torch.int32, device="cuda")
    sp = torch.full((N,), cut, dtype=torch.int32, device="cuda")
    ws = binding.alloc_workspace(w.H_v, torch.bfloat16, N, N * L2, "cuda")
    binding.gdn_chunk_prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], o2, cu2, pool, init, final,
                              scale=w.scale, workspace=ws, start_pos=sp)
    torch.cuda.synchronize()
    assert torch.equal(o2, full_o[ti])
    for i in range(N):
        assert torch.equal(pool[i], full_pool[int(w.final_slot[i])])


def test_prefix_cache_grid_cases():
    """The prefix-cache cases of the third page: a 1100-token shared prefix hits at the
    grid point 1088 and resumes from the exported state bitwise; a ragged 200-token
    prefix floors to 0 (a full recompute, which is the same run)."""
    grid = 1088
    w = W.make_workload("pc", seed=26, H_k=2, H_v=4, d_k=128, d_v=128, dtype="bf16", lengths=[1100 + 900],
                        num_slots=8, export_grid=grid)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    assert exp_states.shape[0] == 1                      # 2000 tokens cross one grid point
    check_prefill(w, prefill_reference(w), d["o"], d["pool"], exp_states)
    hit = (1100 // grid) * grid
    assert hit == 1088 and (200 // grid) * grid == 0
    pool = d["pool"].clone()
    pool[5] = exp_states[0]
    sub = {x: d[x][hit:].contiguous() for x in ("q", "k", "v", "g", "beta")}
    o2 = torch.empty_like(sub["v"])
    n = 2000 - hit
    ws = binding.alloc_workspace(4, torch.bfloat16, 1, n, "cuda")
    binding.gdn_chunk_prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], o2,
                              torch.tensor([0, n], dtype=torch.int32, device="cuda"), pool,
                              torch.tensor([5], dtype=torch.int32, device="cuda"),
                              torch.tensor([6], dtype=torch.int32, device="cuda"), scale=w.scale, workspace=ws,
                              start_pos=torch.tensor([hit], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o2, d["o"][hit:])
    assert torch.equal(pool[6], d["pool"][int(w.final_slot[0])])
    # the same hit served alone (batch size 1) and inside a batch of 3 gives the same bits
    q3 = {x: torch.cat([sub[x], d[x][:100], sub[x]]).contiguous() for x in sub}
    o3 = torch.empty_like(q3["v"])
    pool3 = d["pool"].clone()
    pool3[5] = exp_states[0]
    pool3[4] = exp_states[0]
    ws3 = binding.alloc_workspace(4, torch.bfloat16, 3, 2 * n + 100, "cuda")
    binding.gdn_chunk_prefill(q3["q"], q3["k"], q3["v"], q3["g"], q3["beta"], o3,
                              torch.tensor([0, n, n + 100, 2 * n + 100], dtype=torch.int32, device="cuda"), pool3,
                              torch.tensor([5, -1, 4], dtype=torch.int32, device="cuda"),
                              torch.tensor([6, 7, 3], dtype=torch.int32, device="cuda"), scale=w.scale,
                              workspace=ws3, start_pos=torch.tensor([hit, 0, hit], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o3[:n], o2) and torch.equal(o3[n + 100:], o2)
    assert torch.equal(pool3[6], pool[6]) and torch.equal(pool3[3], pool[6])


def test_prefill_zero_length_and_empty():
    w = W.make_workload("z", seed=27, H_k=1, H_v=2, d_k=64, d_v=64, dtype="f32", lengths=[0, 5, 0],
                        num_slots=12, prefill_init="slots")
    d = to_device(w)
    run_prefill(w, d)
    torch.cuda.synchronize()
    for i in (0, 2):
        assert torch.equal(d["pool"][int(w.final_slot[i])].cpu(), torch.from_numpy(w.pool[int(w.init_slot[i])]))
    check_prefill(w, prefill_reference(w), d["o"], d["pool"])
