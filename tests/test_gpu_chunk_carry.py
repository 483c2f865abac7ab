"""Bitwise state carry across a chunked prefill split at ANY token, not only on the
64-token grid.

The pages leave this open: "[Model] Enable batch-invariant mixed decode and prefill
for Qwen GDN", section "Out of scope", lists recurrent-state invariance across
arbitrary chunked-prefill boundaries; "[WIP][Kernel] Enable GDN batch-invariant prefix
caching", section "Purpose", puts chunks and cache hits on one grid that is a multiple
of 64.  Chunks here lie on the absolute 64-token grid, and within a chunk a row only
ever combines rows at or before it, with padding rows entering as exact zeros.  So a
partial last chunk produces, for its rows, the same bits as the full chunk would.

That gives the carry protocol these tests exercise: a prefill split at token t
returns its outputs up to t (bitwise those of the unsplit run) and the state at the
last grid point t0 = 64 floor(t / 64) (an export on the 64 grid); the next call
starts at t0 from that state and re-feeds the t - t0 < 64 tokens since, whose
outputs come out bitwise equal once more; every later output and the final state are
bitwise those of the unsplit run."""
import dataclasses

import numpy as np
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import run_prefill, tdtype, to_device

pytestmark = pytest.mark.gpu

SHAPES = [("bf16", 128, 128, 2, 4), ("bf16", 64, 64, 1, 3), ("f32", 64, 64, 1, 2), ("f32", 128, 128, 2, 2)]


def _i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", SHAPES)
@pytest.mark.parametrize("start", [0, 40])
def test_partial_chunk_rows_equal_full_chunk_rows(dtype, dk, dv, hk, hv, start):
    """Prefixes of one sequence (1, 37, 100, 200 and all 256 tokens), run side by side
    in one call: each prefix's outputs and grid states are bitwise those of the whole
    sequence, though its last chunk is partial and the whole run's is not."""
    base = W.make_workload("pfx", seed=51, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=[256],
                           num_slots=16, prefill_init="slots", start_pos=[start], export_grid=64)
    cuts = [1, 37, 100, 200, 256]
    pick = lambda a: np.concatenate([a[:L] for L in cuts])
    w = dataclasses.replace(base, lengths=cuts, q=pick(base.q), k=pick(base.k), v=pick(base.v), g=pick(base.g),
                            beta=pick(base.beta), init_slot=np.zeros(len(cuts), np.int32),
                            final_slot=np.arange(len(cuts), dtype=np.int32) + 8,
                            start_pos=np.full(len(cuts), start, np.int32))
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    cu = w.cu_seqlens()
    offs = binding.export_offsets(cuts, [start] * len(cuts), 64)
    full = len(cuts) - 1
    a_full = int(cu[full])
    for i, L in enumerate(cuts[:-1]):
        a = int(cu[i])
        assert torch.equal(d["o"][a:a + L], d["o"][a_full:a_full + L]), ("outputs", L)
        n = offs[i + 1] - offs[i]
        assert torch.equal(exp_states[offs[i]:offs[i] + n], exp_states[offs[full]:offs[full] + n]), ("exports", L)


def _run_part(w, d, pool, lo, hi, start, init_slot, final_slot):
    """gdn_chunk_prefill on tokens [lo, hi) of the single-sequence workload, starting
    at absolute position start from pool[init_slot], exporting on the 64 grid."""
    sub = {x: d[x][lo:hi].contiguous() for x in ("q", "k", "v", "g", "beta")}
    o = torch.empty_like(sub["v"])
    offs = binding.export_offsets([hi - lo], [start], 64)
    exp_states = torch.full((max(offs[-1], 1), w.H_v, w.d_k, w.d_v), float("nan"), device="cuda")
    ws = binding.alloc_workspace(w.H_v, tdtype(w), 1, hi - lo, "cuda")
    binding.gdn_chunk_prefill(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], o, _i32([0, hi - lo]), pool,
                              _i32([init_slot]), _i32([final_slot]), scale=w.scale, workspace=ws,
                              start_pos=_i32([start]), export_grid=64, export_states=exp_states,
                              export_offsets=_i32(offs))
    return o, exp_states


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", SHAPES)
@pytest.mark.parametrize("base_start,splits", [(0, [100]), (0, [1100]), (0, [200]), (0, [50]),
                                               (0, [100, 1100]), (1088, [12, 333, 1000])])
def test_off_grid_split_resumes_bitwise(dtype, dk, dv, hk, hv, base_start, splits):
    """A 1500-token prefill split at off-grid tokens (100 and 1100 as in the prefix
    cases of the third page, the ragged 200, a split before the first grid point, and
    several splits in a row of a sequence that itself resumes at 1088): with the carry
    protocol every output of every part and the final state are bitwise those of the
    unsplit run."""
    L = 1500
    w = W.make_workload("split", seed=53, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=[L],
                        num_slots=8, prefill_init="slots", start_pos=[base_start])
    w.init_slot[:] = 0
    w.final_slot[:] = 1
    d = to_device(w)
    init = 0
    pool0 = d["pool"].clone()
    run_prefill(w, d, export=False)                       # the unsplit run
    torch.cuda.synchronize()
    o_full = d["o"].clone()
    final_full = d["pool"][int(w.final_slot[0])].clone()

    pool = pool0.clone()
    carry, spare = 6, 7                                   # slots that hold the carried grid state
    lo, state_slot = 0, init                              # tokens re-fed from lo (an absolute grid point)
    for t in splits + [L]:
        o, exp_states = _run_part(w, d, pool, lo, t, base_start + lo, state_slot, spare)
        torch.cuda.synchronize()
        assert torch.equal(o, o_full[lo:t]), ("outputs", lo, t)
        if t == L:
            assert torch.equal(pool[spare], final_full)
            break
        # resume at the last grid point at or before t: the state exported there, or
        # (no grid point crossed since lo) the state this part started from
        nxt = ((base_start + t) // 64) * 64 - base_start
        if nxt > lo:
            m = (base_start + nxt) // 64 - (base_start + lo) // 64 - 1
            pool[carry] = exp_states[m]
            state_slot, carry = carry, (5 if carry == 6 else 6)
        lo = nxt
