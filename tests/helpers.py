"""Shared helpers for the parity tests: move a workload to the GPU, run the oracle
on the same values (one call over the whole workload), and compare element by
element."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd.workloads import Workload

# Per-element bound |gpu - ref| <= atol + rtol |ref|, for outputs and every state.
TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-5, 1e-5)}


def tdtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_device(w: Workload, device="cuda"):
    dt = tdtype(w)
    d = {
        "q": torch.from_numpy(w.q).to(device=device, dtype=dt),
        "k": torch.from_numpy(w.k).to(device=device, dtype=dt),
        "v": torch.from_numpy(w.v).to(device=device, dtype=dt),
        "g": torch.from_numpy(w.g).to(device),
        "beta": torch.from_numpy(w.beta).to(device),
        "pool": torch.from_numpy(w.pool).to(device),
        "slot_in": torch.from_numpy(w.slot_in).to(device),
        "slot_out": torch.from_numpy(w.slot_out).to(device),
        "cu": torch.from_numpy(w.cu_seqlens()).to(device),
        "init_slot": torch.from_numpy(w.init_slot).to(device),
        "final_slot": torch.from_numpy(w.final_slot).to(device),
        "start_pos": None if w.start_pos is None else torch.from_numpy(w.start_pos).to(device),
    }
    d["o"] = torch.empty_like(d["v"])
    # the bf16 values on the device must be exactly the generator's values
    assert torch.equal(d["q"].float().cpu(), torch.from_numpy(w.q))
    return d


def assert_close(name, got, ref, atol, rtol, locate=None):
    """Per-element bound |got - ref| <= atol + rtol |ref| over whole arrays, checked in
    slices along the first axis so that full-size outputs need no full-size
    temporaries.  ``locate(index)`` may turn the worst element's index into a
    readable place (sequence, head, ...)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    n0 = got.shape[0]
    step = max(1, (1 << 24) // max(1, got.size // n0))
    worst = (-np.inf, None, 0.0, 0.0, 0.0)       # (err - bound, index, got, ref, err / bound)
    max_err = 0.0
    for a in range(0, n0, step):
        g = np.asarray(got[a:a + step], dtype=np.float64)
        r = np.asarray(ref[a:a + step], dtype=np.float64)
        assert np.all(np.isfinite(g)), "%s: non-finite values in rows %d.." % (name, a)
        err = np.abs(g - r)
        bound = atol + rtol * np.abs(r)
        excess = err - bound
        i = np.unravel_index(np.argmax(excess), excess.shape)
        max_err = max(max_err, float(err.max()))
        if excess[i] > worst[0]:
            idx = (int(i[0]) + a,) + tuple(int(x) for x in i[1:])
            worst = (float(excess[i]), idx, float(g[i]), float(r[i]), float(err[i] / bound[i]))
    where = "" if locate is None else " (%s)" % locate(worst[1])
    msg = "%s: max abs err %.3g, worst err/bound %.3g at %s%s (got %.6g, ref %.6g)" % (
        name, max_err, worst[4], worst[1], where, worst[2], worst[3])
    assert worst[0] <= 0.0, msg


def decode_reference(w: Workload, rows=None):
    """Oracle decode for the workload's decode rows (all, or the listed ones): returns
    (o [B, H_v, d_v], new_states [B, H_v, d_k, d_v]) in fp64, for rows whose slot_in is valid."""
    rows = np.arange(w.num_decode_rows) if rows is None else np.asarray(rows)
    B = len(rows)
    si = w.slot_in[rows]
    compact = np.zeros((B, w.H_v, w.d_k, w.d_v), dtype=np.float64)
    valid = (si >= 0) & (si < w.pool.shape[0])
    compact[valid] = w.pool[si[valid]]
    idx = np.where(valid, np.arange(B), -1).astype(np.int32)
    o = oracle.decode(w.q[rows], w.k[rows], w.v[rows], w.g[rows], w.beta[rows], compact, idx, idx,
                      scale=w.scale)
    return o, compact


class PrefillRef:
    """The oracle's prefill of a workload's prefill part, every sequence and every
    value head, from ONE oracle call: o [T_p, H_v, d_v] (prefill tokens only),
    finals [N, H_v, d_k, d_v], exports [E, H_v, d_k, d_v] and the export offsets.
    ``ref[(i, h)]`` gives sequence i, head h as (o [L, d_v], final, exports [n, ...])."""

    def __init__(self, w: Workload):
        B = w.num_decode_rows
        N = w.num_seqs
        init = np.zeros((N, w.H_v, w.d_k, w.d_v), dtype=np.float64)
        for i in range(N):
            s = int(w.init_slot[i])
            if 0 <= s < w.pool.shape[0]:
                init[i] = w.pool[s]
        self.cu = w.cu_seqlens()
        sp = None if w.start_pos is None else np.asarray(w.start_pos)
        self.o, self.finals, self.exports, self.offsets = oracle.prefill(
            w.q[B:], w.k[B:], w.v[B:], w.g[B:], w.beta[B:], self.cu, scale=w.scale, initial_states=init,
            start_pos=sp, export_grid=w.export_grid)

    def __getitem__(self, key):
        i, h = key
        a, b = int(self.cu[i]), int(self.cu[i + 1])
        return (self.o[a:b, h], self.finals[i, h],
                self.exports[int(self.offsets[i]):int(self.offsets[i + 1]), h])

    def seq_of_token(self, t):
        return int(np.searchsorted(self.cu, t, side="right") - 1)


def prefill_reference(w: Workload) -> PrefillRef:
    return PrefillRef(w)


def check_prefill(w: Workload, ref: PrefillRef, o, pool, exports=None, tag=""):
    """Every output row, final state and export of the workload's prefill part
    against the oracle, within the dtype's bound.  ``o`` holds the prefill tokens
    only; ``pool`` holds the final states at w.final_slot; ``exports`` the flat export
    stream (or None when the call exported nothing)."""
    atol, rtol = TOL[w.dtype]
    got_o = o.float().cpu().numpy()
    assert_close(tag + "o", got_o, ref.o, atol, rtol,
                 locate=lambda ix: "sequence %d, token %d, head %d" % (
                     ref.seq_of_token(ix[0]), ix[0] - int(ref.cu[ref.seq_of_token(ix[0])]), ix[1]))
    valid = [i for i in range(w.num_seqs) if 0 <= int(w.final_slot[i]) < w.pool.shape[0]]
    if valid:
        slots = torch.as_tensor([int(w.final_slot[i]) for i in valid], dtype=torch.long, device=pool.device)
        assert_close(tag + "final states", pool[slots].cpu().numpy(), ref.finals[valid], atol, rtol,
                     locate=lambda ix: "sequence %d, head %d" % (valid[ix[0]], ix[1]))
    if w.export_grid:
        E = int(ref.offsets[-1])
        assert exports is not None or E == 0
        if E:
            assert_close(tag + "exports", exports[:E].cpu().numpy(), ref.exports, atol, rtol,
                         locate=lambda ix: "export %d (sequence %d), head %d" % (
                             ix[0], int(np.searchsorted(ref.offsets, ix[0], side="right") - 1), ix[1]))


def run_prefill(w: Workload, d, export=True, stream=None):
    """Call gdn_chunk_prefill on the workload's prefill part (no decode rows)."""
    assert w.num_decode_rows == 0
    N, T = w.num_seqs, w.total_tokens
    ws = binding.alloc_workspace(w.H_v, tdtype(w), N, T, d["q"].device)
    exp_states = exp_offs = None
    if export and w.export_grid:
        offs = binding.export_offsets(w.lengths, None if w.start_pos is None else list(w.start_pos),
                                      w.export_grid)
        exp_offs = torch.tensor(offs, dtype=torch.int32, device=d["q"].device)
        exp_states = torch.full((max(offs[-1], 1), w.H_v, w.d_k, w.d_v), float("nan"),
                                dtype=torch.float32, device=d["q"].device)
    binding.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["o"], d["cu"], d["pool"],
                              d["init_slot"], d["final_slot"], scale=w.scale, workspace=ws,
                              start_pos=d["start_pos"], export_grid=w.export_grid if export else 0,
                              export_states=exp_states, export_offsets=exp_offs, stream=stream)
    return exp_states, exp_offs
