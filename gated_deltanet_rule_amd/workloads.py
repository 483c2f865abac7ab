"""Seeded synthetic workloads for the gated delta rule path.

This module only *draws inputs*: it holds none of the method's arithmetic, and both
the GPU tests and the CPU oracle take their inputs from it.  Values are drawn on the
host with ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order -- sequence
lengths, cache slots, q, k, v, the raw gate draws, the raw beta draws, the initial
states -- and kept as float32 arrays whose values are exactly representable in the
workload dtype (bf16 values are rounded to nearest-even here, once), so that the
GPU receives and the oracle widens the very same numbers.

Input recipe (the pages print no model shapes, so the shapes follow the workloads
that the pages describe: a packed decode batch of cached rows, a varlen prefill,
a mixed step with cached rows ahead of fresh prefills of 116 / 321 / 1059 / 2000
tokens, and long prompts exporting states on the 1088-token prefix-cache grid):

  q, k   ~ N(0, 1) fp32, L2-normalised per (token, key head) in fp32, then cast
  v      ~ N(0, 1), then cast
  beta   = sigmoid(N(0, 1))           fp32, one per (token, value head)
  g      = -softplus(N(0, 1))         fp32 natural-log decay, one per (token, value head)
  states ~ N(0, 0.1^2) fp32 for cached rows; zeros for fresh prefills
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

CHUNK = 64


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    """Divide each last-axis vector by its Euclidean norm, in fp32 (in place)."""
    x = x.astype(np.float32, copy=False)
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float32), dtype=np.float32)
    x /= n[..., None]
    return x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x, dtype=np.float32))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    # log(1 + e^x), written to avoid overflow for large x
    return (np.maximum(x, np.float32(0.0)) + np.log1p(np.exp(-np.abs(x), dtype=np.float32))).astype(np.float32)


@dataclasses.dataclass
class Workload:
    """One step's inputs.  Tokens [0, num_decode_rows) are cached decode rows (one
    token each); the prefill sequences follow, packed, described by ``lengths``."""

    name: str
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    dtype: str                      # "bf16" or "f32" for q, k, v and o
    scale: float
    num_decode_rows: int
    lengths: list                   # prefill sequence lengths
    q: np.ndarray                   # [T, H_k, d_k] float32 (dtype-exact values)
    k: np.ndarray
    v: np.ndarray                   # [T, H_v, d_v]
    g: np.ndarray                   # [T, H_v] float32
    beta: np.ndarray                # [T, H_v] float32
    pool: np.ndarray                # [num_slots, H_v, d_k, d_v] float32
    slot_in: np.ndarray             # [num_decode_rows] int32
    slot_out: np.ndarray            # [num_decode_rows] int32
    init_slot: np.ndarray           # [num_seqs] int32 (-1 = zero initial state)
    final_slot: np.ndarray          # [num_seqs] int32
    start_pos: Optional[np.ndarray]  # [num_seqs] int32 or None
    export_grid: int

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    @property
    def prefill_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def total_tokens(self) -> int:
        return self.num_decode_rows + self.prefill_tokens

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.lengths, dtype=np.int64))
        return cu


def make_workload(name: str, *, seed: int, H_k: int, H_v: int, d_k: int, d_v: int,
                  dtype: str, num_decode_rows: int = 0, lengths: Sequence[int] = (),
                  num_slots: Optional[int] = None, state_std: float = 0.1,
                  prefill_init: str = "zero", export_grid: int = 0,
                  start_pos: Optional[Sequence[int]] = None, scale: Optional[float] = None,
                  lengths_range: Optional[tuple] = None, num_seqs: Optional[int] = None,
                  fill_pool: bool = True, key_mix: float = 0.0, gate_scale: float = 1.0,
                  beta_shift: float = 0.0) -> Workload:
    """Draw one workload.  ``lengths_range=(lo, hi)`` draws ``num_seqs`` integer
    lengths uniformly in [lo, hi] (both ends inclusive) before anything else.

    Stress knobs (defaults leave the standard recipe untouched): ``key_mix = a > 0``
    adds ``a sqrt(d_k)`` times one random unit direction per key head to every raw key
    before normalisation, so that two keys of a head have a cosine near a^2 / (a^2 + 1)
    (0.9 at a = 3); ``gate_scale`` multiplies g (near 0: almost no decay); ``beta_shift``
    is added to beta's normal draw before the sigmoid (2: beta near 0.9).  The extra
    direction is drawn after everything else, so the other draws do not move."""
    assert dtype in ("bf16", "f32")
    rng = np.random.default_rng(seed)
    if lengths_range is not None:
        lo, hi = lengths_range
        lengths = [int(x) for x in rng.integers(lo, hi + 1, size=num_seqs)]
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    B = int(num_decode_rows)
    if num_slots is None:
        num_slots = max(4 * (B + N), 8)
    perm = rng.permutation(num_slots).astype(np.int32)
    assert B + 2 * N <= num_slots, "not enough cache slots for disjoint decode/prefill slots"
    slot_in = perm[:B].copy()
    slot_out = slot_in.copy()
    final_slot = perm[B:B + N].copy()
    if prefill_init == "zero":
        init_slot = np.full(N, -1, dtype=np.int32)
    else:  # resume from cached states held in other slots
        init_slot = perm[B + N:B + 2 * N].copy()
    T = B + sum(lengths)

    cast = round_to_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    q = cast(_l2_normalise(rng.standard_normal((T, H_k, d_k), dtype=np.float32)))
    k_raw = rng.standard_normal((T, H_k, d_k), dtype=np.float32)
    v = cast(rng.standard_normal((T, H_v, d_v), dtype=np.float32))
    g = -_softplus(rng.standard_normal((T, H_v), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((T, H_v), dtype=np.float32) + np.float32(beta_shift))
    if gate_scale != 1.0:
        g = (g * np.float32(gate_scale)).astype(np.float32)
    if fill_pool:
        pool = rng.standard_normal((num_slots, H_v, d_k, d_v), dtype=np.float32)
        pool *= np.float32(state_std)
    else:
        pool = np.zeros((num_slots, H_v, d_k, d_v), dtype=np.float32)
    if key_mix > 0.0:
        u = _l2_normalise(rng.standard_normal((H_k, d_k), dtype=np.float32))
        k_raw += np.float32(key_mix * math.sqrt(d_k)) * u[None]
    k = cast(_l2_normalise(k_raw))
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    sp = None if start_pos is None else np.asarray(start_pos, dtype=np.int32)
    return Workload(name=name, H_k=H_k, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype, scale=float(scale),
                    num_decode_rows=B, lengths=lengths, q=q, k=k, v=v, g=g, beta=beta, pool=pool,
                    slot_in=slot_in, slot_out=slot_out, init_slot=init_slot, final_slot=final_slot,
                    start_pos=sp, export_grid=int(export_grid))


# The five standard workloads.  Seeds are 1000 + index.
CONFIG_DESCRIPTIONS = {
    0: "single sequence T=256, 1 head, d=64, fp32, zero state",
    1: "decode batch B=64, 16 key / 32 value heads, d=128, bf16, 256 cache slots",
    2: "varlen prefill, 8 sequences with lengths in [64,4096], 16/32 heads, d=128, bf16, export grid 64",
    3: "mixed step: 32 cached decode rows ahead of prefills of 116/321/1059/2000 tokens, 16/32 heads, d=128, bf16",
    4: "long prefill 16 x 8192 tokens, 16/32 heads, d=128, bf16, export grid 1088",
}


def config(index: int, **overrides) -> Workload:
    """The standard workload ``index`` (0..4); keyword overrides resize it (tests)."""
    seed = 1000 + index
    heads = dict(H_k=16, H_v=32, d_k=128, d_v=128, dtype="bf16")
    if index == 0:
        args = dict(H_k=1, H_v=1, d_k=64, d_v=64, dtype="f32", lengths=[256], num_slots=8,
                    fill_pool=True)
    elif index == 1:
        args = dict(heads, num_decode_rows=64, num_slots=256)
    elif index == 2:
        args = dict(heads, lengths_range=(64, 4096), num_seqs=8, num_slots=16, export_grid=64)
    elif index == 3:
        args = dict(heads, num_decode_rows=32, lengths=[116, 321, 1059, 2000], num_slots=256)
    elif index == 4:
        args = dict(heads, lengths=[8192] * 16, num_slots=32, export_grid=1088)
    else:
        raise ValueError("no standard workload %r" % index)
    args.update(overrides)
    return make_workload("cfg%d" % index, seed=seed, **args)
