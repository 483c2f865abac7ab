"""The bf16 prefill kernel's rounding scheme against the per-element bound, on the
stress inputs of the GPU parity suite (keys with cosine near 0.9, gates near or at
zero, beta near one), in the fp64 rounding model of tests/precision_model.py.

It pins the design choices of the kernel's scheme: with it the model stays well
inside the bound, each cheaper alternative named below leaves it, and the all-bf16
scheme it replaced is no better.  The
reference is the fp64 oracle.  The bound is |x - ref| <= 2e-3 + 1e-2 |ref| for
outputs and states.

The model tracks the GPU closely: a kernel build that took U as one fp16 value both
in the solve (against -A_ij as an fp16 pair) and in the state update failed the GPU
parity suite on the d 64 stress inputs with one key head and three value heads, an
export at 1.08 of the bound; the model gives 1.079 for that workload."""
import numpy as np
import pytest

import oracle
from gated_deltanet_rule_amd import workloads as W
from tests import precision_model as PM

ATOL, RTOL = 2e-3, 1e-2


def _worst_ratio(d_k, d_v, key_mix, gate_scale, beta_shift, scheme=PM.KERNEL, **override):
    """Worst error / bound over every chain (5 sequences x 4 value heads) of the
    stress workload: (outputs, states), the states being the final ones and those on
    the 64-token export grid."""
    w = W.make_workload("stress", seed=28, H_k=2, H_v=4, d_k=d_k, d_v=d_v, dtype="bf16",
                        lengths=[700, 64, 1, 333, 129], num_slots=24, prefill_init="slots",
                        key_mix=key_mix, gate_scale=gate_scale, beta_shift=beta_shift)
    cu = w.cu_seqlens()
    ref_o, finals, exports, eoff = oracle.prefill(w.q, w.k, w.v, w.g, w.beta, cu, scale=w.scale,
                                                  pool=w.pool.astype(np.float64), init_slot=w.init_slot,
                                                  final_slot=w.final_slot, export_grid=64)
    worst_o = worst_s = 0.0
    ratio = lambda x, r: float(np.max(np.abs(x - r) / (ATOL + RTOL * np.abs(r))))
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    for seq in range(len(cu) - 1):
        a, b = int(cu[seq]), int(cu[seq + 1])
        for h in range(w.H_v):
            kh = h // (w.H_v // w.H_k)
            o, states = PM.chain(f64(w.q[a:b, kh]), f64(w.k[a:b, kh]), f64(w.v[a:b, h]), f64(w.g[a:b, h]),
                                 f64(w.beta[a:b, h]), w.scale, f64(w.pool[w.init_slot[seq], h]), scheme, **override)
            worst_o = max(worst_o, ratio(o, ref_o[a:b, h]))
            worst_s = max(worst_s, ratio(states[-1], finals[seq, h]))
            for m in range(int(eoff[seq + 1] - eoff[seq])):   # grid point 64 (m + 1)
                worst_s = max(worst_s, ratio(states[m], exports[eoff[seq] + m, h]))
    return worst_o, worst_s


CASES = {
    # (d_k, d_v, key_mix, gate_scale, beta_shift)
    "no decay, d 128": (128, 128, 3.0, 0.0, 3.0),
    "near-zero decay, d 64": (64, 64, 3.0, 0.01, 2.0),
    "no decay, d_k 64, d_v 128": (64, 128, 3.0, 0.0, 3.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_kernel_scheme_meets_the_bound(name):
    """Outputs within 0.35 and states (final and on the grid) within 0.7 of the bound."""
    o, s = _worst_ratio(*CASES[name])
    assert o < 0.35 and s < 0.7, (name, o, s)


def test_kernel_scheme_is_no_worse_than_the_all_bf16_one():
    """Q and K in fp16 and S rounded once to fp16 in K S and Q S (instead of bf16) pay
    for the single fp16 roundings elsewhere: every case's outputs, and the worst
    state over the cases, are no worse than with the all-bf16 scheme."""
    worst, worst0 = 0.0, 0.0
    for name, case in CASES.items():
        o, s = _worst_ratio(*case)
        o0, s0 = _worst_ratio(*case, scheme=PM.EARLIER)
        assert o <= 1.05 * o0, (name, o, o0)
        worst, worst0 = max(worst, s), max(worst0, s0)
    assert worst <= 1.05 * worst0, (worst, worst0)


@pytest.mark.parametrize("name", ["no decay, d 128", "no decay, d_k 64, d_v 128"])
def test_single_fp16_solve_products_exceed_the_bound(name):
    """The off-diagonal solve products -A_ij U_j keep fp16 pairs: with single fp16
    values on both sides the states leave the bound."""
    _, s = _worst_ratio(*CASES[name], solve_a="f16", solve_u="f16")
    assert s > 1.0, (name, s)


def test_single_fp16_u_in_the_solve_exceeds_the_bound():
    """Nor can U enter those products as one fp16 value against an fp16 pair for
    -A_ij (one product fewer per block pair): the states leave the bound."""
    _, s = _worst_ratio(*CASES["no decay, d_k 64, d_v 128"], solve_a="f16x2", solve_u="f16")
    assert s > 1.0, s


@pytest.mark.parametrize("name", ["no decay, d 128", "near-zero decay, d 64"])
def test_single_bf16_output_product_exceeds_the_bound(name):
    """P and U cannot enter the output product as single bf16 values (the earlier
    scheme's first form, which the GPU parity suite caught): fp16 is needed."""
    o, _ = _worst_ratio(*CASES[name], scheme=PM.EARLIER, out_p="bf16", out_u="bf16")
    assert o > 1.0, (name, o)


@pytest.mark.parametrize("name,upd,least", [("no decay, d 128", "bf16", 2.0), ("near-zero decay, d 64", "bf16", 2.0),
                                            ("no decay, d_k 64, d_v 128", "f16", 1.0)])
def test_state_update_without_lo_exceeds_the_bound(name, upd, least):
    """The decayed U enters the state update as an fp16 hi + lo pair: rounded once
    (to bf16, or even to fp16) the states leave the bound on the stress inputs."""
    _, s = _worst_ratio(*CASES[name], upd_u=upd)
    assert s > least, (name, upd, s)


def test_standard_inputs_are_well_inside_the_bound():
    """The standard input recipe (independent unit keys, g = -softplus(N(0,1)), beta =
    sigmoid(N(0,1))) with the kernel's roundings: outputs and states stay far inside
    the bound."""
    o, s = _worst_ratio(128, 128, 0.0, 1.0, 0.0)
    assert o < 0.3 and s < 0.1, (o, s)
