"""Pins for the CPU oracle (no GPU needed).

The pages print no formula and no values for the recurrence, so the oracle is
pinned by mathematics: a hand-worked example, brute force over dense transition
matrices, exact rationals, closed forms for the special cases the rule has, an
independent chunked evaluation, and structural properties (state carry, exports,
decode = one-token prefill).  ``test_mutants_are_caught`` plants plausible mistakes
in a copy of the oracle's source and checks that the pins catch every one.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T, H_k, H_v, d_k, d_v, unit_keys=True, gate_scale=1.0):
    q = rng.standard_normal((T, H_k, d_k))
    k = rng.standard_normal((T, H_k, d_k))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H_v, d_v))
    g = -np.log1p(np.exp(gate_scale * rng.standard_normal((T, H_v))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H_v))))
    return q, k, v, g, beta


def _single(q, k, v, g, beta, S0, scale, lib=None, export_grid=0):
    """Oracle on one sequence, one head: arrays [T, d]."""
    T = q.shape[0]
    o, fin, exp_, _ = oracle.prefill(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                                     np.array([0, T]), scale=scale, initial_states=S0[None, None],
                                     export_grid=export_grid, lib=lib)
    return o[:, 0], fin[0, 0], exp_[:, 0]


# ---------------------------------------------------------------- worked example

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, nums = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in nums.split()])
    return vals


def check_worked_example(lib=None):
    gv = _read_golden("worked_example_d2.txt")
    T = 3
    o, fin, states = _single(gv["q"].reshape(T, 2), gv["k"].reshape(T, 2), gv["v"].reshape(T, 2),
                             np.log(gv["alpha"]), gv["beta"], gv["S0"].reshape(2, 2), 1.0,
                             lib=lib, export_grid=1)
    np.testing.assert_allclose(o, gv["o"].reshape(T, 2), rtol=0, atol=1e-14)
    for t in range(T):
        np.testing.assert_allclose(states[t], gv["S%d" % (t + 1)].reshape(2, 2), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fin, gv["S3"].reshape(2, 2), rtol=0, atol=1e-14)


def test_worked_example():
    check_worked_example()


# ---------------------------------------------------------------- brute force

def check_brute_force(lib=None, d_k=3, d_v=5, seed=0):
    rng = np.random.default_rng(seed)
    T, H_k, H_v = 8, 2, 4
    q, k, v, g, beta = _rand_case(rng, T, H_k, H_v, d_k, d_v, unit_keys=False)
    S0 = rng.standard_normal((1, H_v, d_k, d_v))
    scale = 0.7
    o, fin, _, _ = oracle.prefill(q, k, v, g, beta, np.array([0, T]), scale=scale,
                                  initial_states=S0, lib=lib)
    for h in range(H_v):
        kh = h // (H_v // H_k)                      # contiguous GQA groups
        ob, sb = pins.brute_force_products(np.exp(g[:, h]), beta[:, h], k[:, kh], v[:, h], q[:, kh],
                                           S0[0, h], scale)
        np.testing.assert_allclose(o[:, h], ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], sb[-1], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d_k,d_v", [(3, 5), (4, 4), (5, 2)])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force(d_k, d_v, seed):
    check_brute_force(d_k=d_k, d_v=d_v, seed=seed)


# ---------------------------------------------------------------- exact rationals

def check_exact_rational(lib=None):
    from fractions import Fraction as F
    rng = np.random.default_rng(7)
    T, d_k, d_v = 6, 3, 4
    alpha = [F(1), F(1, 2), F(1, 4), F(1, 2), F(1), F(1, 4)]
    beta = [F(1, 2), F(1), F(1, 2), F(1), F(1, 2), F(1)]
    k = [[F(int(x), 2) for x in rng.integers(-2, 3, d_k)] for _ in range(T)]
    v = [[F(int(x), 4) for x in rng.integers(-4, 5, d_v)] for _ in range(T)]
    q = [[F(int(x), 2) for x in rng.integers(-2, 3, d_k)] for _ in range(T)]
    S0 = [[F(int(x), 8) for x in rng.integers(-8, 9, d_v)] for _ in range(d_k)]
    eo, es = pins.exact_rational(alpha, beta, k, v, q, S0, F(1, 2))
    fl = lambda a: np.array(a, dtype=np.float64)
    o, fin, states = _single(fl(q), fl(k), fl(v), np.log(fl(alpha)), fl(beta), fl(S0), 0.5,
                             lib=lib, export_grid=1)
    np.testing.assert_allclose(o, fl(eo), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(states, fl(es), rtol=1e-14, atol=1e-14)


def test_exact_rational():
    check_exact_rational()


# ---------------------------------------------------------------- special cases

def check_pure_decay(lib=None):
    """beta = 0: the delta write vanishes, S_t = e^{G_t} S0 and o_t = scale e^{G_t} S0^T q_t."""
    rng = np.random.default_rng(3)
    T, d_k, d_v = 40, 6, 7
    q, k, v, g, _ = _rand_case(rng, T, 1, 1, d_k, d_v)
    S0 = rng.standard_normal((d_k, d_v))
    o, fin, states = _single(q[:, 0], k[:, 0], v[:, 0], g[:, 0], np.zeros(T), S0, 0.3,
                             lib=lib, export_grid=1)
    G = np.cumsum(g[:, 0])
    expect_o = 0.3 * np.exp(G)[:, None] * (q[:, 0] @ S0)          # textbook gemv per token
    np.testing.assert_allclose(o, expect_o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin, np.exp(G[-1]) * S0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(states, np.exp(G)[:, None, None] * S0[None], rtol=1e-13, atol=1e-15)


def test_pure_decay():
    check_pure_decay()


def check_exact_recall(lib=None):
    """g = 0, beta = 1, keys = distinct standard basis vectors, S0 = 0, scale 1:
    every key stores its value exactly, and querying any earlier key returns it."""
    rng = np.random.default_rng(4)
    d_k, d_v, T = 16, 5, 12
    perm = rng.permutation(d_k)[:T]
    k = np.eye(d_k)[perm]
    v = rng.standard_normal((T, d_v))
    # query t asks for the key written at step s_t <= t
    s_of_t = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = k[s_of_t]
    o, fin, _ = _single(q, k, v, np.zeros(T), np.ones(T), np.zeros((d_k, d_v)), 1.0, lib=lib)
    assert np.array_equal(o, v[s_of_t])
    expect_S = np.zeros((d_k, d_v))
    expect_S[perm] = v
    assert np.array_equal(fin, expect_S)


def test_exact_recall():
    check_exact_recall()


def test_unit_key_recall_any_state():
    """beta = 1 and |k| = 1: the updated state maps k_t to v_t exactly, whatever g and S."""
    rng = np.random.default_rng(5)
    T, d_k, d_v = 30, 8, 6
    q, k, v, g, _ = _rand_case(rng, T, 1, 1, d_k, d_v)
    S0 = rng.standard_normal((d_k, d_v))
    _, _, states = _single(q[:, 0], k[:, 0], v[:, 0], g[:, 0], np.ones(T), S0, 1.0, export_grid=1)
    recalled = np.einsum("tij,ti->tj", states, k[:, 0])
    np.testing.assert_allclose(recalled, v[:, 0], rtol=0, atol=1e-13)


def test_full_forgetting():
    """alpha -> 0 (g = -200): S_t = beta_t k_t v_t^T and o_t = scale beta_t (k_t . q_t) v_t."""
    rng = np.random.default_rng(6)
    T, d_k, d_v = 10, 5, 4
    q, k, v, _, beta = _rand_case(rng, T, 1, 1, d_k, d_v)
    S0 = rng.standard_normal((d_k, d_v))
    o, _, states = _single(q[:, 0], k[:, 0], v[:, 0], np.full(T, -200.0), beta[:, 0], S0, 0.5,
                           export_grid=1)
    kq = np.sum(k[:, 0] * q[:, 0], axis=1)
    np.testing.assert_allclose(o, 0.5 * (beta[:, 0] * kq)[:, None] * v[:, 0], rtol=1e-13, atol=1e-16)
    expect = beta[:, 0, None, None] * k[:, 0, :, None] * v[:, 0, None, :]
    np.testing.assert_allclose(states, expect, rtol=1e-13, atol=1e-16)


def test_identity_step():
    """g = 0, beta = 0: the state never changes and o_t = scale S0^T q_t."""
    rng = np.random.default_rng(8)
    T, d_k, d_v = 9, 4, 6
    q, k, v, _, _ = _rand_case(rng, T, 1, 1, d_k, d_v)
    S0 = rng.standard_normal((d_k, d_v))
    o, fin, _ = _single(q[:, 0], k[:, 0], v[:, 0], np.zeros(T), np.zeros(T), S0, 0.25)
    np.testing.assert_allclose(o, 0.25 * q[:, 0] @ S0, rtol=1e-14, atol=1e-16)
    assert np.array_equal(fin, S0)


# ---------------------------------------------------------------- chunked form

def check_chunked(lib=None, C=16, seed=0):
    rng = np.random.default_rng(100 + seed)
    lengths = [150, 64, 1, 77]
    T = sum(lengths)
    H_k, H_v, d_k, d_v = 2, 4, 8, 6
    q, k, v, g, beta = _rand_case(rng, T, H_k, H_v, d_k, d_v)
    S0 = 0.1 * rng.standard_normal((len(lengths), H_v, d_k, d_v))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, fin, _, _ = oracle.prefill(q, k, v, g, beta, cu, scale=0.35, initial_states=S0, lib=lib)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        for h in range(H_v):
            kh = h // 2
            oc, sc = pins.chunked_ut(g[a:b, h], beta[a:b, h], k[a:b, kh], v[a:b, h], q[a:b, kh],
                                     S0[i, h], 0.35, C)
            np.testing.assert_allclose(o[a:b, h], oc, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(fin[i, h], sc, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C", [4, 16, 64])
def test_chunked_matches_sequential(C):
    check_chunked(C=C)


# ---------------------------------------------------------------- structure

def check_exports_and_carry(lib=None):
    """Exports equal the final state of the matching prefix run, bitwise; a sequence
    split at any point and resumed from the carried state equals the unsplit run."""
    rng = np.random.default_rng(11)
    T, H_k, H_v, d_k, d_v = 37, 1, 2, 4, 3
    q, k, v, g, beta = _rand_case(rng, T, H_k, H_v, d_k, d_v)
    S0 = 0.1 * rng.standard_normal((1, H_v, d_k, d_v))
    grid, start = 4, 6
    o, fin, exports, offs = oracle.prefill(q, k, v, g, beta, np.array([0, T]), scale=0.5,
                                           initial_states=S0, start_pos=[start], export_grid=grid,
                                           lib=lib)
    points = [p for p in range(start + 1, start + T + 1) if p % grid == 0]
    assert exports.shape[0] == len(points) and list(offs) == [0, len(points)]
    for m, p in enumerate(points):
        n = p - start
        _, fin_n, _, _ = oracle.prefill(q[:n], k[:n], v[:n], g[:n], beta[:n], np.array([0, n]),
                                        scale=0.5, initial_states=S0, lib=lib)
        assert np.array_equal(exports[m], fin_n[0])
    # split at t and resume through the slot pool
    for t in (1, 8, 20, 36):
        pool = np.zeros((3, H_v, d_k, d_v))
        pool[0] = S0[0]
        o1, _, _, _ = oracle.prefill(q[:t], k[:t], v[:t], g[:t], beta[:t], np.array([0, t]),
                                     scale=0.5, pool=pool, init_slot=[0], final_slot=[1], lib=lib)
        o2, _, _, _ = oracle.prefill(q[t:], k[t:], v[t:], g[t:], beta[t:], np.array([0, T - t]),
                                     scale=0.5, pool=pool, init_slot=[1], final_slot=[2], lib=lib)
        assert np.array_equal(np.concatenate([o1, o2]), o)
        assert np.array_equal(pool[2], fin[0])
        assert np.array_equal(pool[0], S0[0])


def test_exports_and_carry():
    check_exports_and_carry()


def check_decode(lib=None):
    """Decode of a packed batch equals one-token prefills bitwise; padding rows are
    skipped with zero output; slot_out may differ from slot_in (copy-on-advance)."""
    rng = np.random.default_rng(12)
    B, H_k, H_v, d_k, d_v, slots = 5, 2, 4, 4, 4, 12
    q, k, v, g, beta = _rand_case(rng, B, H_k, H_v, d_k, d_v)
    pool = rng.standard_normal((slots, H_v, d_k, d_v))
    slot_in = np.array([3, 7, -1, 0, 9], dtype=np.int32)
    slot_out = np.array([3, 8, -1, 1, 9], dtype=np.int32)
    before = pool.copy()
    o = oracle.decode(q, k, v, g, beta, pool, slot_in, slot_out, scale=0.4, lib=lib)
    for b in range(B):
        if slot_in[b] < 0:
            assert np.all(o[b] == 0)
            continue
        ob, fb, _, _ = oracle.prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1],
                                      np.array([0, 1]), scale=0.4, initial_states=before[slot_in[b]][None],
                                      lib=lib)
        assert np.array_equal(o[b], ob[0])
        assert np.array_equal(pool[slot_out[b]], fb[0])
    untouched = [s for s in range(slots) if s not in set(slot_out[slot_in >= 0])]
    assert np.array_equal(pool[untouched], before[untouched])
    # and the decode step is the product form applied once
    for b in (0, 1, 3):
        for h in range(H_v):
            kh = h // 2
            ob, sb = pins.brute_force_products(np.exp(g[b:b + 1, h]), beta[b:b + 1, h], k[b:b + 1, kh],
                                               v[b:b + 1, h], q[b:b + 1, kh], before[slot_in[b], h], 0.4)
            np.testing.assert_allclose(o[b, h], ob[0], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(pool[slot_out[b], h], sb[0], rtol=1e-13, atol=1e-14)


def test_decode():
    check_decode()


def test_zero_length_and_empty():
    rng = np.random.default_rng(13)
    H_v, d = 2, 3
    q, k, v, g, beta = _rand_case(rng, 5, 1, H_v, d, d)
    S0 = rng.standard_normal((3, H_v, d, d))
    cu = np.array([0, 0, 5, 5])                    # sequences of length 0, 5, 0
    o, fin, _, _ = oracle.prefill(q, k, v, g, beta, cu, scale=1.0, initial_states=S0)
    assert np.array_equal(fin[0], S0[0]) and np.array_equal(fin[2], S0[2])
    o_alone, fin_alone, _, _ = oracle.prefill(q, k, v, g, beta, np.array([0, 5]), scale=1.0,
                                              initial_states=S0[1:2])
    assert np.array_equal(o, o_alone) and np.array_equal(fin[1], fin_alone[0])
    pool = rng.standard_normal((2, H_v, d, d))
    before = pool.copy()
    o = oracle.decode(q[:0], k[:0], v[:0], g[:0], beta[:0], pool, [], [], scale=1.0)
    assert o.shape == (0, H_v, d) and np.array_equal(pool, before)


# ---------------------------------------------------------------- planted mistakes

# Square-state pins come first: a mutant that reads the state transposed would index
# out of bounds on a non-square state, so the suite stops at the first pin that fails.
PIN_SUITE = [check_worked_example, lambda lib: check_brute_force(lib, d_k=4, d_v=4, seed=3),
             check_brute_force, check_exact_rational, check_pure_decay, check_exact_recall,
             check_chunked, check_exports_and_carry, check_decode]

MUTANTS = {
    "decay dropped": [("const double alpha = exp(g);", "const double alpha = 1.0;")],
    "delta sign flipped": [("u[j] = beta * (v[j] - pred);", "u[j] = beta * (v[j] + pred);")],
    "beta dropped": [("u[j] = beta * (v[j] - pred);", "u[j] = (v[j] - pred);")],
    "prediction read transposed": [("pred += S[(size_t)i * d_v + j] * k[i];",
                                    "pred += S[(size_t)j * d_v + i] * k[i];")],
    "write along q instead of k": [("S[(size_t)i * d_v + j] += k[i] * u[j];",
                                    "S[(size_t)i * d_v + j] += q[i] * u[j];")],
    "output from the pre-write state": [("acc += S[(size_t)i * d_v + j] * q[i];",
                                         "acc += (S[(size_t)i * d_v + j] - k[i] * u[j]) * q[i];")],
    "decay applied last": [("S[(size_t)i * d_v + j] *= alpha;", "S[(size_t)i * d_v + j] *= 1.0;"),
                           ("S[(size_t)i * d_v + j] += k[i] * u[j];",
                            "S[(size_t)i * d_v + j] = alpha * (S[(size_t)i * d_v + j] + k[i] * u[j]);")],
    "scale dropped": [("o[j] = scale * acc;", "o[j] = acc;")],
    "GQA map interleaved": [("const int kh = h / group;", "const int kh = h % H_k;")],
    "export position off by one": [("+ (t - cu_seqlens[i]) + 1;", "+ (t - cu_seqlens[i]);")],
}


def _run_suite(lib, stop_at_first):
    failures = []
    for check in PIN_SUITE:
        try:
            check(lib)
        except AssertionError as e:  # a pin caught the mistake
            failures.append((getattr(check, "__name__", "check"), str(e)[:80]))
            if stop_at_first:
                break
    return failures


def test_mutants_are_caught():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(oracle._SRC).read()
    with tempfile.TemporaryDirectory() as td:
        clean = os.path.join(td, "clean.so")
        oracle.build(src=oracle._SRC, out=clean)
        assert _run_suite(oracle.open_library(clean), stop_at_first=False) == []
        for name, edits in MUTANTS.items():
            mutated = src
            for old, new in edits:
                assert old in mutated, (name, old)
                mutated = mutated.replace(old, new)
            path = os.path.join(td, "mut.c")
            with open(path, "w") as f:
                f.write(mutated)
            so = os.path.join(td, "mut_%d.so" % abs(hash(name)))
            oracle.build(src=path, out=so)
            caught = _run_suite(oracle.open_library(so), stop_at_first=True)
            assert caught, "planted mistake not caught by any pin: %s" % name
