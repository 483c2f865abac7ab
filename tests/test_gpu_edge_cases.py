"""The rule's special cases through every GPU path -- both prefill kernels (bf16 and
fp32 inputs) and decode -- with partial chunks, starts off the 64-token grid, initial
states from cache slots and exports on the grid.

Each expected value is the case's closed form, computed here in fp64 from the inputs
(not by the oracle):
  pure decay (beta = 0)        the state only decays: S_t = e^(G_t) S_0, where G_t is
                               the sum of the sequence's first t gates, and
                               o_t = scale e^(G_t) S_0^T q_t;
  exact recall (g = 0, beta = 1, keys distinct standard basis vectors, S_0 zero on
                               the key rows)   each token overwrites its key's row of
                               the state with v, so a query equal to a stored key
                               returns that token's v, and a query on an untouched row
                               returns S_0's row -- every product is 0 or 1, so with
                               values exact in the 16-bit formats the kernels use the
                               GPU must give these values bitwise;
  full forgetting (g = -200)   e^g underflows to 0 in fp32: S_t = beta_t k_t v_t^T and
                               o_t = scale beta_t (k_t . q_t) v_t, whatever S_0 was.
The gated delta rule these follow is the one the pages name ("[Model] Enable
batch-invariant mixed decode and prefill for Qwen GDN", sections "Why" and
"Results"); the state after each grid point is the prefix-cache export ("[V1][Hybrid]
GatedDeltaNet Automatic Prefix Caching", section "Purpose")."""
import numpy as np
import pytest
import torch

from gated_deltanet_rule_amd import binding
from gated_deltanet_rule_amd import workloads as W
from tests.helpers import TOL, assert_close, run_prefill, to_device

pytestmark = pytest.mark.gpu

# (dtype, d_k, d_v, H_k, H_v): both prefill kernels, both head sizes, GQA groups of
# 1, 2 and 3 (the bf16 kernel's one- and two-head workgroup shapes)
SHAPES = [("bf16", 128, 128, 2, 4), ("bf16", 64, 64, 1, 3), ("bf16", 128, 64, 2, 2), ("bf16", 64, 128, 1, 2),
          ("f32", 64, 64, 2, 4), ("f32", 128, 128, 1, 3)]
LENGTHS = [130, 1, 63, 200, 0, 64]
STARTS = [0, 5, 64, 1000, 7, 33]


def _grid_points(start, L, grid):
    """Tokens consumed at each grid point p in (start, start + L], p % grid == 0."""
    if not grid:
        return []
    first = (start // grid + 1) * grid
    return [p - start for p in range(first, start + L + 1, grid)]


def _gpu_exports(exp_states, w):
    offs = binding.export_offsets(w.lengths, list(w.start_pos), w.export_grid)
    return offs, (None if exp_states is None else exp_states.cpu().numpy())


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", SHAPES)
def test_pure_decay_prefill(dtype, dk, dv, hk, hv):
    """beta = 0: outputs, final states and exports are the decayed initial state."""
    w = W.make_workload("decay", seed=41, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=LENGTHS,
                        num_slots=32, prefill_init="slots", start_pos=STARTS, export_grid=64, gate_scale=0.05)
    w.beta[:] = 0.0
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    atol, rtol = TOL[dtype]
    o = d["o"].float().cpu().numpy()
    pool = d["pool"].cpu().numpy()
    offs, ex = _gpu_exports(exp_states, w)
    cu = w.cu_seqlens()
    G = w.H_v // w.H_k
    for i, L in enumerate(w.lengths):
        a = int(cu[i])
        S0 = w.pool[int(w.init_slot[i])].astype(np.float64)                  # [H_v, d_k, d_v]
        Gc = np.cumsum(w.g[a:a + L].astype(np.float64), axis=0)              # [L, H_v]
        q = w.q[a:a + L].astype(np.float64)[:, np.arange(w.H_v) // G]        # [L, H_v, d_k]
        ref_o = w.scale * np.exp(Gc)[:, :, None] * np.einsum("thk,hkv->thv", q, S0)
        assert_close("o seq %d" % i, o[a:a + L], ref_o, atol, rtol)
        fin = S0 * (np.exp(Gc[-1])[:, None, None] if L else 1.0)
        assert_close("final seq %d" % i, pool[int(w.final_slot[i])], fin, atol, rtol)
        for m, t in enumerate(_grid_points(int(w.start_pos[i]), L, 64)):
            assert_close("export %d of seq %d" % (m, i), ex[offs[i] + m], S0 * np.exp(Gc[t - 1])[:, None, None],
                         atol, rtol)


def _exact16(x):
    """Values exact in bf16 and in fp16 alike (bf16 values of magnitude 2^-12 or more;
    smaller ones are moved to +-2^-12), the formats the kernels feed matrix cores."""
    x = W.round_to_bf16(np.asarray(x, dtype=np.float32))
    tiny = np.abs(x) < 2.0 ** -12
    x[tiny] = np.where(x[tiny] < 0, -(2.0 ** -12), 2.0 ** -12).astype(np.float32)
    return x


def _recall_workload(dtype, dk, dv, hk, hv, seed):
    """g = 0, beta = 1, scale 1; keys of each (sequence, key head) are distinct standard
    basis vectors on rows [0, n_keys); S_0 is zero on those rows and holds values
    exact in every format on the rows above; each query is the key of an earlier token
    of its sequence or one of the rows above."""
    reserve = 8
    n_keys = dk - reserve
    lengths = [n_keys, 1, n_keys - 23, 40, 0]
    starts = [30, 64, 63, 1000, 5]
    w = W.make_workload("recall", seed=seed, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=lengths,
                        num_slots=24, prefill_init="slots", start_pos=starts, export_grid=64, scale=1.0)
    rng = np.random.default_rng(seed + 1)
    w.v[:] = _exact16(w.v)
    w.g[:] = 0.0
    w.beta[:] = 1.0
    w.q[:] = 0.0
    w.k[:] = 0.0
    cu = w.cu_seqlens()
    qrow = np.zeros((w.total_tokens, hk), dtype=np.int64)
    for i, L in enumerate(lengths):
        a = int(cu[i])
        for kh in range(hk):
            perm = rng.permutation(n_keys)[:L]
            for t in range(L):
                w.k[a + t, kh, perm[t]] = 1.0
                # an earlier (or this) token's key, or a row that only S_0 holds
                r = perm[rng.integers(0, t + 1)] if rng.random() < 0.75 else n_keys + rng.integers(0, reserve)
                w.q[a + t, kh, r] = 1.0
                qrow[a + t, kh] = r
    # S_0: zero on the key rows, values exact in every format on the rows above
    s0 = _exact16(rng.standard_normal(w.pool.shape, dtype=np.float32))
    s0[:, :, :n_keys, :] = 0.0
    w.pool[:] = s0
    return w, n_keys, qrow


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", SHAPES)
def test_exact_recall_prefill_is_bitwise(dtype, dk, dv, hk, hv):
    """g = 0, beta = 1, basis keys: every output is a stored value and every state a
    stack of stored rows, bit for bit, through partial chunks, off-grid starts,
    initial states and exports."""
    w, n_keys, qrow = _recall_workload(dtype, dk, dv, hk, hv, seed=43)
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    o = d["o"].float().cpu().numpy()
    pool = d["pool"].cpu().numpy()
    offs, ex = _gpu_exports(exp_states, w)
    cu = w.cu_seqlens()
    G = hv // hk
    for i, L in enumerate(w.lengths):
        a = int(cu[i])
        S = w.pool[int(w.init_slot[i])].astype(np.float32).copy()          # [H_v, d_k, d_v]
        grid = set(_grid_points(int(w.start_pos[i]), L, 64))
        m = 0
        for t in range(L):
            for h in range(hv):
                kh = h // G
                key = int(np.argmax(w.k[a + t, kh]))
                S[h, key] = w.v[a + t, h]
                want = S[h, qrow[a + t, kh]]
                assert np.array_equal(o[a + t, h], want), (i, t, h)
            if t + 1 in grid:
                assert np.array_equal(ex[offs[i] + m], S), ("export", i, m)
                m += 1
        assert np.array_equal(pool[int(w.final_slot[i])], S), ("final", i)


def _forget_expect(w, a, L, G):
    """Full forgetting: per token t and head h, S_t = beta k v^T, o_t = scale beta (k.q) v."""
    h_k = np.arange(w.H_v) // G
    k = w.k[a:a + L].astype(np.float64)[:, h_k]                              # [L, H_v, d_k]
    q = w.q[a:a + L].astype(np.float64)[:, h_k]
    v = w.v[a:a + L].astype(np.float64)
    b = w.beta[a:a + L].astype(np.float64)
    o = w.scale * (b * np.einsum("thk,thk->th", k, q))[:, :, None] * v
    states = b[:, :, None, None] * k[:, :, :, None] * v[:, :, None, :]         # [L, H_v, d_k, d_v]
    return o, states


@pytest.mark.parametrize("dtype,dk,dv,hk,hv", SHAPES)
def test_full_forgetting_prefill(dtype, dk, dv, hk, hv):
    """g = -200: the state keeps only the last token's write, whatever came before
    (initial states from slots are wiped at the first token)."""
    w = W.make_workload("forget", seed=45, H_k=hk, H_v=hv, d_k=dk, d_v=dv, dtype=dtype, lengths=LENGTHS,
                        num_slots=32, prefill_init="slots", start_pos=STARTS, export_grid=64)
    w.g[:] = -200.0
    d = to_device(w)
    exp_states, _ = run_prefill(w, d)
    torch.cuda.synchronize()
    atol, rtol = TOL[dtype]
    o = d["o"].float().cpu().numpy()
    pool = d["pool"].cpu().numpy()
    offs, ex = _gpu_exports(exp_states, w)
    cu = w.cu_seqlens()
    G = hv // hk
    for i, L in enumerate(w.lengths):
        a = int(cu[i])
        ref_o, states = _forget_expect(w, a, L, G)
        assert_close("o seq %d" % i, o[a:a + L], ref_o, atol, rtol)
        fin = states[-1] if L else w.pool[int(w.init_slot[i])]
        assert_close("final seq %d" % i, pool[int(w.final_slot[i])], fin, atol, rtol)
        for m, t in enumerate(_grid_points(int(w.start_pos[i]), L, 64)):
            assert_close("export %d of seq %d" % (m, i), ex[offs[i] + m], states[t - 1], atol, rtol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_pure_decay_and_full_forgetting(dtype):
    """The decode kernel on the same special cases: beta = 0 decays the cached state,
    g = -200 replaces it by beta k v^T."""
    w = W.make_workload("dedge", seed=47, H_k=2, H_v=4, d_k=128, d_v=128, dtype=dtype, num_decode_rows=12,
                        num_slots=32)
    rows = np.arange(12)
    w.beta[:6] = 0.0                 # rows 0-5: pure decay
    w.g[6:] = -200.0                 # rows 6-11: full forgetting
    d = to_device(w)
    o = torch.empty_like(d["v"])
    binding.gdn_recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], o, d["pool"], d["slot_in"],
                                 d["slot_out"], scale=w.scale)
    torch.cuda.synchronize()
    atol, rtol = TOL[dtype]
    got_o = o.float().cpu().numpy()
    got_s = d["pool"].cpu().numpy()[w.slot_out]
    h_k = np.arange(w.H_v) // (w.H_v // w.H_k)
    S0 = w.pool[w.slot_in].astype(np.float64)                                 # [B, H_v, d_k, d_v]
    q = w.q.astype(np.float64)[:, h_k]
    k = w.k.astype(np.float64)[:, h_k]
    v = w.v.astype(np.float64)
    a = np.exp(w.g.astype(np.float64))
    b = w.beta.astype(np.float64)
    dec_s = a[:6, :, None, None] * S0[:6]
    dec_o = w.scale * np.einsum("bhk,bhkv->bhv", q[:6], dec_s)
    fgt_s = b[6:, :, None, None] * k[6:, :, :, None] * v[6:, :, None, :]
    fgt_o = w.scale * (b[6:] * np.einsum("bhk,bhk->bh", k[6:], q[6:]))[:, :, None] * v[6:]
    assert_close("decay o", got_o[:6], dec_o, atol, rtol)
    assert_close("decay states", got_s[:6], dec_s, atol, rtol)
    assert_close("forget o", got_o[6:], fgt_o, atol, rtol)
    assert_close("forget states", got_s[6:], fgt_s, atol, rtol)
    assert rows.size == 12
