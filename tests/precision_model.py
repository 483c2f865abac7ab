"""An fp64 model of the roundings of the bf16 chunk-prefill kernel, for one
(sequence, value head) chain.

Test infrastructure only: it shares no code with the GPU library or the oracle.  It
follows the chunked form the kernel evaluates (per 64-token chunk: A =
strict_lower(diag(beta) K K^T o D), R = diag(beta) (V - diag(gamma) K S), the 16-row
block solve U_i = T_ii (R_i - sum_{j<i} A_ij U_j) with T_ii = (I + A_ii)^-1, O = scale
(diag(gamma) Q S + (Q K^T o D o lower-incl) U), S <- gamma_last S + K^T (diag(e^(G_last
- G)) U)) and rounds exactly where the kernel feeds a matrix core, each operand in
one of these forms:
    "bf16", "f16"      one rounding to that format
    "bf16x2", "f16x2"  a hi + lo pair in that format (x - hi rounded once more), in
                       three products (hi hi + hi lo + lo hi) when both sides are
                       pairs, two when one side is exact
    "exact"            no rounding
Everything else (accumulation, gates, the diagonal inverses) is kept in fp64, which
is finer than the kernel's fp32 and does not change what the model is for: showing
which roundings a bound can or cannot absorb.

KERNEL is the kernel's scheme: q and k in fp16; S once to fp16 in K S and Q S; -A_ij
and U as fp16 pairs in the solve; T_ii and the right-hand side single fp16; P and U
single fp16 in the output product; the decayed U as an fp16 pair in the state
update.  EARLIER is the previous all-bf16 scheme (S once to bf16, every other operand
a bf16 pair), kept for comparison.
"""
from __future__ import annotations

import numpy as np

from gated_deltanet_rule_amd.workloads import round_to_bf16

C = 64
BLOCK = 16

KERNEL = dict(qk="f16", s="f16", solve_a="f16x2", solve_u="f16x2", tii="f16", rhs="f16", out_p="f16",
              out_u="f16", upd_u="f16x2")
EARLIER = dict(qk="exact", s="bf16", solve_a="bf16x2", solve_u="bf16x2", tii="bf16x2", rhs="bf16x2",
               out_p="bf16x2", out_u="bf16x2", upd_u="bf16x2")


def bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _round(fmt, x):
    x = np.asarray(x, dtype=np.float64)
    if fmt == "exact":
        return x
    return {"bf16": bf16, "f16": f16}[fmt](x)


def parts(form, x):
    """The pieces an operand enters a product as: [x] rounded once, or [hi, lo]."""
    if form.endswith("x2"):
        hi = _round(form[:-2], x)
        return [hi, _round(form[:-2], np.asarray(x, dtype=np.float64) - hi)]
    return [_round(form, x)]


def product(fa, a, fb, b):
    """a @ b with each side in its form; the lo-lo term of two pairs is dropped."""
    pa, pb = parts(fa, a), parts(fb, b)
    out = pa[0] @ pb[0]
    if len(pb) > 1:
        out = out + pa[0] @ pb[1]
    if len(pa) > 1:
        out = out + pa[1] @ pb[0]
    return out


def chain(q, k, v, g, beta, scale, S0, scheme=KERNEL, **override):
    """One chain: q, k [T, d_k]; v [T, d_v]; g, beta [T]; S0 [d_k, d_v].  Returns
    (o [T, d_v] rounded to bf16, the states after each chunk [ceil(T / 64), d_k,
    d_v]; the last one is the final state).  ``override`` replaces single entries of
    the scheme."""
    f = dict(scheme, **override)
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    states = []
    q = _round(f["qk"], q)
    k = _round(f["qk"], k)
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        Q, K, V = q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L]
        G = np.cumsum(g[c0:c0 + L])
        gam, b = np.exp(G), beta[c0:c0 + L]
        D = np.exp(G[:, None] - G[None, :])
        A = np.tril(b[:, None] * (K @ K.T) * D, -1)
        P = np.tril(scale * (Q @ K.T) * D)
        Ss = _round(f["s"], S)
        R = b[:, None] * (V - gam[:, None] * (K @ Ss))
        U = np.zeros_like(R)
        for i in range(0, L, BLOCK):
            ri = slice(i, min(i + BLOCK, L))
            X = R[ri].copy()
            for j in range(0, i, BLOCK):
                rj = slice(j, j + BLOCK)
                X += product(f["solve_a"], -A[ri, rj], f["solve_u"], U[rj])
            Tii = np.linalg.inv(np.eye(ri.stop - i) + A[ri, ri])
            U[ri] = product(f["tii"], Tii, f["rhs"], X)
        PU = product(f["out_p"], P, f["out_u"], U)
        o[c0:c0 + L] = bf16(scale * gam[:, None] * (Q @ Ss) + PU)
        dU = np.exp(G[-1] - G)[:, None] * U
        S = gam[-1] * S + product("exact", K.T, f["upd_u"], dU)
        states.append(S)
    return o, np.array(states)
