"""An fp64 model of the roundings of the bf16 chunk-prefill kernel, for one
(sequence, value head) chain.

Test infrastructure only: it shares no code with the GPU library or the oracle.  It
follows the chunked form the kernel evaluates (per 64-token chunk: A =
strict_lower(diag(beta) K K^T o D), R = diag(beta) (V - diag(gamma) K S), the 16-row
block solve U_i = T_ii (R_i - sum_{j<i} A_ij U_j) with T_ii = (I + A_ii)^-1, O = scale
(diag(gamma) Q S + (Q K^T o D o lower-incl) U), S <- gamma_last S + K^T (diag(e^(G_last
- G)) U)) and rounds to bf16 exactly where the kernel feeds a matrix core: S as one
bf16 value in K S and Q S; the -A_ij, T_ii and P blocks, the right-hand sides, U and
the decayed U as hi + lo pairs in three products (two where the other side is exact).
Everything else (accumulation, gates, the diagonal inverses) is kept in fp64, which
is finer than the kernel's fp32 and does not change what the model is for: showing
which roundings a bound can or cannot absorb.

``split_output=False`` models the earlier form in which P and U entered the output
product as single bf16 values; ``split_state_update=False`` drops the lo part of the
decayed U in the state update.
"""
from __future__ import annotations

import numpy as np

from gated_deltanet_rule_amd.workloads import round_to_bf16

C = 64
BLOCK = 16


def bf16(x):
    return round_to_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def split(x):
    """x = hi + lo: hi the nearest bf16, lo the remainder rounded to bf16 once."""
    x = np.asarray(x, dtype=np.float64)
    hi = bf16(x)
    return hi, bf16(x - hi)


def split_product(a, b):
    """a b with both sides as hi + lo pairs, three products (hi hi + hi lo + lo hi)."""
    ah, al = split(a)
    bh, bl = split(b)
    return ah @ bh + ah @ bl + al @ bh


def chain(q, k, v, g, beta, scale, S0, split_output=True, split_state_update=True):
    """One chain: q, k [T, d_k]; v [T, d_v]; g, beta [T]; S0 [d_k, d_v].  Returns
    (o [T, d_v] rounded to bf16, final state [d_k, d_v])."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        Q, K, V = q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L]
        G = np.cumsum(g[c0:c0 + L])
        gam, b = np.exp(G), beta[c0:c0 + L]
        D = np.exp(G[:, None] - G[None, :])
        A = np.tril(b[:, None] * (K @ K.T) * D, -1)
        P = np.tril(scale * (Q @ K.T) * D)
        Sb = bf16(S)
        R = b[:, None] * (V - gam[:, None] * (K @ Sb))
        U = np.zeros_like(R)
        for i in range(0, L, BLOCK):
            ri = slice(i, min(i + BLOCK, L))
            X = R[ri].copy()
            for j in range(0, i, BLOCK):
                rj = slice(j, j + BLOCK)
                X += split_product(-A[ri, rj], U[rj])
            Tii = np.linalg.inv(np.eye(ri.stop - i) + A[ri, ri])
            U[ri] = split_product(Tii, X)
        if split_output:
            PU = split_product(P, U)
        else:
            PU = bf16(P) @ bf16(U)
        o[c0:c0 + L] = bf16(scale * gam[:, None] * (Q @ Sb) + PU)
        dU = np.exp(G[-1] - G)[:, None] * U
        hi, lo = split(dU)
        S = gam[-1] * S + K.T @ hi + (K.T @ lo if split_state_update else 0.0)
    return o, S
