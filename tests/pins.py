"""Independent evaluations of the gated delta rule used to pin the oracle.

None of these shares code with the oracle (``oracle/gdn_oracle.c``) or with the GPU
library.  Each is a *different* way of writing the same map:

* ``brute_force_products``: the product form S_t = M_t S_{t-1} + beta_t k_t v_t^T with
  dense transition matrices M_t = alpha_t (I - beta_t k_t k_t^T), composed as matrix
  products (for tiny T and d).
* ``exact_rational``: the same product form in exact rational arithmetic
  (``fractions.Fraction``), with alpha_t given directly.
* ``chunked_ut``: the chunked WY/UT evaluation over chunks of C tokens -- an
  in-chunk cumulative log-decay G, the strictly lower matrix
  A = diag(beta) (K K^T o exp(G_r - G_s)), T = (I + A)^{-1}, W = T diag(beta e^G) K,
  U~ = T diag(beta) V, U = U~ - W S0, outputs scale (diag(e^G) Q S0 + (Q K^T o L o D) U)
  and the carried state e^{G_last} S0 + (diag(e^{G_last - G}) K)^T U.  This is the
  algebra that the GPU prefill kernels use, written in fp64 with library matrix
  products and an explicit inverse.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def brute_force_products(alpha, beta, k, v, q, S0, scale):
    """Single (sequence, head): returns (o [T, d_v], states [T, d_k, d_v])."""
    T, d_k = k.shape
    S = np.array(S0, dtype=np.float64)
    outs, states = [], []
    eye = np.eye(d_k)
    for t in range(T):
        M = alpha[t] * (eye - beta[t] * np.outer(k[t], k[t]))
        S = M @ S + beta[t] * np.outer(k[t], v[t])
        states.append(S.copy())
        outs.append(scale * (S.T @ q[t]))
    return np.array(outs), np.array(states)


def exact_rational(alpha, beta, k, v, q, S0, scale):
    """Same product form with Fractions; inputs are sequences of Fractions/ints."""
    T = len(k)
    d_k = len(k[0])
    d_v = len(v[0])
    S = [[Fraction(S0[i][j]) for j in range(d_v)] for i in range(d_k)]
    outs, states = [], []
    for t in range(T):
        a, b = Fraction(alpha[t]), Fraction(beta[t])
        kt = [Fraction(x) for x in k[t]]
        vt = [Fraction(x) for x in v[t]]
        qt = [Fraction(x) for x in q[t]]
        # M S = a (S - b k (k^T S))
        kTS = [sum(kt[i] * S[i][j] for i in range(d_k)) for j in range(d_v)]
        S = [[a * (S[i][j] - b * kt[i] * kTS[j]) + b * kt[i] * vt[j] for j in range(d_v)]
             for i in range(d_k)]
        states.append([row[:] for row in S])
        outs.append([Fraction(scale) * sum(S[i][j] * qt[i] for i in range(d_k)) for j in range(d_v)])
    return outs, states


def chunked_ut(g, beta, k, v, q, S0, scale, C):
    """Single (sequence, head) chunked evaluation; returns (o [T, d_v], S_final)."""
    T, d_k = k.shape
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        L = c1 - c0
        K, V, Q = k[c0:c1], v[c0:c1], q[c0:c1]
        b = beta[c0:c1]
        G = np.cumsum(g[c0:c1])
        D = np.exp(G[:, None] - G[None, :])           # D[r, s] = exp(G_r - G_s)
        strict = np.tril(np.ones((L, L)), -1)
        incl = np.tril(np.ones((L, L)), 0)
        A = (b[:, None] * (K @ K.T)) * D * strict
        Tm = np.linalg.inv(np.eye(L) + A)
        W = Tm @ ((b * np.exp(G))[:, None] * K)
        U = Tm @ (b[:, None] * V) - W @ S
        o[c0:c1] = scale * (np.exp(G)[:, None] * (Q @ S) + ((Q @ K.T) * D * incl) @ U)
        S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ U
    return o, S
