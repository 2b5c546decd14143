"""Exact rational brute force for the KDA recurrence (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see ``oracle/kda_oracle.py``).

This is a second, structurally different statement of the same recurrence,
used to pin the float64 oracle.  Instead of stepping a state, it builds the
dense transition matrix of every token,

    A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)          (generalized Householder
                                                         times per-channel decay)

and expands the state as an explicit sum of matrix products,

    S_t = (A_t ... A_1) S_0 + sum_{s<=t} (A_t ... A_{s+1}) beta_s k_s v_s^T,
    o_t = scale * S_t^T q_t,

all in ``fractions.Fraction`` so that nothing is rounded.  The decay is given
directly as a rational alpha (the float64 oracle is fed g = ln(alpha)).
Sources: "Kimi K3 from Moonshot AI ...", section "Kimi Delta Attention (KDA)"
(delta rule on the generalized Householder transformation) and "Kimi K3
Architecture Explained ...", section "Token mixing" (per-channel forget gate).
"""
from __future__ import annotations

from fractions import Fraction

__all__ = ["rational_kda"]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def _matmul(a, b):
    n, m, p = len(a), len(b), len(b[0])
    return [[sum((a[i][r] * b[r][j] for r in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def _transition(alpha, beta, k):
    n = len(k)
    house = [[Fraction(int(i == j)) - beta * k[i] * k[j] for j in range(n)] for i in range(n)]
    decay = [[alpha[i] if i == j else Fraction(0) for j in range(n)] for i in range(n)]
    return _matmul(house, decay)


def rational_kda(q, k, v, alpha, beta, s0, scale=Fraction(1)):
    """Single (batch, head) sequence.

    q, k: lists of T vectors of dk Fractions; v: T vectors of dv Fractions;
    alpha: T vectors of dk Fractions (retention factors, 0 < alpha <= 1);
    beta: T Fractions; s0: dk x dv nested list.  Returns (o: T x dv, S_T).
    """
    T = len(q)
    dk, dv = len(k[0]), len(v[0])
    A = [_transition(alpha[t], beta[t], k[t]) for t in range(T)]
    outs = []
    S_t = None
    for t in range(T):
        # (A_t ... A_1) S_0
        prod = _eye(dk)
        for r in range(t, -1, -1):
            prod = _matmul(prod, A[r])
        S_t = _matmul(prod, s0)
        for s in range(t + 1):
            tail = _eye(dk)
            for r in range(t, s, -1):
                tail = _matmul(tail, A[r])
            write = [[beta[s] * k[s][i] * v[s][j] for j in range(dv)] for i in range(dk)]
            S_t = _add(S_t, _matmul(tail, write))
        outs.append([scale * sum((S_t[i][j] * q[t][i] for i in range(dk)), Fraction(0))
                     for j in range(dv)])
    return outs, S_t
