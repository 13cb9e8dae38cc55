"""The Falcon recurrence in exact rational arithmetic (fractions.Fraction).

TEST INFRASTRUCTURE ONLY.  For tiny inputs (a handful of steps, d <= 3) with
rational alpha, eta and eps this gives the exact result of the recurrence, so
it bounds the rounding of the fp64 oracle.  Every step follows the same
definition as the C oracle (decay, then the normalized write, then the read;
see falcon_oracle.c for the sources), written independently here with lists
of Fractions.  Only sign and absolute value are needed for Falcon-2's
normalizer, so no irrational operation occurs.
"""
from __future__ import annotations

from fractions import Fraction as Fr

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
_NAMES = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}


def _dot(a, b):
    return sum((x * y for x, y in zip(a, b)), Fr(0))


def recurrent_seq(variant, q, k, v, alpha, eta, *, window=1, eps=Fr(0), S0=None, k_prev=None,
                  v_prev=None, lag=1):
    """One sequence.  q, k: T lists of dk Fractions; v: T lists of dv; alpha,
    eta: T Fractions; the key of step t's pair w is k_{t-w-lag} (lag 1:
    prefix alignment, 0: same-step).  Returns (o as T lists of dv, S as dv
    lists of dk)."""
    variant = _NAMES.get(variant, variant)
    T = len(k)
    dk = len(k[0]) if T else len(S0[0])
    dv = len(v[0]) if T else len(S0)
    W = window
    zk, zv = [Fr(0)] * dk, [Fr(0)] * dv

    def key(tau):
        if tau >= 0:
            return k[tau]
        return k_prev[W + tau] if k_prev is not None else zk

    def val(tau):
        if tau >= 0:
            return v[tau]
        return v_prev[W - 1 + tau] if v_prev is not None else zv

    S = [[Fr(0)] * dk for _ in range(dv)] if S0 is None else [list(r) for r in S0]
    out = []
    for t in range(T):
        a, e = Fr(alpha[t]), Fr(eta[t])
        S = [[a * s for s in row] for row in S]
        if variant in (F3, F3A):
            pairs = [(key(t - w - lag), val(t - w)) for w in range(W)]
            b = e / (sum(_dot(x, x) for x, _ in pairs) + eps)
            if variant == F3:
                coef = [[b * (y[i] - _dot(S[i], x)) for i in range(dv)] for x, y in pairs]
            else:
                coef = [[b * y[i] for i in range(dv)] for _, y in pairs]
            for (x, _), c in zip(pairs, coef):
                for i in range(dv):
                    for j in range(dk):
                        S[i][j] += c[i] * x[j]
        else:
            x, y = key(t - lag), v[t]
            if variant in (F1, F1A):
                n = _dot(x, x) + eps
                u = [e * xj / n for xj in x]
            else:
                l1 = sum((abs(xj) for xj in x), Fr(0))
                u = [e * xj / (abs(xj) * l1 + eps) for xj in x]
            if variant in (F1, F2):
                r = [y[i] - _dot(S[i], x) for i in range(dv)]
            else:
                r = list(y)
            for i in range(dv):
                for j in range(dk):
                    S[i][j] += r[i] * u[j]
        out.append([_dot(S[i], q[t]) for i in range(dv)])
    return out, S
