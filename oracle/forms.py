"""Masked-parallel and chunk-parallel forms of the Falcon recurrence, numpy fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  These exist to
cross-check the recurrent oracle: the authors' abstract of "Fast Weight
Attention for Continual Learning" states that every rule of the family has a
recurrent, a masked-parallel and a chunk-parallel form, with positive-decay
renormalization.  Agreement of three differently organised computations is
one of the oracle's pins.

Algebra used (one (batch, head) sequence, a segment of L steps that starts
from the state S0):

* Each step s contributes "virtual examples" (s, w), w = 0..Wv-1 (Wv = W for
  Falcon-3/3A, 1 otherwise) with key x_{s-w} = k_{s-w-lag} (lag 1: prefix
  alignment, 0: same-step), target y_{s-w} and write vector
  omega_(s,w): u_s for Falcon-1/2 (and the A forms), b_s x_{s-w} for Falcon-3.
* g_s is the cumulative log-decay from the segment start and
  D(t, s) = exp(g_t - g_s) <= 1 for s <= t: every decay factor is a ratio of a
  later to an earlier cumulative product, formed in log space (the reading
  of "positive-decay renormalization").
* Regression family: the residuals Delta of all virtual examples solve the
  unit lower-triangular system
      (I + A) Delta = Y - diag(gamma_s(i)) X S0^T,
      A[i, j] = [s(j) < s(i)] D(s(i), s(j)) (x_i . omega_j);
  inner-product family: Delta = Y.
* o_t = gamma_t S0 q_t + sum_{j: s(j) <= t} D(t, s(j)) (omega_j . q_t) Delta_j
  (read after the write, so the step's own examples are included);
  S_end = gamma_{L-1} S0 + sum_j D(L-1, s(j)) Delta_j omega_j^T.

The masked-parallel form is one segment over the whole sequence; the
chunk-parallel form runs segments of C steps and carries S between them.
"""
from __future__ import annotations

import numpy as np

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
_NAMES = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}


def _halo_keys(k, k_prev, W):
    """Keys k_tau for tau = -W .. T-1 as one array (index tau + W)."""
    T, dk = k.shape
    pre = np.zeros((W, dk)) if k_prev is None else np.asarray(k_prev, np.float64)
    return np.concatenate([pre, k], axis=0)


def _halo_vals(v, v_prev, W):
    """Values v_tau for tau = -(W-1) .. T-1 (index tau + W - 1)."""
    T, dv = v.shape
    if W == 1:
        return v
    pre = np.zeros((W - 1, dv)) if v_prev is None else np.asarray(v_prev, np.float64)
    return np.concatenate([pre, v], axis=0)


def _segment(variant, S0, q, kh, vh, alpha, eta, t0, L, W, eps, lag):
    """Masked form of one segment [t0, t0+L) of one sequence."""
    regression = variant in (F1, F2, F3)
    Wv = W if variant in (F3, F3A) else 1
    dk = kh.shape[1]
    rows_x, rows_y, rows_w, step = [], [], [], []
    for s in range(L):
        t = t0 + s
        xs = [kh[t - w - lag + W] for w in range(Wv)]   # x_{t-w} = k_{t-w-lag}
        ys = [vh[t - w + W - 1] for w in range(Wv)]   # y_{t-w} = v_{t-w}
        if variant in (F1, F1A):
            x = xs[0]
            om = [eta[t] * x / (x @ x + eps)]
        elif variant in (F2, F2A):
            x = xs[0]
            l1 = np.abs(x).sum()
            om = [eta[t] * x / (np.abs(x) * l1 + eps)]
        else:
            b = eta[t] / (sum(x @ x for x in xs) + eps)
            om = [b * x for x in xs]
        rows_x += xs
        rows_y += ys
        rows_w += om
        step += [s] * Wv
    X = np.array(rows_x).reshape(-1, dk)
    Y = np.array(rows_y).reshape(len(rows_x), -1)
    Om = np.array(rows_w).reshape(-1, dk)
    step = np.array(step)
    g = np.cumsum(np.log(alpha[t0:t0 + L]))
    gam = np.exp(g)

    def decay(ti, sj, strict):
        """D(ti, sj) where sj < ti (strict) or sj <= ti, else 0."""
        m = (sj[None, :] < ti[:, None]) if strict else (sj[None, :] <= ti[:, None])
        e = np.where(m, g[ti][:, None] - g[sj][None, :], -np.inf)
        return np.exp(e)

    if regression:
        A = decay(step, step, True) * (X @ Om.T)
        rhs = Y - gam[step][:, None] * (X @ S0.T)
        Delta = np.linalg.solve(np.eye(len(step)) + A, rhs)
    else:
        Delta = Y
    tt = np.arange(L)
    Qs = q[t0:t0 + L]
    P = decay(tt, step, False) * (Qs @ Om.T)
    O = gam[:, None] * (Qs @ S0.T) + P @ Delta
    hend = np.exp(g[-1] - g[step])
    S_end = gam[-1] * S0 + (Delta * hend[:, None]).T @ Om
    return O, S_end


def chunked(variant, q, k, v, alpha, eta, *, chunk, window=1, eps=1e-6, S0=None, k_prev=None,
            v_prev=None, lag=1):
    """Chunk-parallel form with chunks of `chunk` steps (chunk >= T gives the
    masked-parallel form).  Same argument shapes as the recurrent oracle."""
    variant = _NAMES.get(variant, variant)
    q, k, v, alpha, eta = (np.asarray(a, np.float64) for a in (q, k, v, alpha, eta))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    W = window
    o = np.zeros((B, H, T, dv))
    S_out = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            kh = _halo_keys(k[b, h], None if k_prev is None else k_prev[b, h], W)
            vh = _halo_vals(v[b, h], None if v_prev is None else v_prev[b, h], W)
            S = np.zeros((dv, dk)) if S0 is None else np.asarray(S0[b, h], np.float64).copy()
            for t0 in range(0, T, chunk):
                L = min(chunk, T - t0)
                O, S = _segment(variant, S, q[b, h], kh, vh, alpha[b, h], eta[b, h], t0, L, W,
                                eps, lag)
                o[b, h, t0:t0 + L] = O
            S_out[b, h] = S
    return o, S_out


def masked(variant, q, k, v, alpha, eta, **kw):
    """Masked-parallel form: a single segment covering the whole sequence."""
    T = np.asarray(k).shape[2]
    return chunked(variant, q, k, v, alpha, eta, chunk=max(T, 1), **kw)
