"""Pins of the gradient oracle (oracle/grad.py).

The gradient oracle is torch autograd over a second, independent writing of
the recurrence in float64.  It is pinned here by:
  * its forward equals the C oracle's forward (every variant, window, both
    alignments, feature maps, halos and initial state);
  * central finite differences of the C oracle's forward: the directional
    derivative of L = sum(o d_o) + sum(S_T dS_T) along a random direction of
    each input equals <gradient, direction>, and single entries likewise --
    brute force that catches any dropped term, sign or index in either the
    rewritten forward or the way gradients are read off;
  * closed forms that hold for every variant (dq_t = S_t^T d_o_t, since
    o_t = S_t q_t and S_t does not depend on q) and for the inner-product
    family (decayed linear attention: dv_t and dS0 written out as sums);
  * the empty sequence (T = 0): only dS0 = dS_T is nonzero.
"""
import numpy as np
import pytest

import oracle
from oracle import grad

ALL = ["F1", "F2", "F3", "F1A", "F2A", "F3A"]
INPUTS = ["q", "k", "v", "alpha", "eta", "S0", "k_prev", "v_prev"]


def rnd(seed, B=1, H=2, T=9, dk=5, dv=4, W=1, halo=True, S0=True):
    r = np.random.default_rng(seed)
    d = dict(q=r.standard_normal((B, H, T, dk)), k=r.standard_normal((B, H, T, dk)),
             v=r.standard_normal((B, H, T, dv)), alpha=r.uniform(0.5, 0.99, (B, H, T)),
             eta=r.uniform(0.05, 1.0, (B, H, T)))
    d["S0"] = r.standard_normal((B, H, dv, dk)) if S0 else None
    d["k_prev"] = r.standard_normal((B, H, W, dk)) if halo else None
    d["v_prev"] = r.standard_normal((B, H, W - 1, dv)) if (halo and W > 1) else None
    d["d_o"] = r.standard_normal((B, H, T, dv))
    d["dS_T"] = r.standard_normal((B, H, dv, dk))
    return d


def c_loss(variant, d, W, align, phi, eps=1e-6):
    o, S = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=W,
                            eps=eps, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"],
                            align=align, phi=phi)
    return float((o * d["d_o"]).sum() + (S * d["dS_T"]).sum())


def g_all(variant, d, W, align, phi, eps=1e-6):
    return grad.gradients(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], d["d_o"],
                          d["dS_T"], window=W, eps=eps, S0=d["S0"], k_prev=d["k_prev"],
                          v_prev=d["v_prev"], align=align, phi=phi)


CASES = [(v, W, al, ph) for v in ALL for W in ([1, 2, 3] if v in ("F3", "F3A") else [1])
         for al in ("prefix", "same") for ph in ("identity",)]
CASES += [(v, W, "prefix", ph) for v, W in (("F1", 1), ("F1A", 1), ("F2", 1), ("F3", 2))
          for ph in ("l2", "silu")]


@pytest.mark.parametrize("variant,W,align,phi", CASES)
def test_forward_equals_c_oracle(variant, W, align, phi):
    import torch
    d = rnd(11, W=W)
    t = {n: (torch.tensor(d[n]) if d[n] is not None else None) for n in INPUTS}
    o, S = grad.forward(variant, t["q"], t["k"], t["v"], t["alpha"], t["eta"], window=W,
                        S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"], align=align,
                        phi=phi)
    o2, S2 = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=W,
                              S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"], align=align,
                              phi=phi)
    np.testing.assert_allclose(o.numpy(), o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S.numpy(), S2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant,W,align,phi", CASES)
def test_directional_finite_differences(variant, W, align, phi):
    d = rnd(23, W=W)
    g = g_all(variant, d, W, align, phi)
    r = np.random.default_rng(5)
    h = 1e-5
    for name in INPUTS:
        if d[name] is None or name not in g:
            continue
        dirn = r.standard_normal(d[name].shape)
        dirn /= np.linalg.norm(dirn)
        p, m = dict(d), dict(d)
        p[name] = d[name] + h * dirn
        m[name] = d[name] - h * dirn
        fd = (c_loss(variant, p, W, align, phi) - c_loss(variant, m, W, align, phi)) / (2 * h)
        an = float((g[name] * dirn).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("variant", ALL)
def test_entrywise_finite_differences(variant):
    W = 2 if variant in ("F3", "F3A") else 1
    d = rnd(31, T=6, W=W)
    g = g_all(variant, d, W, "prefix", "identity")
    r = np.random.default_rng(7)
    h = 1e-5
    for name in INPUTS:
        if d[name] is None or name not in g:
            continue
        for _ in range(4):
            idx = tuple(r.integers(0, s) for s in d[name].shape)
            if variant in ("F2", "F2A") and name in ("k", "k_prev") and abs(d[name][idx]) < 1e-3:
                continue  # the per-column normalizer has a kink at x_j = 0 (|x_j|)
            p, m = dict(d), dict(d)
            p[name] = d[name].copy()
            m[name] = d[name].copy()
            p[name][idx] += h
            m[name][idx] -= h
            fd = (c_loss(variant, p, W, "prefix", "identity")
                  - c_loss(variant, m, W, "prefix", "identity")) / (2 * h)
            assert abs(fd - g[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx)


@pytest.mark.parametrize("variant", ALL)
def test_dq_is_state_transpose_times_do(variant):
    """o_t = S_t q_t with S_t independent of q: dq_t = S_t^T d_o_t."""
    W = 3 if variant in ("F3", "F3A") else 1
    d = rnd(41, T=7, W=W)
    g = g_all(variant, d, W, "prefix", "identity")
    for t in range(7):
        pre = {n: (d[n][:, :, :t + 1] if n in ("q", "k", "v", "alpha", "eta") else d[n])
               for n in INPUTS}
        _, St = oracle.recurrent(variant, pre["q"], pre["k"], pre["v"], pre["alpha"], pre["eta"],
                                 window=W, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"])
        want = np.einsum("bhvk,bhv->bhk", St, d["d_o"][:, :, t])
        np.testing.assert_allclose(g["q"][:, :, t], want, rtol=0, atol=1e-11)


def test_inner_product_family_closed_form():
    """Falcon-1A is decayed linear attention with write vectors
    u_t = eta_t x_t / (||x_t||^2 + eps), x_t = k_{t-1}:
      S_T = G(0,T] S0 + sum_t G(t,T] v_t u_t^T,   o_s = S_s q_s,
    with G(a,b] the product of alpha over steps a+1..b.  Hence
      dv_t = sum_{s>=t} G(t,s] (u_t . q_s) d_o_s + G(t,T] dS_T u_t,
      dS0  = sum_s G(0,s] d_o_s q_s^T + G(0,T] dS_T."""
    d = rnd(53, B=1, H=1, T=8, W=1)
    g = g_all("F1A", d, 1, "prefix", "identity")
    q, k, v, al, et = (d[n][0, 0] for n in ("q", "k", "v", "alpha", "eta"))
    do, dST = d["d_o"][0, 0], d["dS_T"][0, 0]
    T = q.shape[0]
    x = np.vstack([d["k_prev"][0, 0, -1:], k[:-1]])
    u = et[:, None] * x / ((x * x).sum(1, keepdims=True) + 1e-6)

    def G(a, b):  # product of alpha over steps a+1 .. b (indices a+1..b, 0-based: a+1..b)
        return float(np.prod(al[a + 1:b + 1]))

    dv = np.zeros_like(v)
    for t in range(T):
        for s in range(t, T):
            dv[t] += G(t, s) * (u[t] @ q[s]) * do[s]
        dv[t] += G(t, T - 1) * (dST @ u[t])
    np.testing.assert_allclose(g["v"][0, 0], dv, rtol=0, atol=1e-11)
    dS0 = sum(G(-1, s) * np.outer(do[s], q[s]) for s in range(T)) + G(-1, T - 1) * dST
    np.testing.assert_allclose(g["S0"][0, 0], dS0, rtol=0, atol=1e-11)


@pytest.mark.parametrize("variant", ["F1", "F3A"])
def test_empty_sequence(variant):
    W = 2 if variant == "F3A" else 1
    d = rnd(61, T=0, W=W)
    g = g_all(variant, d, W, "prefix", "identity")
    np.testing.assert_array_equal(g["S0"], d["dS_T"])
    for n in ("q", "k", "v", "alpha", "eta", "k_prev"):
        assert not np.any(g[n])


def test_zero_key_under_l2_map_has_zero_gradient():
    """phi(0) = 0 is a constant branch: the zero key gets no gradient, and no
    NaN leaks into the others."""
    d = rnd(71, T=6)
    d["k"][0, 0, 2] = 0.0
    g = g_all("F1", d, 1, "prefix", "l2")
    assert np.all(np.isfinite(g["k"])) and not np.any(g["k"][0, 0, 2])
