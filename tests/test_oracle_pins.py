"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The pages print no worked numbers, so the oracle is pinned by:
  * hand-derived exact examples (tests/golden/hand_examples.json);
  * exact rational arithmetic on tiny inputs (rounding bound);
  * interpolation / gain identities of the normalized (NLMS/Kaczmarz) step
    (KLA abstract: step eta/(||k||^2+eps), derived from Kaczmarz projection);
  * contraction towards a consistent target (Kaczmarz/NLMS property);
  * reductions between variants (Falcon-3 with W=1 is Falcon-1, Falcon-2 is
    Falcon-1 on keys of constant magnitude, Falcon-1 is KLA/GDN run on keys
    shifted by one step -- prefix alignment in the authors' abstract);
  * the closed form of the inner-product family as decayed linear attention;
  * agreement of the recurrent, masked-parallel and chunk-parallel forms
    (the authors' abstract states all three exist), also under extreme decays;
  * decay-only, continuation and linearity properties.
Each is chosen so that a plausible slip in the oracle (a dropped decay, a
read before the write, the unshifted key, a wrong sign or normalizer, a
residual taken at the undecayed state) fails at least one of them.
"""
import json
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import exact, forms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
ALL = ["F1", "F2", "F3", "F1A", "F2A", "F3A"]


def rnd(seed, B=1, H=2, T=12, dk=5, dv=4, W=1, halo=True, S0=True, alpha_lo=0.5, eta_hi=1.0):
    r = np.random.default_rng(seed)
    d = dict(q=r.standard_normal((B, H, T, dk)), k=r.standard_normal((B, H, T, dk)),
             v=r.standard_normal((B, H, T, dv)),
             alpha=r.uniform(alpha_lo, 1.0, (B, H, T)), eta=r.uniform(0.05, eta_hi, (B, H, T)))
    d["S0"] = r.standard_normal((B, H, dv, dk)) if S0 else None
    d["k_prev"] = r.standard_normal((B, H, W, dk)) if halo else None
    d["v_prev"] = r.standard_normal((B, H, W - 1, dv)) if (halo and W > 1) else None
    return d


def run(variant, d, W=1, eps=1e-6, **kw):
    return oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=W,
                            eps=eps, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"], **kw)


def wins(v):
    return [1, 2, 3] if v in ("F3", "F3A") else [1]


# ---------------------------------------------------------------- golden ----
def _fr(x):
    if isinstance(x, list) and len(x) == 2 and all(isinstance(e, int) for e in x):
        return Fr(x[0], x[1])
    return [_fr(e) for e in x]


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_examples(case):
    W = case["window"]
    f = lambda key: None if case[key] is None else np.array(  # noqa: E731
        [[float(Fr(*e)) for e in row] for row in case[key]])
    q, k, v = f("q"), f("k"), f("v")
    alpha = np.array([float(Fr(*a)) for a in case["alpha"]])
    eta = np.array([float(Fr(*a)) for a in case["eta"]])
    kp = f("k_prev")
    vp = f("v_prev")
    o, S = oracle.recurrent(case["variant"], q[None, None], k[None, None], v[None, None],
                            alpha[None, None], eta[None, None], window=W,
                            eps=float(Fr(*case["eps"])), k_prev=kp[None, None],
                            v_prev=None if vp is None else vp[None, None])
    o_exp = np.array([[float(Fr(*e)) for e in row] for row in case["o"]])
    S_exp = np.array([[float(Fr(*e)) for e in row] for row in case["S"]])
    np.testing.assert_allclose(o[0, 0], o_exp, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], S_exp, rtol=1e-14, atol=1e-15)
    # the exact-arithmetic form reproduces the hand derivation exactly
    oe, Se = exact.recurrent_seq(case["variant"], _fr(case["q"]), _fr(case["k"]),
                                 _fr(case["v"]), _fr(case["alpha"]), _fr(case["eta"]),
                                 window=W, eps=Fr(*case["eps"]), k_prev=_fr(case["k_prev"]),
                                 v_prev=None if case["v_prev"] is None else _fr(case["v_prev"]))
    assert oe == _fr(case["o"])
    assert Se == _fr(case["S"])


# ----------------------------------------------------------------- P1 -------
@pytest.mark.parametrize("variant", ALL)
def test_exact_rational_matches_fp64(variant):
    r = np.random.default_rng(11)
    for W in wins(variant):
        for T, dk, dv in [(1, 2, 2), (4, 3, 2), (6, 2, 3)]:
            ri = lambda *s: r.integers(-4, 5, s)  # noqa: E731
            q, k, v = ri(T, dk), ri(T, dk), ri(T, dv)
            kp, vp = ri(W, dk), ri(W - 1, dv)
            S0 = ri(dv, dk)
            al = [Fr(int(a), 8) for a in r.integers(1, 9, T)]
            et = [Fr(int(a), 4) for a in r.integers(0, 5, T)]
            eps = Fr(1, 16)
            F = lambda a: [[Fr(int(x)) for x in row] for row in a]  # noqa: E731
            oe, Se = exact.recurrent_seq(variant, F(q), F(k), F(v), al, et, window=W, eps=eps,
                                         S0=F(S0), k_prev=F(kp),
                                         v_prev=F(vp) if W > 1 else None)
            o, S = oracle.recurrent(variant, q[None, None], k[None, None], v[None, None],
                                    np.array([float(a) for a in al])[None, None],
                                    np.array([float(a) for a in et])[None, None], window=W,
                                    eps=float(eps), S0=S0[None, None], k_prev=kp[None, None],
                                    v_prev=vp[None, None] if W > 1 else None)
            oe = np.array([[float(x) for x in row] for row in oe])
            Se = np.array([[float(x) for x in row] for row in Se])
            scale = max(1.0, np.abs(oe).max())
            assert np.abs(o[0, 0] - oe).max() <= 1e-13 * scale
            assert np.abs(S[0, 0] - Se).max() <= 1e-13 * max(1.0, np.abs(Se).max())


# ----------------------------------------------------------------- P2 -------
@pytest.mark.parametrize("variant", ["F1", "F2"])
def test_interpolation_read_after_write(variant):
    """alpha=1, eta=1, eps=0: the write makes S_t x_t = y_t exactly; reading
    with q_t = x_t therefore returns y_t (a read before the write would not)."""
    d = rnd(2, T=10, dk=6, dv=3)
    d["alpha"][:] = 1.0
    d["eta"][:] = 1.0
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)
    d["q"] = kh[:, :, :-1].copy()                     # q_t = x_t = k_{t-1}
    o, _ = run(variant, d, eps=0.0)
    np.testing.assert_allclose(o, d["v"], rtol=1e-11, atol=1e-11)


def test_interpolation_falcon3_single_pair():
    """Falcon-3, W=2, keys zero at every other index: each window holds one
    nonzero pair, which the step interpolates exactly (alpha=eta=1, eps=0)."""
    d = rnd(3, T=11, dk=4, dv=3, W=2)
    d["alpha"][:] = 1.0
    d["eta"][:] = 1.0
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)      # k_tau, tau = -2..T-1
    vh = np.concatenate([d["v_prev"], d["v"]], axis=2)      # v_tau, tau = -1..T-1
    taus = np.arange(-2, d["k"].shape[2])
    kh[:, :, taus % 2 == 1] = 0.0
    d["k_prev"], d["k"] = kh[:, :, :2].copy(), kh[:, :, 2:].copy()
    T = d["k"].shape[2]
    q = np.zeros_like(d["q"])
    expect = np.zeros_like(d["v"])
    for t in range(T):
        # window pairs (k_{t-1}, v_t) and (k_{t-2}, v_{t-1})
        if (t - 1) % 2 == 0:
            q[:, :, t], expect[:, :, t] = kh[:, :, t - 1 + 2], vh[:, :, t + 1]
        else:
            q[:, :, t], expect[:, :, t] = kh[:, :, t - 2 + 2], vh[:, :, t]
    d["q"] = q
    o, _ = run("F3", d, W=2, eps=0.0)
    np.testing.assert_allclose(o, expect, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------- P3 -------
def _prefix_states(variant, d, W=1, eps=1e-6):
    """S_t for t = -1..T-1 via prefix runs of the oracle."""
    T = d["k"].shape[2]
    out = [d["S0"][0, 0]]
    for t in range(1, T + 1):
        dd = {key: (val[:, :, :t] if key in ("q", "k", "v", "alpha", "eta") else val)
              for key, val in d.items()}
        out.append(run(variant, dd, W=W, eps=eps)[1][0, 0])
    return out


@pytest.mark.parametrize("variant", ["F1", "F2", "F1A", "F2A"])
def test_gain_identity(variant):
    """alpha=1, eps=0: regression forms give S_t x_t = (1-eta) S_{t-1} x_t +
    eta y_t; inner-product forms give S_t x_t = S_{t-1} x_t + eta y_t."""
    d = rnd(4, B=1, H=1, T=8, dk=5, dv=3)
    d["alpha"][:] = 1.0
    Ss = _prefix_states(variant, d, eps=0.0)
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)[0, 0]
    for t in range(8):
        x, y, e = kh[t], d["v"][0, 0, t], d["eta"][0, 0, t]
        lhs = Ss[t + 1] @ x
        if variant in ("F1", "F2"):
            rhs = (1 - e) * (Ss[t] @ x) + e * y
        else:
            rhs = Ss[t] @ x + e * y
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def test_falcon2_sign_direction():
    """Falcon-2 per-column reading at eps=0: the write direction is
    eta * sign(x) / ||x||_1 (each column normalized by its own |x_j|)."""
    d = rnd(5, B=1, H=1, T=6, dk=7, dv=3)
    Ss = _prefix_states("F2", d, eps=0.0)
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)[0, 0]
    for t in range(6):
        x, y, e, a = kh[t], d["v"][0, 0, t], d["eta"][0, 0, t], d["alpha"][0, 0, t]
        Sp = a * Ss[t]
        want = Sp + np.outer(y - Sp @ x, e * np.sign(x) / np.abs(x).sum())
        np.testing.assert_allclose(Ss[t + 1], want, rtol=1e-11, atol=1e-12)


def test_falcon1_orthogonal_complement_untouched():
    """Falcon-1 writes only along x_t: S_t z = alpha_t S_{t-1} z for z orthogonal
    to x_t, and along x_t the residual is removed in the fraction
    eta ||x||^2 / (||x||^2 + eps)."""
    d = rnd(6, B=1, H=1, T=6, dk=5, dv=3)
    eps = 0.3
    Ss = _prefix_states("F1", d, eps=eps)
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)[0, 0]
    for t in range(6):
        x, y, e, a = kh[t], d["v"][0, 0, t], d["eta"][0, 0, t], d["alpha"][0, 0, t]
        z = np.random.default_rng(t).standard_normal(5)
        z -= (z @ x) / (x @ x) * x
        Sp = a * Ss[t]
        np.testing.assert_allclose(Ss[t + 1] @ z, Sp @ z, rtol=1e-11, atol=1e-12)
        frac = e * (x @ x) / (x @ x + eps)
        np.testing.assert_allclose(Ss[t + 1] @ x, Sp @ x + frac * (y - Sp @ x), rtol=1e-11,
                                   atol=1e-12)


@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_falcon3_orthogonal_window_closed_form(variant):
    """Keys along distinct basis vectors (mutually orthogonal windows): for
    Falcon-3 each pair's residual, taken at the decayed state S', is removed in
    the fraction ||x_w||^2 / (sum_w' ||x_w'||^2 + eps) * eta; for 3A the target
    is added with that weight.  Directions outside the window are only decayed."""
    W, T = 3, 7
    dk = T + W + 2
    d = rnd(7, B=1, H=1, T=T, dk=dk, dv=3, W=W)
    r = np.random.default_rng(70)
    scales = r.uniform(0.5, 2.0, T + W)
    kh = np.zeros((T + W, dk))
    for i in range(T + W):
        kh[i, i] = scales[i]
    d["k_prev"], d["k"] = kh[None, None, :W].copy(), kh[None, None, W:].copy()
    eps = 0.2
    Ss = _prefix_states(variant, d, W=W, eps=eps)
    vh = np.concatenate([d["v_prev"], d["v"]], axis=2)[0, 0]
    for t in range(T):
        Sp = d["alpha"][0, 0, t] * Ss[t]
        xs = [kh[t - w - 1 + W] for w in range(W)]
        ys = [vh[t - w + W - 1] for w in range(W)]
        tot = sum(x @ x for x in xs) + eps
        for x, y in zip(xs, ys):
            wgt = d["eta"][0, 0, t] * (x @ x) / tot
            if variant == "F3":
                want = Sp @ x + wgt * (y - Sp @ x)
            else:
                want = Sp @ x + wgt * y
            np.testing.assert_allclose(Ss[t + 1] @ x, want, rtol=1e-11, atol=1e-12)
        z = np.zeros(dk)
        z[-1] = 1.0
        np.testing.assert_allclose(Ss[t + 1] @ z, Sp @ z, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- P4 -------
@pytest.mark.parametrize("variant,W", [("F1", 1), ("F3", 1), ("F3", 3)])
def test_contraction_to_consistent_target(variant, W):
    """alpha=1, eps=0, eta in (0,2), y = S* x for every pair: ||S_t - S*||_F
    never increases (Kaczmarz / NLMS projection property)."""
    d = rnd(8, B=1, H=1, T=25, dk=6, dv=3, W=W)
    d["alpha"][:] = 1.0
    d["eta"][:] = np.random.default_rng(80).uniform(0.1, 1.9, d["eta"].shape)
    Sstar = np.random.default_rng(81).standard_normal((3, 6))
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)[0, 0]
    # y_tau = S* x_tau = S* k_{tau-1} for tau = -(W-1)..T-1
    ys = np.stack([Sstar @ kh[tau - 1 + W] for tau in range(-(W - 1), 25)])
    d["v"] = ys[W - 1:][None, None].copy()
    d["v_prev"] = ys[:W - 1][None, None].copy() if W > 1 else None
    Ss = _prefix_states(variant, d, W=W, eps=0.0)
    errs = [np.linalg.norm(S - Sstar) for S in Ss]
    assert all(b <= a * (1 + 1e-12) + 1e-13 for a, b in zip(errs, errs[1:]))
    assert errs[-1] < errs[0]


# ----------------------------------------------------------------- P5 -------
def test_falcon3_window1_is_falcon1():
    d = rnd(9, B=2, H=2, T=20)
    for a, b in [("F3", "F1"), ("F3A", "F1A")]:
        oa, Sa = run(a, d, W=1)
        ob, Sb = run(b, d, W=1)
        np.testing.assert_allclose(oa, ob, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(Sa, Sb, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("pair", [("F2", "F1"), ("F2A", "F1A")])
def test_falcon2_equals_falcon1_on_constant_magnitude_keys(pair):
    d = rnd(10, B=1, H=2, T=15, dk=8)
    r = np.random.default_rng(100)
    c = r.uniform(0.5, 2.0, d["k"].shape[:3] + (1,))
    d["k"] = c * np.sign(r.standard_normal(d["k"].shape))
    d["k_prev"] = 1.3 * np.sign(r.standard_normal(d["k_prev"].shape))
    oa, Sa = run(pair[0], d, eps=0.0)
    ob, Sb = run(pair[1], d, eps=0.0)
    np.testing.assert_allclose(oa, ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sa, Sb, rtol=1e-11, atol=1e-12)


def test_falcon1_is_kla_on_shifted_keys():
    """KLA (gated delta rule with beta = eta/(||k||^2+eps)), written in its
    product form S_t = alpha_t S_{t-1} (I - beta k k^T) + beta v k^T, run on the
    keys shifted by one step equals Falcon-1."""
    d = rnd(12, B=1, H=2, T=16, dk=5, dv=4)
    eps = 1e-3
    o, S = run("F1", d, eps=eps)
    for h in range(2):
        ks = np.concatenate([d["k_prev"][0, h], d["k"][0, h]])[:-1]   # k'_t = k_{t-1}
        St = d["S0"][0, h].copy()
        for t in range(16):
            kk = ks[t]
            beta = d["eta"][0, h, t] / (kk @ kk + eps)
            St = d["alpha"][0, h, t] * St @ (np.eye(5) - beta * np.outer(kk, kk)) \
                + beta * np.outer(d["v"][0, h, t], kk)
            np.testing.assert_allclose(o[0, h, t], St @ d["q"][0, h, t], rtol=1e-11,
                                       atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, rtol=1e-11, atol=1e-12)


def test_same_step_pairing_differs():
    """The prefix-aligned pair is not the same-step pair: feeding the unshifted
    keys through the KLA form gives a different result (guards against an
    oracle that forgot the shift)."""
    d = rnd(13, B=1, H=1, T=10, dk=4, dv=3)
    o, _ = run("F1", d)
    St = d["S0"][0, 0].copy()
    o2 = []
    for t in range(10):
        kk = d["k"][0, 0, t]
        beta = d["eta"][0, 0, t] / (kk @ kk + 1e-6)
        St = d["alpha"][0, 0, t] * St @ (np.eye(4) - beta * np.outer(kk, kk)) \
            + beta * np.outer(d["v"][0, 0, t], kk)
        o2.append(St @ d["q"][0, 0, t])
    assert np.abs(np.array(o2) - o[0, 0]).max() > 1e-3


# ----------------------------------------------------------------- P6 -------
@pytest.mark.parametrize("variant", ["F1A", "F2A"])
def test_inner_product_family_is_decayed_linear_attention(variant):
    d = rnd(14, B=1, H=2, T=18, dk=5, dv=4)
    eps = 1e-2
    o, S = run(variant, d, eps=eps)
    for h in range(2):
        xs = np.concatenate([d["k_prev"][0, h], d["k"][0, h]])[:-1]
        e = d["eta"][0, h]
        if variant == "F1A":
            U = e[:, None] * xs / ((xs * xs).sum(1) + eps)[:, None]
        else:
            l1 = np.abs(xs).sum(1, keepdims=True)
            U = e[:, None] * xs / (np.abs(xs) * l1 + eps)
        g = np.cumsum(np.log(d["alpha"][0, h]))
        Tn = len(g)
        for t in range(Tn):
            acc = np.exp(g[t]) * d["S0"][0, h] @ d["q"][0, h, t]
            for s in range(t + 1):
                acc = acc + np.exp(g[t] - g[s]) * (U[s] @ d["q"][0, h, t]) * d["v"][0, h, s]
            np.testing.assert_allclose(o[0, h, t], acc, rtol=1e-11, atol=1e-12)
        Sc = np.exp(g[-1]) * d["S0"][0, h] + sum(
            np.exp(g[-1] - g[s]) * np.outer(d["v"][0, h, s], U[s]) for s in range(Tn))
        np.testing.assert_allclose(S[0, h], Sc, rtol=1e-11, atol=1e-12)


def test_falcon3a_banded_weights():
    """Falcon-3A: o_t = gamma_t S0 q_t + sum_tau c_{t,tau} (x_tau . q_t) y_tau with
    c_{t,tau} = sum_{s=tau}^{min(tau+W-1,t)} D(t,s) b_s (each pair rehearsed in W
    consecutive steps, then only decayed)."""
    W = 3
    d = rnd(15, B=1, H=1, T=14, dk=5, dv=3, W=W)
    eps = 1e-2
    o, _ = run("F3A", d, W=W, eps=eps)
    kh = np.concatenate([d["k_prev"][0, 0], d["k"][0, 0]])    # k_tau at tau + W
    vh = np.concatenate([d["v_prev"][0, 0], d["v"][0, 0]])    # v_tau at tau + W - 1
    x = lambda tau: kh[tau - 1 + W]  # noqa: E731
    y = lambda tau: vh[tau + W - 1]  # noqa: E731
    g = np.cumsum(np.log(d["alpha"][0, 0]))
    e = d["eta"][0, 0]
    b = np.array([e[s] / (sum(x(s - w) @ x(s - w) for w in range(W)) + eps) for s in range(14)])
    for t in range(14):
        acc = np.exp(g[t]) * d["S0"][0, 0] @ d["q"][0, 0, t]
        for tau in range(-(W - 1), t + 1):
            c = sum(np.exp(g[t] - g[s]) * b[s] for s in range(max(tau, 0), min(tau + W - 1, t) + 1))
            acc = acc + c * (x(tau) @ d["q"][0, 0, t]) * y(tau)
        np.testing.assert_allclose(o[0, 0, t], acc, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------- P7 -------
@pytest.mark.parametrize("variant", ALL)
def test_recurrent_masked_chunk_agree(variant):
    for W in ([1, 2, 4] if variant in ("F3", "F3A") else [1]):
        d = rnd(16 + W, B=1, H=2, T=24, dk=6, dv=5, W=W)
        o, S = run(variant, d, W=W)
        kw = dict(window=W, eps=1e-6, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"])
        om, Sm = forms.masked(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], **kw)
        np.testing.assert_allclose(om, o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(Sm, S, rtol=1e-10, atol=1e-12)
        for C in (1, 2, 4, 5, 8, 16):
            oc, Sc = forms.chunked(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                   chunk=C, **kw)
            np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- P8 -------
@pytest.mark.parametrize("variant", ALL)
def test_decay_only(variant):
    W = 2 if variant in ("F3", "F3A") else 1
    d = rnd(20, B=1, H=2, T=10, W=W)
    d["eta"][:] = 0.0
    o, S = run(variant, d, W=W)
    g = np.exp(np.cumsum(np.log(d["alpha"]), axis=-1))
    want_o = g[..., None] * np.einsum("bhvk,bhtk->bhtv", d["S0"], d["q"])
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, g[..., -1, None, None] * d["S0"], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- P9 -------
@pytest.mark.parametrize("variant", ALL)
def test_continuation(variant):
    W = 3 if variant in ("F3", "F3A") else 1
    d = rnd(21, B=2, H=1, T=17, W=W)
    o, S = run(variant, d, W=W)
    T1 = 7
    d1 = {key: (val[:, :, :T1] if key in ("q", "k", "v", "alpha", "eta") else val)
          for key, val in d.items()}
    o1, S1 = run(variant, d1, W=W)
    kh = np.concatenate([d["k_prev"], d["k"]], axis=2)
    d2 = {key: (val[:, :, T1:] if key in ("q", "k", "v", "alpha", "eta") else val)
          for key, val in d.items()}
    d2["S0"] = S1
    d2["k_prev"] = kh[:, :, T1:T1 + W].copy()         # k_{T1-W} .. k_{T1-1}
    if W > 1:
        d2["v_prev"] = d["v"][:, :, T1 - (W - 1):T1].copy()
    o2, S2 = run(variant, d2, W=W)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P10 -------
@pytest.mark.parametrize("variant", ALL)
def test_linearity_in_values_and_state(variant):
    W = 2 if variant in ("F3", "F3A") else 1
    d1 = rnd(22, W=W)
    d2 = rnd(23, W=W)
    for key in ("q", "k", "alpha", "eta", "k_prev"):
        d2[key] = d1[key]
    a, b = 0.7, -1.9
    dm = dict(d1)
    dm["v"] = a * d1["v"] + b * d2["v"]
    dm["S0"] = a * d1["S0"] + b * d2["S0"]
    if W > 1:
        dm["v_prev"] = a * d1["v_prev"] + b * d2["v_prev"]
    o1, S1 = run(variant, d1, W=W)
    o2, S2 = run(variant, d2, W=W)
    om, Sm = run(variant, dm, W=W)
    np.testing.assert_allclose(om, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sm, a * S1 + b * S2, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P11 -------
@pytest.mark.parametrize("variant,alpha", [("F1", 1 - 1e-4), ("F1", 0.5), ("F2", 1 - 1e-4),
                                           ("F3", 0.5), ("F1A", 1 - 1e-4), ("F3A", 0.9)])
def test_renormalization_stress(variant, alpha):
    """Long sequences with near-1 or strong decays: the chunk form (log-space,
    re-referenced at every chunk start) stays finite and equals the recurrence."""
    W = 2 if variant in ("F3", "F3A") else 1
    T = 8192 if alpha > 0.99 else 2048
    d = rnd(24, B=1, H=1, T=T, dk=4, dv=3, W=W)
    d["alpha"][:] = alpha
    o, S = run(variant, d, W=W)
    oc, Sc = forms.chunked(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], chunk=64,
                           window=W, eps=1e-6, S0=d["S0"], k_prev=d["k_prev"],
                           v_prev=d["v_prev"])
    assert np.isfinite(o).all() and np.isfinite(oc).all()
    scale = np.abs(o).max()
    assert np.abs(oc - o).max() <= 1e-9 * scale
    assert np.abs(Sc - S).max() <= 1e-9 * max(1.0, np.abs(S).max())


def test_renormalization_sigmoid_tail_decays():
    d = rnd(25, B=1, H=1, T=1024, dk=4, dv=3)
    d["alpha"] = 1 / (1 + np.exp(-np.random.default_rng(250).uniform(-3, 9, d["alpha"].shape)))
    o, S = run("F1", d)
    oc, Sc = forms.chunked("F1", d["q"], d["k"], d["v"], d["alpha"], d["eta"], chunk=64,
                           eps=1e-6, S0=d["S0"], k_prev=d["k_prev"])
    assert np.abs(oc - o).max() <= 1e-10 * np.abs(o).max()


# ------------------------------------------------------------ decode --------
@pytest.mark.parametrize("variant", ["F1", "F2", "F1A", "F2A"])
def test_decode_step_is_one_recurrent_step(variant):
    r = np.random.default_rng(26)
    N, H, dk, dv, steps = 3, 2, 6, 5, 9
    S = r.standard_normal((N, H, dv, dk)) * 0.1
    kc = r.standard_normal((N, H, dk))
    q, k = r.standard_normal((steps, N, H, dk)), r.standard_normal((steps, N, H, dk))
    v = r.standard_normal((steps, N, H, dv))
    al, et = r.uniform(0.5, 1, (steps, N, H)), r.uniform(0, 1, (steps, N, H))
    S_run, kc_run, outs = S, kc, []
    for s in range(steps):
        o, S_run, kc_run = oracle.decode_step(variant, S_run, kc_run, q[s], k[s], v[s], al[s],
                                              et[s])
        outs.append(o)
        np.testing.assert_array_equal(kc_run, k[s])
    tr = lambda a: np.moveaxis(a, 0, 2)  # noqa: E731
    o_rec, S_rec = oracle.recurrent(variant, tr(q), tr(k), tr(v), tr(al), tr(et), S0=S,
                                    k_prev=kc[:, :, None, :])
    np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["F3", "F3A"])
@pytest.mark.parametrize("W", [1, 2, 4])
def test_decode_step_window_is_one_recurrent_step(variant, W):
    """Windowed decode (caches newest first) over T steps equals the recurrent
    form with the same halo (k_prev / v_prev oldest first); the caches end as
    the last W keys and W-1 values."""
    r = np.random.default_rng(31 + W)
    N, H, dk, dv, steps = 2, 2, 5, 4, 11
    S = r.standard_normal((N, H, dv, dk)) * 0.1
    k_prev = r.standard_normal((N, H, W, dk))
    v_prev = r.standard_normal((N, H, W - 1, dv))
    kc = k_prev[:, :, ::-1, :].copy()          # kc[w] = k_{-1-w}
    vc = v_prev[:, :, ::-1, :].copy()          # vc[w-1] = v_{-w}
    q, k = r.standard_normal((steps, N, H, dk)), r.standard_normal((steps, N, H, dk))
    v = r.standard_normal((steps, N, H, dv))
    al, et = r.uniform(0.5, 1, (steps, N, H)), r.uniform(0, 1, (steps, N, H))
    S_run, kc_run, vc_run, outs = S, kc, vc, []
    for s in range(steps):
        o, S_run, kc_run, vc_run = oracle.decode_step_window(variant, S_run, kc_run, vc_run, q[s],
                                                             k[s], v[s], al[s], et[s])
        outs.append(o)
    tr = lambda a: np.moveaxis(a, 0, 2)  # noqa: E731
    o_rec, S_rec = oracle.recurrent(variant, tr(q), tr(k), tr(v), tr(al), tr(et), window=W,
                                    S0=S, k_prev=k_prev, v_prev=v_prev if W > 1 else None)
    np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)
    for w in range(W):
        np.testing.assert_array_equal(kc_run[:, :, w], k[steps - 1 - w])
    for w in range(W - 1):
        np.testing.assert_array_equal(vc_run[:, :, w], v[steps - 1 - w])


@pytest.mark.parametrize("variant,base", [("F3", "F1"), ("F3A", "F1A")])
def test_decode_step_window_of_one_is_the_scalar_rule(variant, base):
    """Reduction: a window of one pair is Falcon-1 (Falcon-1A) exactly."""
    r = np.random.default_rng(37)
    N, H, dk, dv = 3, 2, 6, 5
    S = r.standard_normal((N, H, dv, dk)) * 0.2
    kc = r.standard_normal((N, H, dk))
    q, k, v = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk)), r.standard_normal((N, H, dv))
    al, et = r.uniform(0.5, 1, (N, H)), r.uniform(0, 1, (N, H))
    o1, S1, _ = oracle.decode_step(base, S, kc, q, k, v, al, et)
    o3, S3, _, _ = oracle.decode_step_window(variant, S, kc[:, :, None, :], None, q, k, v, al, et)
    np.testing.assert_allclose(o3, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S3, S1, rtol=1e-13, atol=1e-14)


def test_decode_step_window_interpolates_its_window():
    """P2 on the decode path: alpha = 1, eta = 1, eps = 0 and a window whose
    only nonzero key is x_{t-1} (slot 1) makes S x_{t-1} = y_{t-1} exactly."""
    r = np.random.default_rng(41)
    N, H, dk, dv, W = 1, 1, 4, 3, 3
    S = r.standard_normal((N, H, dv, dk))
    kc = np.zeros((N, H, W, dk))
    kc[:, :, 1] = r.standard_normal(dk)
    vc = r.standard_normal((N, H, W - 1, dv))
    q, k, v = r.standard_normal((N, H, dk)), r.standard_normal((N, H, dk)), r.standard_normal((N, H, dv))
    one = np.ones((N, H))
    _, S_new, _, _ = oracle.decode_step_window("F3", S, kc, vc, q, k, v, one, one, eps=0.0)
    np.testing.assert_allclose(S_new[0, 0] @ kc[0, 0, 1], vc[0, 0, 0], rtol=1e-12, atol=1e-12)


def test_oracle_rejects_bad_arguments():
    d = rnd(27)
    with pytest.raises(ValueError):
        oracle.recurrent(7, d["q"], d["k"], d["v"], d["alpha"], d["eta"])
    with pytest.raises(ValueError):
        oracle.recurrent("F1", d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=2)


# ------------------------------------------------- same-step alignment ------
# The pages contrast the prefix-aligned pair (k_{t-1}, v_t) with the same-step
# pair (k_t, v_t) of the KLA / gated-delta-rule recurrences.  align="same"
# gives the latter; these pin it.
def run_same(variant, d, W=1, eps=1e-6):
    return run(variant, d, W=W, eps=eps, align="same")


def test_same_step_falcon1_is_kla_product_form():
    """Falcon-1 with same-step pairs is KLA exactly: the gated delta rule in its
    product form S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    with beta_t = eta_t / (||k_t||^2 + eps), on the unshifted keys."""
    d = rnd(51, B=1, H=2, T=14, dk=5, dv=4)
    eps = 1e-3
    o, S = run_same("F1", d, eps=eps)
    for h in range(2):
        St = d["S0"][0, h].copy()
        for t in range(14):
            kk = d["k"][0, h, t]
            beta = d["eta"][0, h, t] / (kk @ kk + eps)
            St = d["alpha"][0, h, t] * St @ (np.eye(5) - beta * np.outer(kk, kk)) \
                + beta * np.outer(d["v"][0, h, t], kk)
            np.testing.assert_allclose(o[0, h, t], St @ d["q"][0, h, t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S[0, h], St, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("variant", ALL)
def test_same_step_is_prefix_alignment_on_keys_moved_one_step(variant):
    """Same-step pairs on keys k equal prefix-aligned pairs on k' with
    k'_tau = k_{tau+1}: the halo moves with them (k'_{-W..-1} = k_{-W+1..0}),
    and k'_{T-1} is never read."""
    for W in ([1, 2, 4] if variant in ("F3", "F3A") else [1]):
        d = rnd(52 + W, B=1, H=2, T=13, dk=5, dv=4, W=W)
        o, S = run_same(variant, d, W=W)
        kh = np.concatenate([d["k_prev"], d["k"]], axis=2)          # k_tau, tau = -W..T-1
        d2 = dict(d)
        d2["k_prev"] = kh[:, :, 1:W + 1].copy()                      # k_{-W+1} .. k_0
        d2["k"] = np.concatenate([kh[:, :, W + 1:], np.full_like(kh[:, :, :1], 7.0)], axis=2)
        o2, S2 = run(variant, d2, W=W)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["F1", "F2"])
def test_same_step_interpolation(variant):
    """alpha = eta = 1, eps = 0: the same-step write makes S_t k_t = v_t, so a
    read with q_t = k_t returns v_t."""
    d = rnd(57, T=9, dk=6, dv=3)
    d["alpha"][:] = 1.0
    d["eta"][:] = 1.0
    d["q"] = d["k"].copy()
    o, _ = run_same(variant, d, eps=0.0)
    np.testing.assert_allclose(o, d["v"], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("variant", ALL)
def test_same_step_exact_rational_matches_fp64(variant):
    r = np.random.default_rng(58)
    for W in wins(variant):
        T, dk, dv = 5, 3, 2
        ri = lambda *s: r.integers(-4, 5, s)  # noqa: E731
        q, k, v = ri(T, dk), ri(T, dk), ri(T, dv)
        kp, vp, S0 = ri(W, dk), ri(W - 1, dv), ri(dv, dk)
        al = [Fr(int(a), 8) for a in r.integers(1, 9, T)]
        et = [Fr(int(a), 4) for a in r.integers(0, 5, T)]
        eps = Fr(1, 16)
        F = lambda a: [[Fr(int(x)) for x in row] for row in a]  # noqa: E731
        oe, Se = exact.recurrent_seq(variant, F(q), F(k), F(v), al, et, window=W, eps=eps,
                                     S0=F(S0), k_prev=F(kp), v_prev=F(vp) if W > 1 else None,
                                     lag=0)
        o, S = oracle.recurrent(variant, q[None, None], k[None, None], v[None, None],
                                np.array([float(a) for a in al])[None, None],
                                np.array([float(a) for a in et])[None, None], window=W,
                                eps=float(eps), S0=S0[None, None], k_prev=kp[None, None],
                                v_prev=vp[None, None] if W > 1 else None, align="same")
        oe = np.array([[float(x) for x in row] for row in oe])
        Se = np.array([[float(x) for x in row] for row in Se])
        assert np.abs(o[0, 0] - oe).max() <= 1e-13 * max(1.0, np.abs(oe).max())
        assert np.abs(S[0, 0] - Se).max() <= 1e-13 * max(1.0, np.abs(Se).max())


@pytest.mark.parametrize("variant", ALL)
def test_same_step_recurrent_masked_chunk_agree(variant):
    for W in ([1, 3] if variant in ("F3", "F3A") else [1]):
        d = rnd(60 + W, B=1, H=2, T=20, dk=5, dv=4, W=W)
        o, S = run_same(variant, d, W=W)
        kw = dict(window=W, eps=1e-6, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"], lag=0)
        for C in (1, 3, 8, 20):
            oc, Sc = forms.chunked(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                   chunk=C, **kw)
            np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("variant", ["F1", "F2", "F1A", "F2A"])
def test_same_step_decode_is_one_recurrent_step(variant):
    r = np.random.default_rng(63)
    N, H, dk, dv, steps = 2, 2, 5, 4, 8
    S = r.standard_normal((N, H, dv, dk)) * 0.1
    kc = r.standard_normal((N, H, dk))
    q, k = r.standard_normal((steps, N, H, dk)), r.standard_normal((steps, N, H, dk))
    v = r.standard_normal((steps, N, H, dv))
    al, et = r.uniform(0.5, 1, (steps, N, H)), r.uniform(0, 1, (steps, N, H))
    S_run, kc_run, outs = S, kc, []
    for s in range(steps):
        o, S_run, kc_run = oracle.decode_step(variant, S_run, kc_run, q[s], k[s], v[s], al[s],
                                              et[s], align="same")
        outs.append(o)
    tr = lambda a: np.moveaxis(a, 0, 2)  # noqa: E731
    o_rec, S_rec = oracle.recurrent(variant, tr(q), tr(k), tr(v), tr(al), tr(et), S0=S,
                                    k_prev=kc[:, :, None, :], align="same")
    np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(kc_run, k[steps - 1])


@pytest.mark.parametrize("variant", ["F3", "F3A"])
@pytest.mark.parametrize("W", [1, 2, 4])
def test_same_step_decode_window_is_one_recurrent_step(variant, W):
    r = np.random.default_rng(65 + W)
    N, H, dk, dv, steps = 2, 2, 5, 4, 9
    S = r.standard_normal((N, H, dv, dk)) * 0.1
    k_prev = r.standard_normal((N, H, W, dk))
    v_prev = r.standard_normal((N, H, W - 1, dv))
    kc, vc = k_prev[:, :, ::-1, :].copy(), v_prev[:, :, ::-1, :].copy()
    q, k = r.standard_normal((steps, N, H, dk)), r.standard_normal((steps, N, H, dk))
    v = r.standard_normal((steps, N, H, dv))
    al, et = r.uniform(0.5, 1, (steps, N, H)), r.uniform(0, 1, (steps, N, H))
    S_run, kc_run, vc_run, outs = S, kc, vc, []
    for s in range(steps):
        o, S_run, kc_run, vc_run = oracle.decode_step_window(
            variant, S_run, kc_run, vc_run, q[s], k[s], v[s], al[s], et[s], align="same")
        outs.append(o)
    tr = lambda a: np.moveaxis(a, 0, 2)  # noqa: E731
    o_rec, S_rec = oracle.recurrent(variant, tr(q), tr(k), tr(v), tr(al), tr(et), window=W,
                                    S0=S, k_prev=k_prev, v_prev=v_prev if W > 1 else None,
                                    align="same")
    np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------- feature maps phi ------
# phi is left open by the pages; the oracle offers phi on every key and query.
def np_phi(name, x):
    x = np.asarray(x, np.float64)
    if name == "l2":
        n = np.sqrt((x * x).sum(-1, keepdims=True))
        return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)
    if name == "silu":
        return x * (1.0 / (1.0 + np.exp(-x)))
    return x


@pytest.mark.parametrize("align", ["prefix", "same"])
@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("variant", ALL)
def test_phi_is_the_identity_form_on_mapped_inputs(variant, phi, align):
    """The feature-map option equals the identity form run on keys, halo keys
    and queries mapped by numpy's own L2 normalization / SiLU (values and
    targets untouched), with a zero key in the mix."""
    for W in ([1, 3] if variant in ("F3", "F3A") else [1]):
        d = rnd(70 + W, B=1, H=2, T=11, dk=5, dv=4, W=W)
        d["k"][0, 1, 4] = 0.0
        o, S = run(variant, d, W=W, align=align, phi=phi)
        d2 = dict(d, q=np_phi(phi, d["q"]), k=np_phi(phi, d["k"]), k_prev=np_phi(phi, d["k_prev"]))
        o2, S2 = run(variant, d2, W=W, align=align)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-13)


def test_phi_l2_falcon1_gain():
    """L2-normalized keys have unit norm: Falcon-1 at alpha = 1, eps = 0 then
    writes exactly eta of the residual along x (S_t x = (1-eta) S' x + eta y)."""
    d = rnd(74, B=1, H=1, T=6, dk=4, dv=3)
    d["alpha"][:] = 1.0
    eta = d["eta"][0, 0]
    St = [d["S0"][0, 0]]
    for t in range(6):
        dt_ = {kk: (vv[:, :, :t + 1] if (vv is not None and vv.ndim == 4 and kk in ("q", "k", "v"))
                    else vv) for kk, vv in d.items()}
        dt_["alpha"], dt_["eta"] = d["alpha"][:, :, :t + 1], d["eta"][:, :, :t + 1]
        _, S = run("F1", dt_, eps=0.0, phi="l2")
        St.append(S[0, 0])
    kh = np.concatenate([d["k_prev"][0, 0], d["k"][0, 0]])
    for t in range(6):
        x = np_phi("l2", kh[t])                        # x_t = phi(k_{t-1})
        lhs = St[t + 1] @ x
        rhs = (1 - eta[t]) * (St[t] @ x) + eta[t] * d["v"][0, 0, t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("phi", ["l2", "silu"])
def test_phi_decode_steps_are_recurrent_steps(phi):
    r = np.random.default_rng(77)
    N, H, dk, dv, steps, W = 2, 2, 5, 4, 7, 3
    S = r.standard_normal((N, H, dv, dk)) * 0.1
    k_prev, v_prev = r.standard_normal((N, H, W, dk)), r.standard_normal((N, H, W - 1, dv))
    q, k = r.standard_normal((steps, N, H, dk)), r.standard_normal((steps, N, H, dk))
    v = r.standard_normal((steps, N, H, dv))
    al, et = r.uniform(0.5, 1, (steps, N, H)), r.uniform(0, 1, (steps, N, H))
    tr = lambda a: np.moveaxis(a, 0, 2)  # noqa: E731
    for align in ("prefix", "same"):
        # windowed rule (caches hold raw keys, newest first)
        S_run, kc, vc, outs = S, k_prev[:, :, ::-1].copy(), v_prev[:, :, ::-1].copy(), []
        for s in range(steps):
            o, S_run, kc, vc = oracle.decode_step_window("F3", S_run, kc, vc, q[s], k[s], v[s],
                                                         al[s], et[s], align=align, phi=phi)
            outs.append(o)
        o_rec, S_rec = oracle.recurrent("F3", tr(q), tr(k), tr(v), tr(al), tr(et), window=W, S0=S,
                                        k_prev=k_prev, v_prev=v_prev, align=align, phi=phi)
        np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)
        # single-key rule
        S_run, kc1, outs = S, k_prev[:, :, -1].copy(), []
        for s in range(steps):
            o, S_run, kc1 = oracle.decode_step("F2", S_run, kc1, q[s], k[s], v[s], al[s], et[s],
                                               align=align, phi=phi)
            outs.append(o)
        o_rec, S_rec = oracle.recurrent("F2", tr(q), tr(k), tr(v), tr(al), tr(et), S0=S,
                                        k_prev=k_prev[:, :, -1:], align=align, phi=phi)
        np.testing.assert_allclose(tr(np.array(outs)), o_rec, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S_run, S_rec, rtol=1e-12, atol=1e-13)
