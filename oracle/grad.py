"""fp64 gradients of the Falcon recurrence: the oracle of the backward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the GPU package.

The forward here is the same step-by-step recurrence as falcon_oracle.c,
written a second time with plain torch CPU ops in float64 so that torch's
autograd can differentiate it exactly ("Fast Weight Attention for Continual
Learning", authors' abstract: a fixed-size fast-weight state, decayed by a
positive gate, corrected with a normalized first-order step towards the
prefix-aligned example (phi(k_{t-1}), v_t), read after the write; step size
eta / (||x||^2 + eps) and decay-then-residual order from the KLA abstract on
the same listing; the per-column and window rules as read in falcon_oracle.c).

What is differentiated is the vector-Jacobian product of the forward map
(q, k, v, alpha, eta, S0, k_prev, v_prev) -> (o, S_T) with the cotangents
(d_o, dS_T):  L = sum(o * d_o) + sum(S_T * dS_T), and gradients of L with
respect to every input.  The forward is pinned against the C oracle, and the
gradients against central finite differences of the C oracle's forward (the
tests), so neither the rewritten forward nor autograd is trusted on its own.

Non-smooth points take the derivative torch gives: |x| has slope 0 at 0
(per-column rule), and the L2 feature map of a zero key is the constant 0.
"""
from __future__ import annotations

import numpy as np
import torch

VARIANTS = {"F1": 1, "F2": 2, "F3": 3, "F1A": 11, "F2A": 12, "F3A": 13}
LAG = {"prefix": 1, "same": 0}


def _phi(x, phi):
    if phi == "identity":
        return x
    if phi == "l2":
        n2 = (x * x).sum(-1, keepdim=True)
        safe = torch.where(n2 > 0, n2, torch.ones_like(n2))
        return x * torch.where(n2 > 0, safe.rsqrt(), torch.zeros_like(n2))
    if phi == "silu":
        return x / (1.0 + torch.exp(-x))
    raise ValueError(phi)


def forward(variant, q, k, v, alpha, eta, *, window=1, eps=1e-6, S0=None, k_prev=None,
            v_prev=None, align="prefix", phi="identity"):
    """The recurrence on float64 torch tensors (batched over the leading
    [B, H] axes, one loop over time).  Returns (o [B,H,T,dv], S_T [B,H,dv,dk])."""
    var = VARIANTS.get(variant, variant)
    lag = LAG[align]
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    W = window if var in (3, 13) else 1
    delta = var in (1, 2, 3)
    zk = torch.zeros(B, H, dk, dtype=k.dtype)
    zv = torch.zeros(B, H, dv, dtype=v.dtype)
    kphi = _phi(k, phi)
    qphi = _phi(q, phi)
    kpphi = _phi(k_prev, phi) if k_prev is not None else None

    def key(tau):  # k_tau, from the halo (oldest first) before the sequence
        if tau >= 0:
            return kphi[:, :, tau]
        if kpphi is not None and tau >= -W:
            return kpphi[:, :, W + tau]
        return zk

    def val(tau):
        if tau >= 0:
            return v[:, :, tau]
        if v_prev is not None and W > 1 and tau >= -(W - 1):
            return v_prev[:, :, W - 1 + tau]
        return zv

    S = S0.clone() if S0 is not None else torch.zeros(B, H, dv, dk, dtype=k.dtype)
    outs = []
    for t in range(T):
        a = alpha[:, :, t, None, None]
        e = eta[:, :, t, None]
        Sd = a * S                                   # decay first
        if var in (1, 11, 2, 12):
            x = key(t - lag)
            y = v[:, :, t]
            if var in (1, 11):
                u = e * x / ((x * x).sum(-1, keepdim=True) + eps)
            else:
                l1 = x.abs().sum(-1, keepdim=True)
                u = e * x / (x.abs() * l1 + eps)
            if delta:
                r = y - torch.einsum("bhvk,bhk->bhv", Sd, x)   # residual at the decayed state
            else:
                r = y
            S = Sd + r[..., :, None] * u[..., None, :]
        else:
            xs = [key(t - w - lag) for w in range(W)]
            ys = [val(t - w) for w in range(W)]
            nrm = sum((x * x).sum(-1, keepdim=True) for x in xs)
            b = e / (nrm + eps)
            S = Sd
            for x, y in zip(xs, ys):
                r = y - torch.einsum("bhvk,bhk->bhv", Sd, x) if delta else y
                S = S + (b * r)[..., :, None] * x[..., None, :]
        outs.append(torch.einsum("bhvk,bhk->bhv", S, qphi[:, :, t]))   # read after the write
    o = torch.stack(outs, 2) if T else torch.zeros(B, H, 0, dv, dtype=k.dtype)
    return o, S


def gradients(variant, q, k, v, alpha, eta, d_o, dS_T=None, *, window=1, eps=1e-6, S0=None,
              k_prev=None, v_prev=None, align="prefix", phi="identity"):
    """Gradients of sum(o * d_o) + sum(S_T * dS_T) in float64.

    Inputs are array-likes (numpy or torch, any float dtype: they are widened
    to float64 as given).  Returns a dict with keys q, k, v, alpha, eta and,
    for the optional inputs that were given, S0, k_prev, v_prev; plus o and
    S_T, the forward results."""
    def t64(a, grad=True):
        if a is None:
            return None
        x = torch.as_tensor(np.asarray(a, dtype=np.float64) if not torch.is_tensor(a)
                            else a.detach().to(torch.float64).cpu()).clone()
        x.requires_grad_(grad)
        return x

    names = ["q", "k", "v", "alpha", "eta", "S0", "k_prev", "v_prev"]
    vals = [q, k, v, alpha, eta, S0, k_prev, v_prev]
    ins = {n: t64(a) for n, a in zip(names, vals)}
    W = window if VARIANTS.get(variant, variant) in (3, 13) else 1
    if W == 1:
        ins["v_prev"] = None
    with torch.enable_grad():
        o, S = forward(variant, ins["q"], ins["k"], ins["v"], ins["alpha"], ins["eta"],
                       window=window, eps=eps, S0=ins["S0"], k_prev=ins["k_prev"],
                       v_prev=ins["v_prev"], align=align, phi=phi)
        L = (o * t64(d_o, False)).sum()
        if dS_T is not None:
            L = L + (S * t64(dS_T, False)).sum()
        leaves = [n for n in names if ins[n] is not None]
        gs = torch.autograd.grad(L, [ins[n] for n in leaves], allow_unused=True)
    out = {}
    for n, g in zip(leaves, gs):
        out[n] = (torch.zeros_like(ins[n]) if g is None else g).detach().numpy()
    out["o"] = o.detach().numpy()
    out["S_T"] = S.detach().numpy()
    return out
