"""Seeded synthetic inputs for the Falcon recurrence (no method arithmetic here).

This module only draws random numbers and rounds them to the storage type;
the GPU path and the CPU oracle both consume exactly the arrays it returns
(the oracle after widening the stored bits to float64), so the only
difference left between them is arithmetic.

Recipe (one SeedSequence per workload, children spawned in the fixed order
q, k, v, alpha-logit, eta-logit, key-scale, span, S0, k_prev, v_prev):

* q, k, v ~ N(0, 1) drawn in float32; bf16 storage is the round-to-nearest-
  even of the float32 bits.
* alpha = sigmoid(N(mu, sd)) per token and head (float32), eta =
  sigmoid(N(0, 1)) (float32).
* optional: keys scaled per (batch, token) by LogNormal(0, 1), shared by all
  heads; a planted span of near-1 decays, alpha = sigmoid(N(9, 0.5)), of a
  given length at a seeded offset in every (batch, head).
* optional: S0 ~ N(0, sd^2) float32; halo keys / values ~ N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sigmoid32(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float32)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-z))).astype(np.float32)


@dataclass
class ChunkInputs:
    """Inputs of one chunk-forward call, in storage form.

    q, k [B,H,T,dk], v [B,H,T,dv]: float32, or uint16 holding bf16 bits.
    alpha, eta [B,H,T] float32.  S0 [B,H,dv,dk] float32 or None.
    k_prev [B,H,W,dk], v_prev [B,H,W-1,dv] in the storage type, or None.
    """
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    eta: np.ndarray
    window: int = 1
    S0: np.ndarray | None = None
    k_prev: np.ndarray | None = None
    v_prev: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    def widen(self, a):
        """Storage array -> float64 (exact)."""
        if a is None:
            return None
        if self.dtype == "bf16" and a.dtype == np.uint16:
            return bits_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)

    def f64(self, sl=None):
        """Float64 copies for the oracle, optionally restricted to a
        (batch, head) index tuple `sl`."""
        def pick(a):
            if a is None:
                return None
            return a if sl is None else a[sl]
        return dict(q=self.widen(pick(self.q)), k=self.widen(pick(self.k)),
                    v=self.widen(pick(self.v)), alpha=np.asarray(pick(self.alpha), np.float64),
                    eta=np.asarray(pick(self.eta), np.float64),
                    S0=None if self.S0 is None else np.asarray(pick(self.S0), np.float64),
                    k_prev=self.widen(pick(self.k_prev)), v_prev=self.widen(pick(self.v_prev)))

    def to_torch(self, device):
        import torch

        def t(a):
            if a is None:
                return None
            x = torch.from_numpy(np.ascontiguousarray(a))
            if a.dtype == np.uint16:
                x = x.view(torch.bfloat16)
            return x.to(device)
        return dict(q=t(self.q), k=t(self.k), v=t(self.v), alpha=t(self.alpha), eta=t(self.eta),
                    S0=t(self.S0), k_prev=t(self.k_prev), v_prev=t(self.v_prev))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def make_chunk_inputs(B, H, T, dk, dv, *, dtype="bf16", seed=0, alpha_mu=3.0, alpha_sd=1.0,
                      eta_mu=0.0, eta_sd=1.0, key_lognormal=False, span=0, window=1,
                      S0_sd=0.0, halo=False) -> ChunkInputs:
    ss = np.random.SeedSequence(seed)
    cq, ck, cv, ca, ce, cs, csp, cS, ckp, cvp = ss.spawn(10)
    g = lambda c: np.random.Generator(np.random.PCG64(c))  # noqa: E731
    q = g(cq).standard_normal((B, H, T, dk), dtype=np.float32)
    k = g(ck).standard_normal((B, H, T, dk), dtype=np.float32)
    v = g(cv).standard_normal((B, H, T, dv), dtype=np.float32)
    alpha = sigmoid32(g(ca).normal(alpha_mu, alpha_sd, (B, H, T)).astype(np.float32))
    eta = sigmoid32(g(ce).normal(eta_mu, eta_sd, (B, H, T)).astype(np.float32))
    meta = {}
    if key_lognormal:
        s = np.exp(g(cs).standard_normal((B, 1, T, 1), dtype=np.float32)).astype(np.float32)
        k = (k * s).astype(np.float32)
    if span and span > 0:
        gs = g(csp)
        L = min(span, T)
        offs = gs.integers(0, T - L + 1, size=(B, H))
        hi = sigmoid32(gs.normal(9.0, 0.5, (B, H, L)).astype(np.float32))
        for b in range(B):
            for h in range(H):
                alpha[b, h, offs[b, h]:offs[b, h] + L] = hi[b, h]
        meta["span_offsets"] = offs
    S0 = None
    if S0_sd > 0:
        S0 = (g(cS).standard_normal((B, H, dv, dk), dtype=np.float32) * np.float32(S0_sd))
        S0 = S0.astype(np.float32)
    k_prev = v_prev = None
    if halo:
        k_prev = _store(g(ckp).standard_normal((B, H, window, dk), dtype=np.float32), dtype)
        if window > 1:
            v_prev = _store(g(cvp).standard_normal((B, H, window - 1, dv), dtype=np.float32),
                            dtype)
    return ChunkInputs(dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype), alpha, eta,
                       window, S0, k_prev, v_prev, meta)


def make_cotangents(B, H, T, dk, dv, *, dtype="bf16", seed=0, dS_sd=0.1):
    """Seeded cotangents for a backward call: d_o [B,H,T,dv] in the input
    storage (standard normal, rounded like the inputs) and dS_final
    [B,H,dv,dk] fp32 (normal, sd dS_sd; None when dS_sd is 0).  Widened to
    float64 they are the oracle's cotangents bit for bit."""
    ss = np.random.SeedSequence([seed, 7])
    co, cs = ss.spawn(2)
    g = lambda c: np.random.Generator(np.random.PCG64(c))  # noqa: E731
    d_o = _store(g(co).standard_normal((B, H, T, dv), dtype=np.float32), dtype)
    dS = None
    if dS_sd > 0:
        dS = (g(cs).standard_normal((B, H, dv, dk), dtype=np.float32) * np.float32(dS_sd))
        dS = dS.astype(np.float32)
    return d_o, dS


# The workloads, by what they are.  `seed` is SeedSequence(1000 + i); the last is the
# windowed (Falcon-3) decode step at the same serving shape as the Falcon-1 one.
WORKLOADS = {
    "falcon1_fp32_B1H1T256d64": dict(variant="F1", B=1, H=1, T=256, d=64, dtype="fp32",
                                     chunk=32, alpha_mu=2.0, alpha_sd=0.5, seed=1001),
    "falcon1_bf16_B8H16T4096d128": dict(variant="F1", B=8, H=16, T=4096, d=128, dtype="bf16",
                                        chunk=64, alpha_mu=3.0, alpha_sd=1.0, seed=1002),
    "falcon2_bf16_B4H32T8192d128": dict(variant="F2", B=4, H=32, T=8192, d=128, dtype="bf16",
                                        chunk=64, alpha_mu=4.0, alpha_sd=1.0, seed=1003,
                                        key_lognormal=True, span=2048),
    "falcon3_w4_bf16_B2H16T32768d128": dict(variant="F3", B=2, H=16, T=32768, d=128,
                                            dtype="bf16", chunk=64, window=4, alpha_mu=3.0,
                                            alpha_sd=1.0, seed=1004),
    "decode_falcon1_N256H32d128_1024steps": dict(variant="F1", N=256, H=32, d=128, steps=1024,
                                                 dtype="bf16", alpha_mu=3.0, alpha_sd=1.0,
                                                 S0_sd=0.02, seed=1005),
    # the Falcon-3 decode step at the same serving shape, window of four
    "decode_falcon3_w4_N256H32d128_1024steps": dict(variant="F3", N=256, H=32, d=128,
                                                    steps=1024, window=4, dtype="bf16",
                                                    alpha_mu=3.0, alpha_sd=1.0, S0_sd=0.02,
                                                    seed=1006),
}


def workload_inputs(name: str, **override) -> ChunkInputs:
    """Inputs of a chunk-forward workload; B/H/T may be overridden to draw a
    smaller instance with the same distributions."""
    w = dict(WORKLOADS[name])
    w.update(override)
    return make_chunk_inputs(w["B"], w["H"], w["T"], w["d"], w["d"], dtype=w["dtype"],
                             seed=w["seed"], alpha_mu=w["alpha_mu"], alpha_sd=w["alpha_sd"],
                             key_lognormal=w.get("key_lognormal", False), span=w.get("span", 0),
                             window=w.get("window", 1))


@dataclass
class DecodeInputs:
    """Decode inputs: S0 [N,H,dv,dk] float32, k_cache0 [N,H,W,dk] (newest key
    first), v_cache0 [N,H,W-1,dv] (newest value first; empty for W = 1) and
    per-step q,k [steps,N,H,dk], v [steps,N,H,dv] (storage type), alpha, eta
    [steps,N,H] float32."""
    dtype: str
    S0: np.ndarray
    k_cache0: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    eta: np.ndarray
    v_cache0: np.ndarray = None

    def widen(self, a):
        if self.dtype == "bf16" and a.dtype == np.uint16:
            return bits_to_f32(a).astype(np.float64)
        return np.asarray(a, dtype=np.float64)


@dataclass
class VarlenInputs:
    """Packed sequences: q, k [H,Ttot,dk], v [H,Ttot,dv] (storage type), alpha,
    eta [H,Ttot] float32, cu [N+1] int32 offsets, S0 [N,H,dv,dk] float32 or
    None, k_prev [N,H,W,dk] / v_prev [N,H,W-1,dv] (storage type) or None."""
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    eta: np.ndarray
    cu: np.ndarray
    window: int = 1
    S0: np.ndarray | None = None
    k_prev: np.ndarray | None = None
    v_prev: np.ndarray | None = None

    def sequence(self, n) -> ChunkInputs:
        """Sequence n as a one-batch ChunkInputs (a view into the packed arrays)."""
        a, b = int(self.cu[n]), int(self.cu[n + 1])
        pick = lambda x: None if x is None else x[n:n + 1]  # noqa: E731
        return ChunkInputs(self.dtype, self.q[None, :, a:b], self.k[None, :, a:b],
                           self.v[None, :, a:b], self.alpha[None, :, a:b],
                           self.eta[None, :, a:b], self.window, pick(self.S0),
                           pick(self.k_prev), pick(self.v_prev))


def make_varlen_inputs(lengths, H, dk, dv, *, dtype="bf16", seed=0, window=1, alpha_mu=3.0,
                       alpha_sd=1.0, S0_sd=0.0, halo=False, tail=0) -> VarlenInputs:
    """N sequences of the given lengths packed back to back in every head's
    plane ([H, sum(lengths) + tail, d]; `tail` rows after the last sequence
    belong to none).  Same distributions as make_chunk_inputs; children
    spawned in the order q, k, v, alpha-logit, eta-logit, S0, k_prev, v_prev."""
    lengths = [int(x) for x in lengths]
    N, Ttot = len(lengths), sum(lengths) + tail
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cq, ck, cv, ca, ce, cS, ckp, cvp = np.random.SeedSequence(seed).spawn(8)
    g = lambda c: np.random.Generator(np.random.PCG64(c))  # noqa: E731
    q = g(cq).standard_normal((H, Ttot, dk), dtype=np.float32)
    k = g(ck).standard_normal((H, Ttot, dk), dtype=np.float32)
    v = g(cv).standard_normal((H, Ttot, dv), dtype=np.float32)
    alpha = sigmoid32(g(ca).normal(alpha_mu, alpha_sd, (H, Ttot)).astype(np.float32))
    eta = sigmoid32(g(ce).normal(0.0, 1.0, (H, Ttot)).astype(np.float32))
    S0 = None
    if S0_sd > 0:
        S0 = (g(cS).standard_normal((N, H, dv, dk), dtype=np.float32) * np.float32(S0_sd))
        S0 = S0.astype(np.float32)
    k_prev = v_prev = None
    if halo:
        k_prev = _store(g(ckp).standard_normal((N, H, window, dk), dtype=np.float32), dtype)
        if window > 1:
            v_prev = _store(g(cvp).standard_normal((N, H, window - 1, dv), dtype=np.float32),
                            dtype)
    return VarlenInputs(dtype, _store(q, dtype), _store(k, dtype), _store(v, dtype), alpha, eta,
                        cu, window, S0, k_prev, v_prev)


def make_decode_inputs(N, H, dk, dv, steps, *, dtype="bf16", seed=1005, alpha_mu=3.0,
                       alpha_sd=1.0, S0_sd=0.02, window=1) -> DecodeInputs:
    ss = np.random.SeedSequence(seed)
    cq, ck, cv, ca, ce, cs, csp, cS, ckp, cvp = ss.spawn(10)
    g = lambda c: np.random.Generator(np.random.PCG64(c))  # noqa: E731
    q = g(cq).standard_normal((steps, N, H, dk), dtype=np.float32)
    k = g(ck).standard_normal((steps, N, H, dk), dtype=np.float32)
    v = g(cv).standard_normal((steps, N, H, dv), dtype=np.float32)
    alpha = sigmoid32(g(ca).normal(alpha_mu, alpha_sd, (steps, N, H)).astype(np.float32))
    eta = sigmoid32(g(ce).normal(0.0, 1.0, (steps, N, H)).astype(np.float32))
    S0 = (g(cS).standard_normal((N, H, dv, dk), dtype=np.float32) * np.float32(S0_sd))
    kc = g(ckp).standard_normal((N, H, window, dk), dtype=np.float32)
    vc = g(cvp).standard_normal((N, H, window - 1, dv), dtype=np.float32)
    return DecodeInputs(dtype, S0.astype(np.float32), _store(kc, dtype), _store(q, dtype),
                        _store(k, dtype), _store(v, dtype), alpha, eta, _store(vc, dtype))


def make_decode_inputs_torch(N, H, dk, dv, steps, *, device, seed=1005, alpha_mu=3.0,
                             alpha_sd=1.0, S0_sd=0.02, window=1):
    """Same distributions drawn on the device with torch's seeded generator,
    for workloads too large to draw on the host (the oracle then receives
    host copies of the sampled heads).  Returns a dict of bf16/fp32 tensors;
    the value cache (window - 1 slots) is drawn last, so a window of one
    draws exactly what it did before windows existed."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def n(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    out = {}
    out["S0"] = n(N, H, dv, dk) * S0_sd
    out["k_cache0"] = n(N, H, window, dk).to(torch.bfloat16)
    out["q"] = n(steps, N, H, dk).to(torch.bfloat16)
    out["k"] = n(steps, N, H, dk).to(torch.bfloat16)
    out["v"] = n(steps, N, H, dv).to(torch.bfloat16)
    out["alpha"] = torch.sigmoid(n(steps, N, H) * alpha_sd + alpha_mu)
    out["eta"] = torch.sigmoid(n(steps, N, H))
    out["v_cache0"] = n(N, H, window - 1, dv).to(torch.bfloat16)
    return out
