"""fp64 CPU oracle of the Falcon fast-weight recurrence.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library never imports, links
or calls anything here, and nothing here imports the GPU package.

Contents
--------
recurrent(...)    the step-by-step form, in plain C (falcon_oracle.c), threads
                  over the independent (batch, head) sequences.
decode_step(...)  one step of the same recurrence for N x H heads.
decode_step_window(...)  the same for Falcon-3/3A, with key and value caches.
Every entry takes align="prefix" (the pair of step t is (k_{t-1}, v_t), the
authors' alignment) or align="same" (k_t, v_t: the same-step alignment of the
KLA/GDN recurrences the pages contrast it with), and phi="identity" (the
default), "l2" (x / ||x||, 0 for x = 0) or "silu" (x / (1 + exp(-x))): a
feature map applied to every key and query.
forms             numpy fp64 masked-parallel and chunk-parallel forms, used only
                  to cross-check the recurrent form (the authors' abstract of
                  "Fast Weight Attention for Continual Learning" states that the
                  rules have recurrent, masked-parallel and chunk-parallel forms).
exact             the recurrent form in exact rational arithmetic, for tiny
                  inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "falcon_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
VARIANTS = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}
ALIGN_LAG = {"prefix": 1, "same": 0}
PHI = {"identity": 0, "l2": 1, "silu": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
             SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_recurrent_ex.restype = ctypes.c_int
        lib.oracle_recurrent_ex.argtypes = [ctypes.c_int] * 9 + [ctypes.c_double] + [dp] * 10 + [ctypes.c_int]
        lib.oracle_decode_step_ex.restype = ctypes.c_int
        lib.oracle_decode_step_ex.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double] + [dp] * 8
        lib.oracle_decode_step_window_ex.restype = ctypes.c_int
        lib.oracle_decode_step_window_ex.argtypes = [ctypes.c_int] * 8 + [ctypes.c_double] + [dp] * 9
        lib.oracle_num_cpus.restype = ctypes.c_int
        lib.oracle_num_cpus.argtypes = []
        _lib = lib
    return _lib


def num_cpus() -> int:
    return _load().oracle_num_cpus()


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(variant, q, k, v, alpha, eta, *, window=1, eps=1e-6, S0=None, k_prev=None,
              v_prev=None, nthreads=0, align="prefix", phi="identity"):
    """Run the recurrence.  q, k: [B,H,T,dk]; v: [B,H,T,dv]; alpha, eta: [B,H,T];
    k_prev holds the W keys before the sequence (oldest first) in either
    alignment.

    Returns (o [B,H,T,dv], S_T [B,H,dv,dk]) in float64.
    """
    variant = VARIANTS.get(variant, variant)
    lag = ALIGN_LAG[align]
    q, k, v, alpha, eta = map(_f64, (q, k, v, alpha, eta))
    S0, k_prev, v_prev = map(_f64, (S0, k_prev, v_prev))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
    assert alpha.shape == (B, H, T) and eta.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dv, dk)
    if k_prev is not None:
        assert k_prev.shape == (B, H, window, dk)
    if v_prev is not None:
        assert v_prev.shape == (B, H, window - 1, dv)
    o = np.zeros((B, H, T, dv), np.float64)
    S = np.zeros((B, H, dv, dk), np.float64)
    rc = _load().oracle_recurrent_ex(variant, B, H, T, dk, dv, window, lag, PHI[phi], float(eps), _ptr(q),
                                      _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(S0),
                                      _ptr(k_prev), _ptr(v_prev), _ptr(o), _ptr(S), int(nthreads))
    if rc < 0:
        raise ValueError(f"oracle_recurrent rejected its arguments (code {rc})")
    return o, S


def recurrent_threads_used(B, H, nthreads=0):
    n = nthreads if nthreads > 0 else num_cpus()
    return min(n, B * H)


def decode_step(variant, S, k_cache, q, k, v, alpha, eta, *, eps=1e-6, align="prefix",
                phi="identity"):
    """One decode step.  S [N,H,dv,dk] and k_cache [N,H,dk] are copied, updated
    and returned together with o [N,H,dv]: (o, S_new, k_cache_new)."""
    variant = VARIANTS.get(variant, variant)
    lag = ALIGN_LAG[align]
    S = _f64(S).copy()
    k_cache = _f64(k_cache).copy()
    q, k, v, alpha, eta = map(_f64, (q, k, v, alpha, eta))
    N, H, dv, dk = S.shape
    k_cache = k_cache.reshape(N, H, dk).copy()
    o = np.zeros((N, H, dv), np.float64)
    rc = _load().oracle_decode_step_ex(variant, N, H, dk, dv, lag, PHI[phi], float(eps), _ptr(S),
                                        _ptr(k_cache), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(eta), _ptr(o))
    if rc < 0:
        raise ValueError(f"oracle_decode_step rejected its arguments (code {rc})")
    return o, S, k_cache


def decode_step_window(variant, S, k_cache, v_cache, q, k, v, alpha, eta, *, eps=1e-6,
                       align="prefix", phi="identity"):
    """One Falcon-3 / Falcon-3A decode step with a window of W pairs.

    S [N,H,dv,dk]; k_cache [N,H,W,dk] with k_cache[..., w, :] = k_{t-1-w};
    v_cache [N,H,W-1,dv] with v_cache[..., w-1, :] = v_{t-w}.  Returns
    (o, S_new, k_cache_new, v_cache_new), all float64 copies."""
    variant = VARIANTS.get(variant, variant)
    lag = ALIGN_LAG[align]
    S = _f64(S).copy()
    q, k, v, alpha, eta = map(_f64, (q, k, v, alpha, eta))
    N, H, dv, dk = S.shape
    k_cache = _f64(k_cache).reshape(N, H, -1, dk).copy()
    W = k_cache.shape[2]
    v_cache = (_f64(v_cache).reshape(N, H, W - 1, dv).copy() if W > 1
               else np.zeros((N, H, 0, dv), np.float64))
    o = np.zeros((N, H, dv), np.float64)
    vbuf = v_cache if W > 1 else np.zeros((N, H, 1, dv), np.float64)
    rc = _load().oracle_decode_step_window_ex(variant, N, H, dk, dv, W, lag, PHI[phi], float(eps), _ptr(S),
                                           _ptr(k_cache), _ptr(vbuf), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(alpha), _ptr(eta), _ptr(o))
    if rc < 0:
        raise ValueError(f"oracle_decode_step_window rejected its arguments (code {rc})")
    return o, S, k_cache, v_cache
