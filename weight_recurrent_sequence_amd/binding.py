"""Thin ctypes binding of libfalcon.so (the C ABI in include/falcon.h).

Argument marshalling only: shapes and dtypes are checked, raw device
pointers and the current HIP stream are handed to the library, and every
step of the computation runs in the library's kernels.  PyTorch provides
device memory and streams.  There is no fallback: without the built
library, or without a GPU, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfalcon.so")

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
VARIANTS = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}
SAME_STEP = 0x100  # flag OR-ed into a variant: same-step pairs (k_t, v_t)
ALIGN = {"prefix": 0, "same": SAME_STEP}
PHI_L2, PHI_SILU = 0x200, 0x400  # flags: feature map on keys and queries
PHI = {"identity": 0, "l2": PHI_L2, "silu": PHI_SILU}
FP32, BF16 = 0, 1
STATUS = {0: "FALCON_OK", -1: "FALCON_ERR_NULL", -2: "FALCON_ERR_SHAPE",
          -3: "FALCON_ERR_UNSUPPORTED", -4: "FALCON_ERR_WORKSPACE", -5: "FALCON_ERR_HIP",
          -6: "FALCON_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 128 << 20  # FALCON_NOALLOC_SCRATCH_BYTES
EXPORTS = ("falcon_chunk_fwd_workspace", "falcon_chunk_fwd", "falcon_chunk_fwd_varlen_workspace",
           "falcon_chunk_fwd_varlen", "falcon_decode_step",
           "falcon_decode_step_window", "falcon_status_string")


class FalconError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m weight_recurrent_sequence_amd._build`"
                " (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.falcon_chunk_fwd_workspace.restype = sz
        L.falcon_chunk_fwd_workspace.argtypes = [ci] * 9
        L.falcon_chunk_fwd.restype = ci
        L.falcon_chunk_fwd.argtypes = [vp] * 10 + [ci] * 9 + [cf, vp, sz, vp]
        L.falcon_chunk_fwd_varlen_workspace.restype = sz
        L.falcon_chunk_fwd_varlen_workspace.argtypes = [ci] * 9
        L.falcon_chunk_fwd_varlen.restype = ci
        L.falcon_chunk_fwd_varlen.argtypes = [vp] * 11 + [ci] * 10 + [cf, vp, sz, vp]
        L.falcon_chunk_bwd_workspace.restype = sz
        L.falcon_chunk_bwd_workspace.argtypes = [ci] * 9
        L.falcon_chunk_bwd.restype = ci
        L.falcon_chunk_bwd.argtypes = [vp] * 18 + [ci] * 9 + [cf, vp, sz, vp]
        L.falcon_chunk_bwd_varlen_workspace.restype = sz
        L.falcon_chunk_bwd_varlen_workspace.argtypes = [ci] * 9
        L.falcon_chunk_bwd_varlen.restype = ci
        L.falcon_chunk_bwd_varlen.argtypes = [vp] * 19 + [ci] * 10 + [cf, vp, sz, vp]
        for name, nvp, nci in (("falcon_chunk_fwd_save", 10, 9), ("falcon_chunk_bwd_saved", 18, 9),
                               ("falcon_chunk_fwd_varlen_save", 11, 10),
                               ("falcon_chunk_bwd_varlen_saved", 19, 10)):
            getattr(L, name).restype = ci
            getattr(L, name).argtypes = [vp] * nvp + [ci] * nci + [cf, vp, sz, vp]
        L.falcon_chunk_fwd_noalloc.restype = ci
        L.falcon_chunk_fwd_noalloc.argtypes = [vp] * 10 + [ci] * 9 + [cf, vp]
        L.falcon_decode_step.restype = ci
        L.falcon_decode_step.argtypes = [vp] * 8 + [ci] * 7 + [cf, vp]
        L.falcon_decode_step_window.restype = ci
        L.falcon_decode_step_window.argtypes = [vp] * 9 + [ci] * 7 + [cf, vp]
        L.falcon_status_string.restype = ctypes.c_char_p
        L.falcon_status_string.argtypes = [ci]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().falcon_status_string(int(status)).decode()


def _variant(v, align="prefix", phi="identity") -> int:
    """Variant code with the flags: align="prefix" pairs (k_{t-1}, v_t),
    align="same" pairs (k_t, v_t); phi="identity", "l2" or "silu" maps keys
    and queries."""
    return (VARIANTS[v] if isinstance(v, str) else int(v)) | ALIGN[align] | PHI[phi]


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(B, H, T, dk, dv, dtype, variant, window=1, chunk=64, phi="identity") -> int:
    return int(lib().falcon_chunk_fwd_workspace(B, H, T, dk, dv, dtype, _variant(variant, phi=phi),
                                                window, chunk))


def chunk_fwd(q, k, v, alpha, eta, variant, *, window=1, chunk=64, eps=1e-6, S0=None,
              k_prev=None, v_prev=None, o=None, S_final=None, return_state=True,
              workspace=None, stream=None, align="prefix", phi="identity", _save=False):
    """Chunk-parallel forward.  q,k [B,H,T,dk]; v [B,H,T,dv] (bf16 or fp32);
    alpha, eta [B,H,T] fp32; S0 [B,H,dv,dk] fp32 or None; k_prev [B,H,W,dk],
    v_prev [B,H,W-1,dv] or None.  `workspace` (uint8 device tensor of at
    least workspace_bytes(...) bytes) is allocated per call when omitted.
    Returns (o, S_final) (S_final None if return_state is False and none was
    given)."""
    import torch
    var = _variant(variant, align, phi)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(alpha, "alpha", (B, H, T), torch.float32, dev)
    _check(eta, "eta", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    _check(k_prev, "k_prev", (B, H, window, dk), dt, dev)
    if window > 1:
        _check(v_prev, "v_prev", (B, H, window - 1, dv), dt, dev)
    else:
        v_prev = None
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _check(o, "o", (B, H, T, dv), dt, dev)
    if S_final is None and return_state:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (B, H, dv, dk), torch.float32, dev)
    query = lib().falcon_chunk_bwd_workspace if _save else lib().falcon_chunk_fwd_workspace
    ws_n = int(query(B, H, T, dk, dv, dtc, var, window, chunk))
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
            raise ValueError(f"workspace: need {ws_n} bytes on {dev}")
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n > 0 else None
    name = "falcon_chunk_fwd_save" if _save else "falcon_chunk_fwd"
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(S0),
                              _ptr(k_prev), _ptr(v_prev), _ptr(o), _ptr(S_final), B, H, T, dk,
                              dv, dtc, var, window, chunk, float(eps), _ptr(ws), ws_n,
                              _stream(stream))
    if st != 0:
        raise FalconError(st, name)
    return o, S_final


def chunk_fwd_noalloc(q, k, v, alpha, eta, variant, *, window=1, chunk=64, eps=1e-6, S0=None,
                      k_prev=None, v_prev=None, o=None, S_final=None, stream=None,
                      align="prefix", phi="identity"):
    """chunk_fwd through falcon_chunk_fwd_noalloc: the library's built-in
    scratch buffer replaces the workspace (no device allocation by the call;
    o and S_final are allocated here when not given).  Raises FalconError
    (FALCON_ERR_SCRATCH) when the call needs more than NOALLOC_SCRATCH_BYTES.
    Returns (o, S_final)."""
    import torch
    var = _variant(variant, align, phi)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(alpha, "alpha", (B, H, T), torch.float32, dev)
    _check(eta, "eta", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    _check(k_prev, "k_prev", (B, H, window, dk), dt, dev)
    if window > 1:
        _check(v_prev, "v_prev", (B, H, window - 1, dv), dt, dev)
    else:
        v_prev = None
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _check(o, "o", (B, H, T, dv), dt, dev)
    if S_final is None:
        S_final = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (B, H, dv, dk), torch.float32, dev)
    st = lib().falcon_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta),
                                        _ptr(S0), _ptr(k_prev), _ptr(v_prev), _ptr(o),
                                        _ptr(S_final), B, H, T, dk, dv, dtc, var, window, chunk,
                                        float(eps), _stream(stream))
    if st != 0:
        raise FalconError(st, "falcon_chunk_fwd_noalloc")
    return o, S_final


def chunk_fwd_save(q, k, v, alpha, eta, variant, *, saved, **kw):
    """chunk_fwd that also leaves the backward's records and checkpoints in
    `saved` (uint8 device tensor of at least bwd_workspace_bytes(...) bytes),
    for chunk_bwd_saved on the same inputs.  Returns (o, S_final)."""
    return chunk_fwd(q, k, v, alpha, eta, variant, workspace=saved, _save=True, **kw)


def bwd_workspace_bytes(B, H, T, dk, dv, dtype, variant, window=1, chunk=64, align="prefix",
                        phi="identity") -> int:
    return int(lib().falcon_chunk_bwd_workspace(B, H, T, dk, dv, dtype,
                                                _variant(variant, align, phi), window, chunk))


def chunk_bwd(q, k, v, alpha, eta, d_o, variant, *, dS_final=None, window=1, chunk=64,
              eps=1e-6, S0=None, k_prev=None, v_prev=None, want_dS0=True, want_dk_prev=None,
              workspace=None, stream=None, align="prefix", phi="identity", _saved=False):
    """Gradients of the chunk forward.  Inputs as for chunk_fwd, plus d_o
    [B,H,T,dv] (input dtype) and dS_final [B,H,dv,dk] fp32 or None.  Returns a
    dict with dq, dk, dv (input dtype), dalpha, deta (fp32), dS0 (fp32, or
    None), dk_prev (input dtype, when k_prev is given or want_dk_prev) and,
    for a window above one, dv_prev (likewise)."""
    import torch
    var = _variant(variant, align, phi)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    _check(q, "q", (B, H, T, dk), dt, dev)
    _check(k, "k", (B, H, T, dk), dt, dev)
    _check(v, "v", (B, H, T, dv), dt, dev)
    _check(d_o, "d_o", (B, H, T, dv), dt, dev)
    _check(alpha, "alpha", (B, H, T), torch.float32, dev)
    _check(eta, "eta", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, dv, dk), torch.float32, dev)
    _check(dS_final, "dS_final", (B, H, dv, dk), torch.float32, dev)
    _check(k_prev, "k_prev", (B, H, window, dk), dt, dev)
    if window > 1:
        _check(v_prev, "v_prev", (B, H, window - 1, dv), dt, dev)
    else:
        v_prev = None
    g = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
             dalpha=torch.empty_like(alpha), deta=torch.empty_like(eta),
             dS0=torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None)
    if want_dk_prev is None:
        want_dk_prev = k_prev is not None
    g["dk_prev"] = torch.empty((B, H, window, dk), dtype=dt, device=dev) if want_dk_prev else None
    # a window above one also reads W-1 values before the sequence
    want_dv_prev = window > 1 and (v_prev is not None or want_dk_prev)
    g["dv_prev"] = torch.empty((B, H, window - 1, dv), dtype=dt, device=dev) if want_dv_prev else None
    ws_n = int(lib().falcon_chunk_bwd_workspace(B, H, T, dk, dv, dtc, var, window, chunk))
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
            raise ValueError(f"workspace: need {ws_n} bytes on {dev}")
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n > 0 else None
    if _saved and workspace is None and ws_n > 0:
        raise ValueError("chunk_bwd_saved needs the buffer chunk_fwd_save filled")
    name = "falcon_chunk_bwd_saved" if _saved else "falcon_chunk_bwd"
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(S0),
                              _ptr(k_prev), _ptr(v_prev), _ptr(d_o), _ptr(dS_final),
                              _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]),
                              _ptr(g["deta"]), _ptr(g["dS0"]), _ptr(g["dk_prev"]), _ptr(g["dv_prev"]),
                              B, H, T, dk, dv, dtc, var, window, chunk, float(eps), _ptr(ws),
                              ws_n, _stream(stream))
    if st != 0:
        raise FalconError(st, name)
    return g


def chunk_bwd_saved(q, k, v, alpha, eta, d_o, variant, *, saved, **kw):
    """chunk_bwd from the buffer a chunk_fwd_save call on the same inputs
    filled (the forward is not re-run).  Returns the dict chunk_bwd returns."""
    return chunk_bwd(q, k, v, alpha, eta, d_o, variant, workspace=saved, _saved=True, **kw)


def bwd_varlen_workspace_bytes(N, H, max_seqlen, dk, dv, dtype, variant, window=1, chunk=64,
                               align="prefix", phi="identity") -> int:
    return int(lib().falcon_chunk_bwd_varlen_workspace(N, H, max_seqlen, dk, dv, dtype,
                                                       _variant(variant, align, phi), window,
                                                       chunk))


def chunk_bwd_varlen(q, k, v, alpha, eta, cu_seqlens, d_o, variant, *, max_seqlen=None,
                     dS_final=None, window=1, chunk=64, eps=1e-6, S0=None, k_prev=None,
                     v_prev=None, want_dS0=True, want_dk_prev=None, workspace=None, stream=None,
                     align="prefix", phi="identity", _saved=False):
    """Gradients of chunk_fwd_varlen.  q, k, v, d_o [H,total_T,d]; alpha, eta
    [H,total_T]; cu_seqlens int32 [N+1] on the device; S0, dS_final
    [N,H,d,d]; k_prev [N,H,W,d], v_prev [N,H,W-1,d].  Returns a dict as
    chunk_bwd does (dq, dk, dv, dalpha, deta in the packed layout; dS0 and the
    halo gradients per sequence).  Rows outside every sequence are left as
    allocated (torch.zeros here)."""
    import torch
    var = _variant(variant, align, phi)
    H, Ttot, dk = k.shape
    dv = v.shape[-1]
    N = cu_seqlens.numel() - 1
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    if max_seqlen is None:
        c = cu_seqlens.cpu()
        max_seqlen = int((c[1:] - c[:-1]).max()) if N > 0 else 0
    _check(q, "q", (H, Ttot, dk), dt, dev)
    _check(v, "v", (H, Ttot, dv), dt, dev)
    _check(d_o, "d_o", (H, Ttot, dv), dt, dev)
    _check(alpha, "alpha", (H, Ttot), torch.float32, dev)
    _check(eta, "eta", (H, Ttot), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _check(S0, "S0", (N, H, dv, dk), torch.float32, dev)
    _check(dS_final, "dS_final", (N, H, dv, dk), torch.float32, dev)
    _check(k_prev, "k_prev", (N, H, window, dk), dt, dev)
    if window > 1:
        _check(v_prev, "v_prev", (N, H, window - 1, dv), dt, dev)
    else:
        v_prev = None
    g = dict(dq=torch.zeros_like(q), dk=torch.zeros_like(k), dv=torch.zeros_like(v),
             dalpha=torch.zeros_like(alpha), deta=torch.zeros_like(eta),
             dS0=torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev) if want_dS0 else None)
    if want_dk_prev is None:
        want_dk_prev = k_prev is not None
    g["dk_prev"] = torch.empty((N, H, window, dk), dtype=dt, device=dev) if want_dk_prev else None
    want_dv_prev = window > 1 and (v_prev is not None or want_dk_prev)
    g["dv_prev"] = torch.empty((N, H, window - 1, dv), dtype=dt, device=dev) if want_dv_prev else None
    ws_n = int(lib().falcon_chunk_bwd_varlen_workspace(N, H, max_seqlen, dk, dv, dtc, var, window,
                                                       chunk))
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
            raise ValueError(f"workspace: need {ws_n} bytes on {dev}")
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n > 0 else None
    if _saved and workspace is None and ws_n > 0:
        raise ValueError("chunk_bwd_varlen_saved needs the buffer chunk_fwd_varlen_save filled")
    name = "falcon_chunk_bwd_varlen_saved" if _saved else "falcon_chunk_bwd_varlen"
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(S0),
                              _ptr(k_prev), _ptr(v_prev), _ptr(d_o), _ptr(dS_final),
                              _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                              _ptr(g["dalpha"]), _ptr(g["deta"]), _ptr(g["dS0"]),
                              _ptr(g["dk_prev"]), _ptr(g["dv_prev"]), _ptr(cu_seqlens),
                              N, H, Ttot, max_seqlen, dk, dv, dtc, var, window, chunk,
                              float(eps), _ptr(ws), ws_n, _stream(stream))
    if st != 0:
        raise FalconError(st, name)
    return g


def chunk_bwd_varlen_saved(q, k, v, alpha, eta, cu_seqlens, d_o, variant, *, saved, **kw):
    """chunk_bwd_varlen from the buffer a chunk_fwd_varlen_save call on the
    same inputs filled."""
    return chunk_bwd_varlen(q, k, v, alpha, eta, cu_seqlens, d_o, variant, workspace=saved,
                            _saved=True, **kw)


def varlen_workspace_bytes(N, H, max_seqlen, dk, dv, dtype, variant, window=1, chunk=64,
                           phi="identity") -> int:
    return int(lib().falcon_chunk_fwd_varlen_workspace(N, H, max_seqlen, dk, dv, dtype,
                                                       _variant(variant, phi=phi), window, chunk))


def chunk_fwd_varlen(q, k, v, alpha, eta, cu_seqlens, variant, *, max_seqlen=None, window=1,
                     chunk=64, eps=1e-6, S0=None, k_prev=None, v_prev=None, o=None,
                     S_final=None, return_state=True, workspace=None, stream=None,
                     align="prefix", phi="identity", _save=False):
    """Chunk-parallel forward over N packed sequences.  q, k [H,total_T,dk];
    v [H,total_T,dv]; alpha, eta [H,total_T] fp32; cu_seqlens int32 [N+1] on
    the device (sequence n = rows cu_seqlens[n] .. cu_seqlens[n+1]-1 of every
    head); S0 [N,H,dv,dk]; k_prev [N,H,W,dk]; v_prev [N,H,W-1,dv].
    max_seqlen bounds every sequence's length; when None it is read from
    cu_seqlens (a device-to-host copy, which synchronizes).  Returns
    (o [H,total_T,dv], S_final [N,H,dv,dk] or None)."""
    import torch
    var = _variant(variant, align, phi)
    H, Ttot, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev \
            or not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens: int32 [N+1] contiguous tensor on the inputs' device")
    N = cu_seqlens.numel() - 1
    if max_seqlen is None:
        c = cu_seqlens.cpu()
        max_seqlen = int((c[1:] - c[:-1]).max().item()) if N > 0 else 0
    _check(q, "q", (H, Ttot, dk), dt, dev)
    _check(k, "k", (H, Ttot, dk), dt, dev)
    _check(v, "v", (H, Ttot, dv), dt, dev)
    _check(alpha, "alpha", (H, Ttot), torch.float32, dev)
    _check(eta, "eta", (H, Ttot), torch.float32, dev)
    _check(S0, "S0", (N, H, dv, dk), torch.float32, dev)
    _check(k_prev, "k_prev", (N, H, window, dk), dt, dev)
    if window > 1:
        _check(v_prev, "v_prev", (N, H, window - 1, dv), dt, dev)
    else:
        v_prev = None
    if o is None:
        o = torch.empty((H, Ttot, dv), dtype=dt, device=dev)
    _check(o, "o", (H, Ttot, dv), dt, dev)
    if S_final is None and return_state:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    _check(S_final, "S_final", (N, H, dv, dk), torch.float32, dev)
    query = (lib().falcon_chunk_bwd_varlen_workspace if _save
             else lib().falcon_chunk_fwd_varlen_workspace)
    ws_n = int(query(N, H, max_seqlen, dk, dv, dtc, var, window, chunk))
    if workspace is not None:
        if workspace.device != dev or workspace.numel() * workspace.element_size() < ws_n:
            raise ValueError(f"workspace: need {ws_n} bytes on {dev}")
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n > 0 else None
    name = "falcon_chunk_fwd_varlen_save" if _save else "falcon_chunk_fwd_varlen"
    st = getattr(lib(), name)(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta),
                              _ptr(S0), _ptr(k_prev), _ptr(v_prev), _ptr(o),
                              _ptr(S_final), _ptr(cu_seqlens), N, H, Ttot, max_seqlen,
                              dk, dv, dtc, var, window, chunk, float(eps), _ptr(ws),
                              ws_n, _stream(stream))
    if st != 0:
        raise FalconError(st, name)
    return o, S_final


def chunk_fwd_varlen_save(q, k, v, alpha, eta, cu_seqlens, variant, *, saved, **kw):
    """chunk_fwd_varlen that also leaves the backward's records and
    checkpoints in `saved` (at least bwd_varlen_workspace_bytes(...) bytes),
    for chunk_bwd_varlen_saved on the same inputs."""
    return chunk_fwd_varlen(q, k, v, alpha, eta, cu_seqlens, variant, workspace=saved, _save=True,
                            **kw)


def decode_step(S, k_cache, q, k, v, alpha, eta, variant, *, eps=1e-6, o=None, stream=None,
                align="prefix", phi="identity"):
    """One decode step.  S [N,H,dv,dk] fp32 and k_cache [N,H,1,dk] are
    updated in place; q,k [N,H,dk], v [N,H,dv] (bf16 or fp32), alpha, eta
    [N,H] fp32.  Returns o [N,H,dv]."""
    import torch
    var = _variant(variant, align, phi)
    N, H, dv, dk = S.shape
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    _check(S, "S", (N, H, dv, dk), torch.float32, dev)
    _check(k_cache, "k_cache", (N, H, 1, dk), dt, dev)
    _check(q, "q", (N, H, dk), dt, dev)
    _check(k, "k", (N, H, dk), dt, dev)
    _check(v, "v", (N, H, dv), dt, dev)
    _check(alpha, "alpha", (N, H), torch.float32, dev)
    _check(eta, "eta", (N, H), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _check(o, "o", (N, H, dv), dt, dev)
    st = lib().falcon_decode_step(_ptr(S), _ptr(k_cache), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(alpha), _ptr(eta), _ptr(o), N, H, dk, dv, dtc, var, 1,
                                  float(eps), _stream(stream))
    if st != 0:
        raise FalconError(st, "falcon_decode_step")
    return o


def decode_step_window(S, k_cache, v_cache, q, k, v, alpha, eta, variant, *, eps=1e-6, o=None,
                       stream=None, align="prefix", phi="identity"):
    """One Falcon-3 / Falcon-3A decode step.  S [N,H,dv,dk] fp32, k_cache
    [N,H,W,dk] (slot w = k_{t-1-w}) and v_cache [N,H,W-1,dv] (slot w-1 =
    v_{t-w}; None when W = 1) are updated in place; q,k [N,H,dk], v [N,H,dv]
    (bf16 or fp32), alpha, eta [N,H] fp32.  Returns o [N,H,dv]."""
    import torch
    var = _variant(variant, align, phi)
    N, H, dv, dk = S.shape
    dev, dt = k.device, k.dtype
    dtc = _dt(k)
    W = k_cache.shape[2] if k_cache.dim() == 4 else -1
    _check(S, "S", (N, H, dv, dk), torch.float32, dev)
    _check(k_cache, "k_cache", (N, H, W, dk), dt, dev)
    if W > 1 or v_cache is not None:
        _check(v_cache, "v_cache", (N, H, W - 1, dv), dt, dev)
    _check(q, "q", (N, H, dk), dt, dev)
    _check(k, "k", (N, H, dk), dt, dev)
    _check(v, "v", (N, H, dv), dt, dev)
    _check(alpha, "alpha", (N, H), torch.float32, dev)
    _check(eta, "eta", (N, H), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _check(o, "o", (N, H, dv), dt, dev)
    st = lib().falcon_decode_step_window(_ptr(S), _ptr(k_cache), _ptr(v_cache) if W > 1 else None,
                                         _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(eta), _ptr(o),
                                         N, H, dk, dv, dtc, var, W, float(eps), _stream(stream))
    if st != 0:
        raise FalconError(st, "falcon_decode_step_window")
    return o
