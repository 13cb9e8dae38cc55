"""GPU tests of the training pair falcon_chunk_fwd_save / falcon_chunk_bwd_saved
(and their packed forms): the saving forward returns exactly what
falcon_chunk_fwd returns, and the backward from the saved buffer returns
exactly what falcon_chunk_bwd (which re-runs the forward itself) returns.
Both sides run the same kernels on the same inputs, so the comparison is
bitwise; the backward's own parity with the fp64 oracle is tested in
test_gpu_bwd.py and test_gpu_varlen_bwd.py."""
import numpy as np
import pytest

from tests.gpu_util import announce, ensure_built
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "deta", "dS0", "dk_prev", "dv_prev")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def to_dev(a, dev):
    import torch
    if a is None:
        return None
    x = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        x = x.view(torch.bfloat16)
    return x.to(dev)


def same(a, b, what):
    import torch
    if a is None or b is None:
        assert a is None and b is None, what
        return
    assert torch.equal(a, b), what


# (variant, d, window, align, feature map)
CASES = [("F1", 128, 1, "prefix", "identity"), ("F1A", 64, 1, "prefix", "identity"),
         ("F2", 128, 1, "prefix", "identity"), ("F2A", 64, 1, "same", "identity"),
         ("F3", 128, 3, "prefix", "identity"), ("F3A", 64, 4, "prefix", "identity"),
         ("F1", 64, 1, "same", "l2"), ("F3", 64, 2, "prefix", "silu")]


@pytest.mark.parametrize("T", [150, 64, 1])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_saved_pair_equals_recompute(dev, case, T):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, D, W, align, phi = case
    B, H = 2, 3
    inp = I.make_chunk_inputs(B, H, T, D, D, dtype="bf16", seed=1700 + D + W + T, window=W,
                              S0_sd=0.3, halo=True)
    t = inp.to_torch(dev)
    kw = dict(window=W, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"], align=align, phi=phi)
    n = fal.bwd_workspace_bytes(B, H, T, D, D, fal.BF16, variant, W, 64, align=align, phi=phi)
    saved = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    announce(f"chunk_fwd_save {variant} d{D} W{W} T{T} align={align} phi={phi}")
    o_s, S_s = fal.chunk_fwd_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant,
                                  saved=saved, **kw)
    o_r, S_r = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, **kw)
    torch.cuda.synchronize()
    same(o_s, o_r, "o")
    same(S_s, S_r, "S_final")
    # two backward calls from one saved buffer, with different cotangents
    for rep in range(2):
        d_o, dS = I.make_cotangents(B, H, T, D, D, seed=1750 + rep)
        d_o, dS = to_dev(d_o, dev), to_dev(dS, dev)
        announce(f"chunk_bwd_saved {variant} d{D} W{W} T{T} call {rep}")
        g_s = fal.chunk_bwd_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant,
                                  saved=saved, dS_final=dS, want_dk_prev=True, **kw)
        g_r = fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant,
                            dS_final=dS, want_dk_prev=True, **kw)
        torch.cuda.synchronize()
        for k in GRADS:
            same(g_s[k], g_r[k], (k, rep))


LENGTHS = [130, 0, 1, 63, 200, 64, 17]


@pytest.mark.parametrize("case", [("F1", 128, 1), ("F2A", 64, 1), ("F3", 128, 3)],
                         ids=lambda c: "-".join(map(str, c)))
def test_saved_pair_varlen_equals_recompute(dev, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, D, W = case
    H = 2
    vi = I.make_varlen_inputs(LENGTHS, H, D, D, dtype="bf16", seed=1780 + D + W, window=W,
                              S0_sd=0.3, halo=True)
    t = {n: to_dev(getattr(vi, n), dev) for n in ("q", "k", "v", "k_prev", "v_prev", "alpha",
                                                   "eta", "S0")}
    cu = torch.from_numpy(vi.cu).to(dev)
    N, mx = len(LENGTHS), max(LENGTHS)
    kw = dict(max_seqlen=mx, window=W, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"])
    n = fal.bwd_varlen_workspace_bytes(N, H, mx, D, D, fal.BF16, variant, W, 64)
    saved = torch.empty(n, dtype=torch.uint8, device=dev)
    announce(f"chunk_fwd_varlen_save {variant} d{D} W{W} lengths {LENGTHS}")
    o_s, S_s = fal.chunk_fwd_varlen_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, variant,
                                         saved=saved, **kw)
    o_r, S_r = fal.chunk_fwd_varlen(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, variant, **kw)
    torch.cuda.synchronize()
    same(o_s, o_r, "o")
    same(S_s, S_r, "S_final")
    d_o, _ = I.make_cotangents(1, H, int(vi.cu[-1]), D, D, seed=1790, dS_sd=0)
    _, dS = I.make_cotangents(N, H, 0, D, D, seed=1791)
    d_o, dS = to_dev(d_o[0], dev), to_dev(dS, dev)
    announce(f"chunk_bwd_varlen_saved {variant} d{D} W{W}")
    g_s = fal.chunk_bwd_varlen_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, d_o, variant,
                                     saved=saved, dS_final=dS, **kw)
    g_r = fal.chunk_bwd_varlen(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, d_o, variant,
                               dS_final=dS, **kw)
    torch.cuda.synchronize()
    for k in GRADS:
        same(g_s[k], g_r[k], k)


@pytest.mark.parametrize("case", [("F1", 128, 1), ("F3A", 64, 4)], ids=lambda c: "-".join(map(str, c)))
def test_saved_pair_no_steps(dev, case):
    """T = 0: the saving forward only copies S0 to S_final (no buffer is
    needed), and the backward from it gives dS0 = dS_final and zero halo
    gradients, as the recompute path does."""
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, D, W = case
    B, H = 2, 3
    inp = I.make_chunk_inputs(B, H, 0, D, D, dtype="bf16", seed=1800 + D, window=W, S0_sd=0.3,
                              halo=True)
    t = inp.to_torch(dev)
    kw = dict(window=W, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"])
    assert fal.bwd_workspace_bytes(B, H, 0, D, D, fal.BF16, variant, W, 64) == 0
    saved = torch.empty(0, dtype=torch.uint8, device=dev)
    announce(f"chunk_fwd_save {variant} d{D} W{W} T0")
    o_s, S_s = fal.chunk_fwd_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant,
                                  saved=saved, **kw)
    o_r, S_r = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, **kw)
    torch.cuda.synchronize()
    same(S_s, S_r, "S_final")
    assert torch.equal(S_s, t["S0"])
    _, dS = I.make_cotangents(B, H, 0, D, D, seed=1810)
    d_o = torch.empty((B, H, 0, D), dtype=torch.bfloat16, device=dev)
    dS = to_dev(dS, dev)
    announce(f"chunk_bwd_saved {variant} d{D} W{W} T0")
    g_s = fal.chunk_bwd_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant,
                              saved=saved, dS_final=dS, want_dk_prev=True, **kw)
    g_r = fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant, dS_final=dS,
                        want_dk_prev=True, **kw)
    torch.cuda.synchronize()
    for k in GRADS:
        same(g_s[k], g_r[k], k)
    assert torch.equal(g_s["dS0"], dS)


@pytest.mark.parametrize("case", [("F1A", 128, 1), ("F3A", 128, 4), ("F3", 64, 3), ("F1", 128, 1)],
                         ids=lambda c: "-".join(map(str, c)))
def test_saved_pair_with_aliased_state(dev, case):
    """S_final aliasing S0 in the saving forward: o is still falcon_chunk_fwd's,
    the checkpoints come from the unmodified S0 (the backward from them equals
    the recomputing backward bitwise), and S_final is the recurrence's final
    state (for the rules whose forward runs other kernels, from the
    checkpoint run's split kernels: equal up to rounding)."""
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, D, W = case
    B, H, T = 2, 3, 150
    inp = I.make_chunk_inputs(B, H, T, D, D, dtype="bf16", seed=1780 + D + W, window=W, S0_sd=0.3,
                              halo=True)
    t = inp.to_torch(dev)
    kw = dict(window=W, k_prev=t["k_prev"], v_prev=t["v_prev"])
    n = fal.bwd_workspace_bytes(B, H, T, D, D, fal.BF16, variant, W, 64)
    saved = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    S_alias = t["S0"].clone()
    announce(f"chunk_fwd_save {variant} d{D} W{W} T{T} S_final = S0")
    o_s, _ = fal.chunk_fwd_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, saved=saved,
                                S0=S_alias, S_final=S_alias, **kw)
    o_r, S_r = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, S0=t["S0"], **kw)
    torch.cuda.synchronize()
    same(o_s, o_r, "o")
    err = ((S_alias - S_r).abs().amax(dim=(2, 3)) / S_r.abs().amax(dim=(2, 3))).max().item()
    assert err <= 1e-2, err
    d_o, dS = I.make_cotangents(B, H, T, D, D, seed=1790)
    d_o, dS = to_dev(d_o, dev), to_dev(dS, dev)
    announce(f"chunk_bwd_saved {variant} d{D} W{W} T{T} after an aliased save")
    g_s = fal.chunk_bwd_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant, saved=saved,
                              S0=t["S0"], dS_final=dS, want_dk_prev=True, **kw)
    g_r = fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant, S0=t["S0"],
                        dS_final=dS, want_dk_prev=True, **kw)
    torch.cuda.synchronize()
    for k in GRADS:
        same(g_s.get(k), g_r.get(k), k)
