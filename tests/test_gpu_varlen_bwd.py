"""GPU parity of falcon_chunk_bwd_varlen (the backward of N packed sequences
of different lengths): against one batched falcon_chunk_bwd call per
sequence (bitwise: the same kernels do the same arithmetic on each
sequence), and against the fp64 gradient oracle run on each sequence."""
import numpy as np
import pytest

from oracle import grad as G
from tests.gpu_util import TOL, announce, ensure_built, slice_rel_err, to_np
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

# empty, single-step, ragged and several-tile sequences
LENGTHS = [130, 0, 1, 63, 200, 64, 17]
GRADS = ("dq", "dk", "dv", "dalpha", "deta")


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


def packed_cotangents(vi, seed):
    H, Ttot, D = vi.v.shape
    N = len(vi.cu) - 1
    d_o, _ = I.make_cotangents(1, H, Ttot, D, D, seed=seed, dS_sd=0)
    _, dS = I.make_cotangents(N, H, 0, D, D, seed=seed + 1)
    return d_o[0], dS


def run_packed(dev, vi, variant, d_o, dS, align="prefix"):
    import torch
    import weight_recurrent_sequence_amd as fal
    t = {n: to_dev(getattr(vi, n), dev) for n in ("q", "k", "v", "k_prev", "v_prev", "alpha",
                                                   "eta", "S0")}
    cu = torch.from_numpy(vi.cu).to(dev)
    announce(f"chunk_bwd_varlen {variant} H{vi.k.shape[0]} lengths {np.diff(vi.cu).tolist()} "
             f"W{vi.window} align={align}")
    g = fal.chunk_bwd_varlen(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, to_dev(d_o, dev),
                             variant, dS_final=to_dev(dS, dev), window=vi.window, S0=t["S0"],
                             k_prev=t["k_prev"], v_prev=t["v_prev"], align=align)
    torch.cuda.synchronize()
    return g


CASES = [("F1", 128, 1), ("F1A", 64, 1), ("F2", 128, 1), ("F3", 128, 3), ("F3A", 64, 4)]


@pytest.mark.parametrize("align", ["prefix", "same"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_varlen_bwd_equals_one_call_per_sequence(dev, case, align):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, D, W = case
    vi = I.make_varlen_inputs(LENGTHS, 2, D, D, dtype="bf16", seed=1500 + D + W, window=W,
                              S0_sd=0.3, halo=True)
    d_o, dS = packed_cotangents(vi, 1500 + D + W)
    g = run_packed(dev, vi, variant, d_o, dS, align=align)
    for n in range(len(LENGTHS)):
        a, b = int(vi.cu[n]), int(vi.cu[n + 1])
        s = vi.sequence(n).to_torch(dev)
        announce(f"chunk_bwd {variant} sequence {n} T{b - a}")
        r = fal.chunk_bwd(s["q"], s["k"], s["v"], s["alpha"], s["eta"],
                          to_dev(np.ascontiguousarray(d_o[None, :, a:b]), dev), variant,
                          dS_final=to_dev(dS[n:n + 1], dev), window=W, S0=s["S0"],
                          k_prev=s["k_prev"], v_prev=s["v_prev"], align=align)
        torch.cuda.synchronize()
        for k in GRADS:
            assert torch.equal(g[k][:, a:b], r[k][0]), (n, k)
        for k in ("dS0", "dk_prev", "dv_prev"):
            if g[k] is not None:
                assert torch.equal(g[k][n], r[k][0]), (n, k)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_varlen_bwd_matches_oracle(dev, case):
    variant, D, W = case
    vi = I.make_varlen_inputs(LENGTHS, 2, D, D, dtype="bf16", seed=1520 + D + W, window=W,
                              S0_sd=0.3, halo=True)
    d_o, dS = packed_cotangents(vi, 1520 + D + W)
    g = run_packed(dev, vi, variant, d_o, dS)
    got = {k: (None if v is None else to_np(v)) for k, v in g.items()}
    tol = TOL["bf16"]
    for n in (0, 3, 4):
        a, b = int(vi.cu[n]), int(vi.cu[n + 1])
        d = vi.sequence(n).f64()
        ref = G.gradients(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                          vi.sequence(n).widen(d_o[None, :, a:b]), dS[n:n + 1].astype(np.float64),
                          window=W, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"])
        for k, name, ax in (("dq", "q", (2, 3)), ("dk", "k", (2, 3)), ("dv", "v", (2, 3)),
                            ("dalpha", "alpha", (2,)), ("deta", "eta", (2,))):
            e = slice_rel_err(got[k][None, :, a:b], ref[name], ax)
            assert e <= tol, (n, k, e)
        assert slice_rel_err(got["dS0"][n:n + 1], ref["S0"], (2, 3)) <= tol, n


def test_varlen_bwd_leaves_other_rows(dev):
    """Rows outside every sequence keep what the output buffers held (the
    binding allocates zeros): one sequence over rows 0..39 of planes of 110."""
    import torch
    import weight_recurrent_sequence_amd as fal
    vi = I.make_varlen_inputs([40, 70], 2, 64, 64, dtype="bf16", seed=1540, S0_sd=0.2, halo=True)
    t = {n: to_dev(getattr(vi, n), dev) for n in ("q", "k", "v", "alpha", "eta")}
    d_o, dS = packed_cotangents(vi, 1540)
    cu = torch.from_numpy(np.array([0, 40], np.int32)).to(dev)
    announce("chunk_bwd_varlen F1 one sequence of 40 rows in planes of 110")
    g = fal.chunk_bwd_varlen(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, to_dev(d_o, dev),
                             "F1", max_seqlen=40, dS_final=to_dev(dS[:1], dev),
                             S0=to_dev(vi.S0[:1], dev), k_prev=to_dev(vi.k_prev[:1], dev))
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.any(g[k][:, :40].float()), k
        assert not torch.any(g[k][:, 40:].float()), k


@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("case", [("F1", 1), ("F3", 3)], ids=lambda c: "-".join(map(str, c)))
def test_varlen_bwd_feature_map_long_tail(dev, case, phi):
    """Packed planes longer than their sequences with a feature map: the
    mapped key and query copies live at per-(sequence, head) rows of the
    workspace, so a long tail (600 rows after two sequences of 40 and 70, H =
    3: the last head's plane rows lie past N * H * max_seqlen) stays inside
    it.  Gradients against the oracle per sequence; nothing past the
    workspace is written; the tail rows of the gradients are not written."""
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W = case
    L, H, tail = [40, 70], 3, 600
    vi = I.make_varlen_inputs(L, H, 128, 128, dtype="bf16", seed=1560 + W, window=W,
                              S0_sd=0.2, halo=True, tail=tail)
    d_o, dS = packed_cotangents(vi, 1560 + W)
    t = {n: to_dev(getattr(vi, n), dev) for n in ("q", "k", "v", "k_prev", "v_prev", "alpha",
                                                   "eta", "S0")}
    cu = torch.from_numpy(vi.cu).to(dev)
    N, maxT = len(L), max(L)
    need = fal.bwd_varlen_workspace_bytes(N, H, maxT, 128, 128, fal.BF16, variant, W, 64, phi=phi)
    guard = 1 << 20
    ws = torch.full((need + guard,), 0x5A, dtype=torch.uint8, device=dev)
    announce(f"chunk_bwd_varlen {variant} W{W} phi={phi} lengths {L} tail {tail} H{H}")
    g = fal.chunk_bwd_varlen(t["q"], t["k"], t["v"], t["alpha"], t["eta"], cu, to_dev(d_o, dev),
                             variant, max_seqlen=maxT, dS_final=to_dev(dS, dev), window=W,
                             S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"], phi=phi,
                             workspace=ws[:need])
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0x5A).all()), "the call wrote past its workspace"
    got = {k: (None if v is None else to_np(v)) for k, v in g.items()}
    for k in GRADS:
        assert not np.any(got[k][:, sum(L):]), k
    for n in range(N):
        a, b = int(vi.cu[n]), int(vi.cu[n + 1])
        d = vi.sequence(n).f64()
        ref = G.gradients(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                          vi.sequence(n).widen(d_o[None, :, a:b]), dS[n:n + 1].astype(np.float64),
                          window=W, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"], phi=phi)
        for k, name, ax in (("dq", "q", (2, 3)), ("dk", "k", (2, 3)), ("dv", "v", (2, 3)),
                            ("dalpha", "alpha", (2,)), ("deta", "eta", (2,))):
            e = slice_rel_err(got[k][None, :, a:b], ref[name], ax)
            assert e <= TOL["bf16"], (n, k, e)
