"""GPU parity of the feature maps (FALCON_PHI_L2, FALCON_PHI_SILU on keys and
queries) against the fp64 oracle's phi option: chunk forward (batched and
packed), continuation, and both decode steps."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, announce, ensure_built, slice_rel_err, to_np
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

ALL = ["F1", "F2", "F3", "F1A", "F2A", "F3A"]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def chunk_check(dev, inp, variant, W, chunk, phi, align="prefix"):
    import torch
    import weight_recurrent_sequence_amd as fal
    t = inp.to_torch(dev)
    B, H, T, D = inp.k.shape
    announce(f"chunk_fwd {variant} {inp.dtype} B{B} H{H} T{T} d{D} W{W} chunk{chunk} "
             f"phi={phi} align={align}")
    o, S = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, window=W,
                         chunk=chunk, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"],
                         align=align, phi=phi)
    torch.cuda.synchronize()
    d = inp.f64()
    o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                    window=W, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"],
                                    align=align, phi=phi)
    tol = TOL[inp.dtype]
    e_o = slice_rel_err(to_np(o), o_ref, (2, 3))
    e_S = slice_rel_err(to_np(S), S_ref, (2, 3))
    assert np.isfinite(to_np(o)).all()
    assert e_o <= tol and e_S <= tol, (e_o, e_S)


@pytest.mark.parametrize("cfg", [("bf16", 128, 64), ("bf16", 64, 16), ("fp32", 64, 32),
                                 ("fp32", 128, 16)], ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("variant", ALL)
def test_phi_chunk_grid(dev, variant, phi, cfg):
    dtype, D, chunk = cfg
    W = 3 if variant in ("F3", "F3A") else 1
    inp = I.make_chunk_inputs(2, 3, 150, D, D, dtype=dtype, seed=1100 + D + chunk, window=W,
                              halo=True, S0_sd=0.3)
    chunk_check(dev, inp, variant, W, chunk, phi)


@pytest.mark.parametrize("T", [1, 17, 65])
@pytest.mark.parametrize("case", [("F1", "l2", 1), ("F3", "silu", 4), ("F2A", "l2", 1)])
def test_phi_same_step_and_lengths(dev, case, T):
    variant, phi, W = case
    inp = I.make_chunk_inputs(1, 2, T, 128, 128, dtype="bf16", seed=1150 + T, window=W,
                              halo=True, S0_sd=0.2)
    chunk_check(dev, inp, variant, W, 64, phi, align="same")


@pytest.mark.parametrize("phi", ["l2", "silu"])
def test_phi_continuation(dev, phi):
    """Halos keep raw keys: two calls with a carried state and raw halo equal
    the oracle over the whole sequence."""
    import torch
    import weight_recurrent_sequence_amd as fal
    W = 3
    inp = I.make_chunk_inputs(1, 2, 200, 64, 64, dtype="fp32", seed=1160, window=W)
    t = inp.to_torch(dev)
    T1 = 90
    part = lambda a, lo, hi: a[:, :, lo:hi].contiguous()  # noqa: E731
    announce(f"chunk_fwd continuation F3 phi={phi}")
    o1, S1 = fal.chunk_fwd(*(part(t[x], 0, T1) for x in ("q", "k", "v", "alpha", "eta")), "F3",
                           window=W, chunk=32, phi=phi)
    o2, S2 = fal.chunk_fwd(*(part(t[x], T1, 200) for x in ("q", "k", "v", "alpha", "eta")), "F3",
                           window=W, chunk=32, S0=S1, k_prev=part(t["k"], T1 - W, T1),
                           v_prev=part(t["v"], T1 - W + 1, T1), phi=phi)
    torch.cuda.synchronize()
    d = inp.f64()
    o_ref, S_ref = oracle.recurrent("F3", d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=W,
                                    phi=phi)
    assert slice_rel_err(to_np(torch.cat([o1, o2], dim=2)), o_ref, (2, 3)) <= TOL["fp32"]
    assert slice_rel_err(to_np(S2), S_ref, (2, 3)) <= TOL["fp32"]


@pytest.mark.parametrize("case", [("F1", "l2"), ("F3", "silu")])
def test_phi_packed(dev, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, phi = case
    W = 2 if variant == "F3" else 1
    vi = I.make_varlen_inputs([70, 0, 1, 130], 2, 128, 128, dtype="bf16", seed=1170, window=W,
                              halo=True, S0_sd=0.2)
    td = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).view(  # noqa: E731
        torch.bfloat16).to(dev)
    tf = lambda a: None if a is None else torch.from_numpy(a).to(dev)  # noqa: E731
    announce(f"chunk_fwd_varlen {variant} phi={phi}")
    o, S = fal.chunk_fwd_varlen(td(vi.q), td(vi.k), td(vi.v), tf(vi.alpha), tf(vi.eta),
                                torch.from_numpy(vi.cu).to(dev), variant, window=W, chunk=64,
                                S0=tf(vi.S0), k_prev=td(vi.k_prev), v_prev=td(vi.v_prev), phi=phi)
    torch.cuda.synchronize()
    o_np, S_np = to_np(o), to_np(S)
    for n in range(4):
        d = vi.sequence(n).f64()
        o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                        window=W, S0=d["S0"], k_prev=d["k_prev"],
                                        v_prev=d["v_prev"], phi=phi)
        a, b = vi.cu[n], vi.cu[n + 1]
        if b > a:
            assert slice_rel_err(o_np[None, :, a:b], o_ref, (2, 3)) <= TOL["bf16"]
        assert slice_rel_err(S_np[n:n + 1], S_ref, (2, 3)) <= TOL["bf16"]


def tens(a, dtype, dev):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and a.dtype == np.uint16:
        x = x.view(torch.bfloat16)
    return x.to(dev)


@pytest.mark.parametrize("align", ["prefix", "same"])
@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("variant", ["F1", "F2A"])
def test_phi_decode(dev, variant, phi, align):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, D, steps, dtype = 3, 4, 128, 6, "bf16"
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=1180, S0_sd=0.1)
    S, kc = tens(di.S0, "fp32", dev), tens(di.k_cache0, dtype, dev)
    S_o, kc_o = di.S0.astype(np.float64), di.widen(di.k_cache0)[:, :, 0]
    for s in range(steps):
        announce(f"decode_step {variant} phi={phi} align={align} step {s}")
        o = fal.decode_step(S, kc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                            tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                            tens(di.eta[s], "fp32", dev), variant, align=align, phi=phi)
        o_ref, S_o, kc_o = oracle.decode_step(variant, S_o, kc_o, di.widen(di.q[s]),
                                              di.widen(di.k[s]), di.widen(di.v[s]), di.alpha[s],
                                              di.eta[s], align=align, phi=phi)
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= TOL[dtype]
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= TOL[dtype]
    np.testing.assert_array_equal(to_np(kc)[:, :, 0], kc_o)


@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_phi_decode_window(dev, variant, phi):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, D, W, steps, dtype = 3, 4, 64, 4, 6, "fp32"
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=1190, S0_sd=0.1, window=W)
    S, kc, vc = (tens(di.S0, "fp32", dev), tens(di.k_cache0, dtype, dev),
                 tens(di.v_cache0, dtype, dev))
    S_o, kc_o, vc_o = di.S0.astype(np.float64), di.widen(di.k_cache0), di.widen(di.v_cache0)
    for s in range(steps):
        announce(f"decode_step_window {variant} phi={phi} step {s}")
        o = fal.decode_step_window(S, kc, vc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                                   tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                                   tens(di.eta[s], "fp32", dev), variant, phi=phi)
        o_ref, S_o, kc_o, vc_o = oracle.decode_step_window(
            variant, S_o, kc_o, vc_o, di.widen(di.q[s]), di.widen(di.k[s]), di.widen(di.v[s]),
            di.alpha[s], di.eta[s], phi=phi)
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= TOL[dtype]
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= TOL[dtype]
    np.testing.assert_array_equal(to_np(kc), kc_o)
