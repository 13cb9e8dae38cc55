"""GPU parity of falcon_chunk_fwd on the method's pinned edge cases.

Each case mirrors a pin of the oracle (tests/test_oracle_pins.py) on the GPU:
the chunk form on the GPU is compared element by element with the fp64
recurrent oracle on the same stored bits, per (batch, head) slice
(max|gpu - oracle| / max|oracle|, acceptance 1e-4 for fp32 inputs and 2e-2
for bf16 inputs, fp32 state in both cases):

* decay only (eta = 0): the state only decays, S_t = gamma_t S0;
* constant strong decay alpha = 0.5 and near-one decay alpha = 1 - 1e-4 over
  8192 steps: the positive-decay renormalization ("Fast Weight Attention for
  Continual Learning", authors' abstract: stable renormalization of the
  products of decays) must keep every factor finite at any length;
* eps = 0 on nonzero keys (the halo keys make x_0 nonzero too);
* a zero key in the middle of the sequence (its pair writes nothing);
* keys scaled per (batch, token) by LogNormal(0, 1), the Falcon-2 workload's
  stress of the normalizers, here for every variant.

Each runs at bf16 / d = 128 / chunk 64 (the benchmark's configuration) and
at fp32 / d = 64 / chunk 32, for Falcon-1, -2, -3 (window 4) and the
inner-product variants.  Also here: the workspace is filled with NaN bytes
before each call and the result must equal, bit for bit, a run on a
zero-filled workspace (a kernel that reads a workspace byte it did not write
first would show it).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, announce, ensure_built, slice_rel_err, to_np
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

VARIANTS = [("F1", 1), ("F2", 1), ("F3", 4), ("F1A", 1), ("F2A", 1), ("F3A", 4)]
CONFIGS = [("bf16", 128, 64), ("fp32", 64, 32)]
CASES = ["eta0", "alpha_half", "alpha_near_one", "eps0", "zero_key", "lognormal_keys"]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def case_inputs(case, variant, W, dtype, D, seed):
    """Inputs of one edge case (B = 1, H = 2), with the eps it runs at."""
    T = 8192 if case in ("alpha_half", "alpha_near_one") else 700
    eps = 1e-6
    inp = I.make_chunk_inputs(1, 2, T, D, D, dtype=dtype, seed=seed, window=W,
                              key_lognormal=(case == "lognormal_keys"),
                              halo=(case == "eps0"), S0_sd=0.3)
    if case == "eta0":
        inp.eta[:] = 0.0
    elif case == "alpha_half":
        inp.alpha[:] = np.float32(0.5)
    elif case == "alpha_near_one":
        inp.alpha[:] = np.float32(1.0 - 1e-4)
    elif case == "eps0":
        eps = 0.0
    elif case == "zero_key":
        # k_300 = 0: the pair of step 301 (prefix-aligned; step 300 for
        # same-step pairs) has a zero key, and for a window it is one of W
        inp.k[:, :, 300, :] = 0
        inp.k[:, 1, 301:305, :] = 0  # and a run of them in the second head
    return inp, eps


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"{c[0]}-d{c[1]}-c{c[2]}")
@pytest.mark.parametrize("var", VARIANTS, ids=lambda v: v[0])
def test_edge_case(dev, var, cfg, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W = var
    dtype, D, chunk = cfg
    seed = 5000 + 17 * CASES.index(case) + D + W
    inp, eps = case_inputs(case, variant, W, dtype, D, seed)
    t = inp.to_torch(dev)
    B, H, T, _ = inp.k.shape
    announce(f"edge {case}: chunk_fwd {variant} W{W} {dtype} d{D} chunk{chunk} B{B} H{H} T{T} "
             f"eps={eps}")
    o, S = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, window=W,
                         chunk=chunk, eps=eps, S0=t["S0"], k_prev=t["k_prev"],
                         v_prev=t["v_prev"])
    torch.cuda.synchronize()
    d = inp.f64()
    o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                    window=W, eps=eps, S0=d["S0"], k_prev=d["k_prev"],
                                    v_prev=d["v_prev"])
    o_np, S_np = to_np(o), to_np(S)
    assert np.isfinite(o_ref).all() and np.isfinite(S_ref).all()
    assert np.isfinite(o_np).all() and np.isfinite(S_np).all()
    e_o = slice_rel_err(o_np, o_ref, (2, 3))
    e_S = slice_rel_err(S_np, S_ref, (2, 3))
    announce(f"edge {case} {variant} {dtype}: max rel err o={e_o:.2e} S={e_S:.2e}")
    tol = TOL[dtype]
    assert e_o <= tol and e_S <= tol, (e_o, e_S)
    if case == "eta0":
        # decay only: S_T = gamma_T S0 exactly up to the rounding of the decays
        g = np.exp(np.sum(np.log(d["alpha"]), axis=-1))
        np.testing.assert_allclose(S_np, g[..., None, None] * d["S0"], rtol=1e-4, atol=1e-30)


# ---- NaN-poisoned workspace --------------------------------------------------
POISON = [("F1", 1, "bf16", 128, 64), ("F2", 1, "bf16", 128, 64), ("F3", 4, "bf16", 128, 64),
          ("F1A", 1, "bf16", 128, 64), ("F2A", 1, "bf16", 64, 32), ("F3A", 4, "bf16", 128, 64),
          ("F3", 3, "bf16", 64, 16), ("F3A", 8, "bf16", 128, 64), ("F3", 2, "bf16", 128, 32),
          ("F1", 1, "fp32", 64, 32), ("F2", 1, "fp32", 128, 32), ("F3", 4, "fp32", 64, 16),
          ("F1A", 1, "fp32", 64, 64)]


def _ws_run(fal, t, variant, W, chunk, fill, phi="identity", align="prefix"):
    import torch
    B, H, T, D = t["k"].shape
    dt = fal.BF16 if t["k"].dtype == torch.bfloat16 else fal.FP32
    n = fal.workspace_bytes(B, H, T, D, D, dt, variant, W, chunk, phi=phi)
    ws = torch.full((max(n, 1),), fill, dtype=torch.uint8, device=t["k"].device)
    return fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, window=W,
                         chunk=chunk, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"],
                         workspace=ws, phi=phi, align=align)


@pytest.mark.parametrize("T", [1, 130, 333])
@pytest.mark.parametrize("case", POISON, ids=lambda c: "-".join(map(str, c)))
def test_poisoned_workspace(dev, case, T):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W, dtype, D, chunk = case
    inp = I.make_chunk_inputs(2, 2, T, D, D, dtype=dtype, seed=5300 + T + W, window=W,
                              halo=True, S0_sd=0.2)
    t = inp.to_torch(dev)
    announce(f"poisoned workspace: chunk_fwd {variant} W{W} {dtype} d{D} chunk{chunk} T{T}")
    o0, S0 = _ws_run(fal, t, variant, W, chunk, 0)
    oN, SN = _ws_run(fal, t, variant, W, chunk, 0xFF)  # 0xFFFF.. is a NaN in bf16 and fp32
    torch.cuda.synchronize()
    assert torch.isfinite(oN.float()).all() and torch.isfinite(SN).all()
    assert torch.equal(o0, oN) and torch.equal(S0, SN)


@pytest.mark.parametrize("with_s0", [True, False])
def test_poisoned_workspace_segments(dev, with_s0):
    """Falcon-3A chains of 64 tiles or more run in segments whose group
    states and copy of S0 live in the workspace: every byte read there is
    written first by the same call."""
    import torch
    import weight_recurrent_sequence_amd as fal
    inp = I.make_chunk_inputs(2, 2, 2100, 128, 128, dtype="bf16", seed=5390 + with_s0, window=4,
                              halo=True, S0_sd=0.2 if with_s0 else 0.0)
    t = inp.to_torch(dev)
    announce(f"poisoned workspace: chunk_fwd F3A W4 bf16 d128 chunk64 T2100 segments S0={with_s0}")
    o0, S0 = _ws_run(fal, t, "F3A", 4, 64, 0)
    oN, SN = _ws_run(fal, t, "F3A", 4, 64, 0xFF)
    torch.cuda.synchronize()
    assert torch.isfinite(oN.float()).all() and torch.isfinite(SN).all()
    assert torch.equal(o0, oN) and torch.equal(S0, SN)


@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("align", ["prefix", "same"])
def test_poisoned_workspace_feature_map(dev, phi, align):
    import torch
    import weight_recurrent_sequence_amd as fal
    for variant, W in (("F1", 1), ("F3", 3)):
        inp = I.make_chunk_inputs(2, 2, 150, 128, 128, dtype="bf16", seed=5400 + W, window=W,
                                  halo=True, S0_sd=0.2)
        t = inp.to_torch(dev)
        announce(f"poisoned workspace: chunk_fwd {variant} W{W} phi={phi} align={align}")
        o0, S0 = _ws_run(fal, t, variant, W, 64, 0, phi=phi, align=align)
        oN, SN = _ws_run(fal, t, variant, W, 64, 0xFF, phi=phi, align=align)
        torch.cuda.synchronize()
        assert torch.equal(o0, oN) and torch.equal(S0, SN)


def test_poisoned_workspace_varlen(dev):
    import torch
    import weight_recurrent_sequence_amd as fal
    for variant, W, chunk in (("F1", 1, 64), ("F2", 1, 64), ("F3A", 4, 64), ("F3", 2, 32)):
        vi = I.make_varlen_inputs([130, 0, 1, 63, 200], 3, 128, 128, dtype="bf16",
                                  seed=5500 + W, window=W, S0_sd=0.2, halo=True, tail=9)
        tv = {n: torch.from_numpy(getattr(vi, n)).view(torch.bfloat16).to(dev)
              for n in ("q", "k", "v", "k_prev") + (("v_prev",) if W > 1 else ())}
        g = {n: torch.from_numpy(getattr(vi, n)).to(dev) for n in ("alpha", "eta", "S0")}
        cu = torch.from_numpy(vi.cu).to(dev)
        n = fal.varlen_workspace_bytes(5, 3, 200, 128, 128, fal.BF16, variant, W, chunk)
        outs = []
        for fill in (0, 0xFF):
            ws = torch.full((n,), fill, dtype=torch.uint8, device=dev)
            announce(f"poisoned workspace: chunk_fwd_varlen {variant} W{W} chunk{chunk} fill {fill}")
            outs.append(fal.chunk_fwd_varlen(tv["q"], tv["k"], tv["v"], g["alpha"], g["eta"], cu,
                                             variant, max_seqlen=200, window=W, chunk=chunk,
                                             S0=g["S0"], k_prev=tv["k_prev"],
                                             v_prev=tv.get("v_prev"), workspace=ws,
                                             o=torch.zeros_like(tv["v"])))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("case", [("F1", 1), ("F1A", 1), ("F2", 1), ("F3", 4), ("F3A", 3)])
def test_poisoned_workspace_backward(dev, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W = case
    for T in (1, 200):
        inp = I.make_chunk_inputs(2, 2, T, 128, 128, dtype="bf16", seed=5600 + T + W, window=W,
                                  halo=True, S0_sd=0.2)
        t = inp.to_torch(dev)
        d_o, dS = I.make_cotangents(2, 2, T, 128, 128, seed=5600 + T)
        d_o = torch.from_numpy(d_o).view(torch.bfloat16).to(dev)
        dS = torch.from_numpy(dS).to(dev)
        n = fal.bwd_workspace_bytes(2, 2, T, 128, 128, fal.BF16, variant, W, 64)
        res = []
        for fill in (0, 0xFF):
            ws = torch.full((n,), fill, dtype=torch.uint8, device=dev)
            announce(f"poisoned workspace: chunk_bwd {variant} W{W} T{T} fill {fill}")
            res.append(fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant,
                                     dS_final=dS, window=W, S0=t["S0"], k_prev=t["k_prev"],
                                     v_prev=t["v_prev"], workspace=ws))
        torch.cuda.synchronize()
        for key in res[0]:
            if res[0][key] is not None:
                assert torch.equal(res[0][key], res[1][key]), (key, T)
