"""GPU parity of falcon_decode_step and falcon_decode_step_window against the
fp64 oracle's decode steps.

Every step's output and the final state and key cache are compared per head
(max|gpu - oracle| / max|oracle|, 1e-4 for fp32 inputs, 2e-2 for bf16)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, announce, ensure_built, slice_rel_err, to_np
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def tens(a, dtype, dev):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and a.dtype == np.uint16:
        x = x.view(torch.bfloat16)
    return x.to(dev)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", ["F1", "F2", "F1A", "F2A"])
def test_decode_grid(dev, variant, dtype, D):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, steps = 3, 5, 12
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=600 + D, S0_sd=0.1)
    S = tens(di.S0, "fp32", dev)
    kc = tens(di.k_cache0, dtype, dev)
    S_o, kc_o = di.S0.astype(np.float64), di.widen(di.k_cache0)[:, :, 0]
    tol = TOL[dtype]
    for s in range(steps):
        announce(f"decode_step {variant} {dtype} N{N} H{H} d{D} step {s}")
        o = fal.decode_step(S, kc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                            tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                            tens(di.eta[s], "fp32", dev), variant)
        o_ref, S_o, kc_o = oracle.decode_step(variant, S_o, kc_o, di.widen(di.q[s]),
                                              di.widen(di.k[s]), di.widen(di.v[s]),
                                              di.alpha[s], di.eta[s])
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= tol
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= tol
    np.testing.assert_array_equal(to_np(kc)[:, :, 0], kc_o)


def test_decode_full_workload_sampled(dev):
    """256 sequences x 32 heads, d = 128, 1024 consecutive steps from
    N(0, 0.02^2) states, in the benchmark's launch configuration; the oracle
    follows a sample of heads through all 1024 steps."""
    import torch
    import weight_recurrent_sequence_amd as fal
    w = I.WORKLOADS["decode_falcon1_N256H32d128_1024steps"]
    N, H, D, steps = w["N"], w["H"], w["d"], w["steps"]
    x = I.make_decode_inputs_torch(N, H, D, D, steps, device=dev, seed=w["seed"])
    sample = [(0, 0), (17, 5), (128, 31), (255, 16)]
    ns = torch.tensor([n for n, _ in sample], device=dev)
    hs = torch.tensor([h for _, h in sample], device=dev)
    S = x["S0"].clone()
    kc = x["k_cache0"].clone()
    outs = torch.empty(steps, len(sample), D, dtype=torch.bfloat16, device=dev)
    announce("decode_step F1 bf16 N256 H32 d128, 1024 steps")
    for s in range(steps):
        o = fal.decode_step(S, kc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s], x["eta"][s],
                            "F1")
        outs[s] = o[ns, hs]
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    S_o = f64(x["S0"][ns, hs])[None]
    kc_o = f64(x["k_cache0"][ns, hs, 0])[None]
    o_ref = np.empty((steps, len(sample), D))
    for s in range(steps):
        o1, S_o, kc_o = oracle.decode_step("F1", S_o, kc_o, f64(x["q"][s][ns, hs])[None],
                                           f64(x["k"][s][ns, hs])[None],
                                           f64(x["v"][s][ns, hs])[None],
                                           f64(x["alpha"][s][ns, hs])[None],
                                           f64(x["eta"][s][ns, hs])[None])
        o_ref[s] = o1[0]
    e_o = slice_rel_err(np.moveaxis(to_np(outs), 0, 1), np.moveaxis(o_ref, 0, 1), (1, 2))
    e_S = slice_rel_err(to_np(S[ns, hs]), S_o[0], (1, 2))
    announce(f"decode full workload: max rel err o={e_o:.2e} S={e_S:.2e}")
    assert e_o <= TOL["bf16"] and e_S <= TOL["bf16"], (e_o, e_S)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_decode_window_grid(dev, variant, W, dtype, D):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, steps = 3, 4, 10
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=700 + 10 * W + D, S0_sd=0.1,
                              window=W)
    S = tens(di.S0, "fp32", dev)
    kc = tens(di.k_cache0, dtype, dev)
    vc = tens(di.v_cache0, dtype, dev) if W > 1 else None
    S_o, kc_o, vc_o = di.S0.astype(np.float64), di.widen(di.k_cache0), di.widen(di.v_cache0)
    tol = TOL[dtype]
    for s in range(steps):
        announce(f"decode_step_window {variant} W{W} {dtype} N{N} H{H} d{D} step {s}")
        o = fal.decode_step_window(S, kc, vc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                                   tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                                   tens(di.eta[s], "fp32", dev), variant)
        o_ref, S_o, kc_o, vc_o = oracle.decode_step_window(
            variant, S_o, kc_o, vc_o, di.widen(di.q[s]), di.widen(di.k[s]), di.widen(di.v[s]),
            di.alpha[s], di.eta[s])
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= tol
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= tol
    # the caches only move values: bit-exact
    np.testing.assert_array_equal(to_np(kc), kc_o)
    if W > 1:
        np.testing.assert_array_equal(to_np(vc), vc_o)


def test_decode_window_continues_a_chunk_call(dev):
    """A Falcon-3 chunk call over T tokens followed by decode steps equals one
    chunk call over all tokens: the caches are the chunk call's halo reversed
    (newest first)."""
    import torch
    import weight_recurrent_sequence_amd as fal
    B, H, T, D, W, extra = 1, 3, 40, 64, 4, 6
    inp = I.make_chunk_inputs(B, H, T + extra, D, D, dtype="fp32", seed=77, window=W)
    t = inp.to_torch(dev)
    sl = lambda a, lo, hi: a[:, :, lo:hi].contiguous()  # noqa: E731
    announce("decode_step_window continues chunk_fwd F3 W4 fp32")
    o_all, S_all = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F3", window=W,
                                 chunk=16, return_state=True)
    _, S_T = fal.chunk_fwd(sl(t["q"], 0, T), sl(t["k"], 0, T), sl(t["v"], 0, T),
                           sl(t["alpha"], 0, T), sl(t["eta"], 0, T), "F3", window=W, chunk=16,
                           return_state=True)
    kc = t["k"][:, :, T - W:T].flip(2).contiguous()          # k_{T-1} .. k_{T-W}
    vc = t["v"][:, :, T - W + 1:T].flip(2).contiguous()      # v_{T-1} .. v_{T-W+1}
    S = S_T.contiguous()
    for s in range(T, T + extra):
        o = fal.decode_step_window(S, kc, vc, t["q"][:, :, s].contiguous(),
                                   t["k"][:, :, s].contiguous(), t["v"][:, :, s].contiguous(),
                                   t["alpha"][:, :, s].contiguous(), t["eta"][:, :, s].contiguous(),
                                   "F3")
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), to_np(o_all[:, :, s]), (2,)) <= 1e-4
    assert slice_rel_err(to_np(S), to_np(S_all), (2, 3)) <= 1e-4


@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_decode_window_full_workload_sampled(dev, variant):
    """256 sequences x 32 heads, d = 128, window 4, 1024 consecutive steps in
    the benchmark's launch configuration; the oracle follows a sample of heads
    through every step, caches included."""
    import torch
    import weight_recurrent_sequence_amd as fal
    w = I.WORKLOADS["decode_falcon3_w4_N256H32d128_1024steps"]
    N, H, D, W, steps = w["N"], w["H"], w["d"], w["window"], w["steps"]
    x = I.make_decode_inputs_torch(N, H, D, D, steps, device=dev, seed=w["seed"], window=W)
    sample = [(0, 0), (77, 9), (200, 31), (255, 30)]
    ns = torch.tensor([n for n, _ in sample], device=dev)
    hs = torch.tensor([h for _, h in sample], device=dev)
    S, kc, vc = x["S0"].clone(), x["k_cache0"].clone(), x["v_cache0"].clone()
    outs = torch.empty(steps, len(sample), D, dtype=torch.bfloat16, device=dev)
    announce(f"decode_step_window {variant} W{W} bf16 N{N} H{H} d{D}, {steps} steps")
    for s in range(steps):
        o = fal.decode_step_window(S, kc, vc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                                   x["eta"][s], variant)
        outs[s] = o[ns, hs]
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    S_o = f64(x["S0"][ns, hs])[None]
    kc_o = f64(x["k_cache0"][ns, hs])[None]
    vc_o = f64(x["v_cache0"][ns, hs])[None]
    o_ref = np.empty((steps, len(sample), D))
    for s in range(steps):
        o1, S_o, kc_o, vc_o = oracle.decode_step_window(
            variant, S_o, kc_o, vc_o, f64(x["q"][s][ns, hs])[None], f64(x["k"][s][ns, hs])[None],
            f64(x["v"][s][ns, hs])[None], f64(x["alpha"][s][ns, hs])[None],
            f64(x["eta"][s][ns, hs])[None])
        o_ref[s] = o1[0]
    e_o = slice_rel_err(np.moveaxis(to_np(outs), 0, 1), np.moveaxis(o_ref, 0, 1), (1, 2))
    e_S = slice_rel_err(to_np(S[ns, hs]), S_o[0], (1, 2))
    announce(f"decode window full workload {variant}: max rel err o={e_o:.2e} S={e_S:.2e}")
    assert e_o <= TOL["bf16"] and e_S <= TOL["bf16"], (e_o, e_S)
    np.testing.assert_array_equal(f64(kc[ns, hs]), kc_o[0])
    np.testing.assert_array_equal(f64(vc[ns, hs]), vc_o[0])



# ---- same-step pairs: x = k_t (the new key), caches as in the prefix form ----
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", ["F1", "F2", "F1A", "F2A"])
def test_same_step_decode(dev, variant, dtype):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, D, steps = 3, 4, 128, 8
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=800, S0_sd=0.1)
    S, kc = tens(di.S0, "fp32", dev), tens(di.k_cache0, dtype, dev)
    S_o, kc_o = di.S0.astype(np.float64), di.widen(di.k_cache0)[:, :, 0]
    for s in range(steps):
        announce(f"decode_step same-step {variant} {dtype} step {s}")
        o = fal.decode_step(S, kc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                            tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                            tens(di.eta[s], "fp32", dev), variant, align="same")
        o_ref, S_o, kc_o = oracle.decode_step(variant, S_o, kc_o, di.widen(di.q[s]),
                                              di.widen(di.k[s]), di.widen(di.v[s]),
                                              di.alpha[s], di.eta[s], align="same")
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= TOL[dtype]
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= TOL[dtype]
    np.testing.assert_array_equal(to_np(kc)[:, :, 0], kc_o)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [1, 2, 4, 8])
@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_same_step_decode_window(dev, variant, W, D):
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, steps, dtype = 3, 4, 8, "bf16"
    di = I.make_decode_inputs(N, H, D, D, steps, dtype=dtype, seed=810 + W + D, S0_sd=0.1,
                              window=W)
    S, kc = tens(di.S0, "fp32", dev), tens(di.k_cache0, dtype, dev)
    vc = tens(di.v_cache0, dtype, dev) if W > 1 else None
    S_o, kc_o, vc_o = di.S0.astype(np.float64), di.widen(di.k_cache0), di.widen(di.v_cache0)
    for s in range(steps):
        announce(f"decode_step_window same-step {variant} W{W} d{D} step {s}")
        o = fal.decode_step_window(S, kc, vc, tens(di.q[s], dtype, dev), tens(di.k[s], dtype, dev),
                                   tens(di.v[s], dtype, dev), tens(di.alpha[s], "fp32", dev),
                                   tens(di.eta[s], "fp32", dev), variant, align="same")
        o_ref, S_o, kc_o, vc_o = oracle.decode_step_window(
            variant, S_o, kc_o, vc_o, di.widen(di.q[s]), di.widen(di.k[s]), di.widen(di.v[s]),
            di.alpha[s], di.eta[s], align="same")
        torch.cuda.synchronize()
        assert slice_rel_err(to_np(o), o_ref, (2,)) <= TOL[dtype]
    assert slice_rel_err(to_np(S), S_o, (2, 3)) <= TOL[dtype]
    np.testing.assert_array_equal(to_np(kc), kc_o)
    if W > 1:
        np.testing.assert_array_equal(to_np(vc), vc_o)


@pytest.mark.parametrize("W", [1, 4])
def test_decode_steps_replayed_from_a_graph(dev, W):
    """The decode steps captured once as a HIP graph (as bench.py times them):
    three replays, each from the initial state with eager steps run between
    them, leave the state, caches and last output the eager steps leave, bit
    for bit."""
    import torch
    import weight_recurrent_sequence_amd as fal
    N, H, D, steps = 4, 3, 128, 16
    variant = "F3" if W > 1 else "F1"
    x = I.make_decode_inputs_torch(N, H, D, D, steps, device=dev, seed=690 + W, window=W)
    S = x["S0"].clone()
    kc = x["k_cache0"].clone()
    vc = x["v_cache0"].clone() if W > 1 else None
    o = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)

    def step(s):
        if W > 1:
            fal.decode_step_window(S, kc, vc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                                   x["eta"][s], variant, o=o)
        else:
            fal.decode_step(S, kc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s], x["eta"][s],
                            variant, o=o)

    def reset():
        S.copy_(x["S0"])
        kc.copy_(x["k_cache0"])
        if vc is not None:
            vc.copy_(x["v_cache0"])
        torch.cuda.synchronize()

    announce(f"decode {variant} W{W} N{N} H{H} d{D}: {steps} eager steps")
    reset()
    for s in range(steps):
        step(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (S, kc, o) + ((vc,) if vc is not None else ())]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    reset()
    announce(f"decode {variant} W{W}: capturing {steps} steps")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(steps):
            step(s)
    for rep in range(3):
        reset()
        announce(f"decode {variant} W{W}: graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (S, kc, o) + ((vc,) if vc is not None else ())]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
        # eager work between the replays
        reset()
        step(0)
        torch.cuda.synchronize()
