"""GPU parity of falcon_chunk_fwd against the fp64 oracle (recurrent form).

Acceptance (per (batch, head) slice): max|gpu - oracle| / max|oracle| <= 1e-4
for fp32 inputs, <= 2e-2 for bf16 inputs, for the outputs o and the final
state; fp32 state in both cases.  Inputs are seeded and synthetic; the oracle
consumes the very same stored bits.
"""
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


def gpu_run(dev, inp, variant, W, chunk, eps=1e-6, label="", align="prefix"):
    import torch
    import weight_recurrent_sequence_amd as fal
    t = inp.to_torch(dev)
    B, H, T, D = inp.k.shape
    announce(f"chunk_fwd {variant} {inp.dtype} B{B} H{H} T{T} d{D} W{W} chunk{chunk} "
             f"align={align} {label}")
    o, S = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant, window=W,
                         chunk=chunk, eps=eps, S0=t["S0"], k_prev=t["k_prev"],
                         v_prev=t["v_prev"], align=align)
    torch.cuda.synchronize()
    return o, S


def oracle_run(inp, variant, W, eps=1e-6, sl=None, align="prefix"):
    d = inp.f64(sl)
    return oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"], window=W,
                            eps=eps, S0=d["S0"], k_prev=d["k_prev"], v_prev=d["v_prev"],
                            align=align)


def check(dev, inp, variant, W, chunk, label="", align="prefix"):
    o, S = gpu_run(dev, inp, variant, W, chunk, label=label, align=align)
    o_ref, S_ref = oracle_run(inp, variant, W, align=align)
    e_o = slice_rel_err(to_np(o), o_ref, (2, 3))
    e_S = slice_rel_err(to_np(S), S_ref, (2, 3))
    tol = TOL[inp.dtype]
    assert np.isfinite(to_np(o)).all()
    assert e_o <= tol and e_S <= tol, (e_o, e_S)
    return e_o, e_S


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", ALL)
def test_grid(dev, variant, dtype, D, chunk):
    W = 3 if variant in ("F3", "F3A") else 1
    inp = I.make_chunk_inputs(2, 3, 150, D, D, dtype=dtype, seed=100 + D + chunk, window=W,
                              halo=True, S0_sd=0.3)
    check(dev, inp, variant, W, chunk)


@pytest.mark.parametrize("T", [192, 193, 450, 777])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("variant", ["F1A", "F2A"])
def test_fused_steady_state(dev, variant, D, T):
    """The fused inner-product kernel past its prologue: 3 to 13 tiles, so
    the key fills of the main loop (and, for the per-column rule, the keys
    turned into write vectors in LDS from tile 2 on) are exercised, with a
    start state, a halo key and LogNormal key scales for Falcon-2A."""
    inp = I.make_chunk_inputs(2, 2, T, D, D, dtype="bf16", seed=300 + T + D, halo=True,
                              S0_sd=0.3, key_lognormal=variant == "F2A")
    check(dev, inp, variant, 1, 64, label="fused steady state")
    check(dev, inp, variant, 1, 64, label="fused steady state, same-step", align="same")


@pytest.mark.parametrize("T", [0, 1, 2, 15, 16, 17, 63, 64, 65, 129])
@pytest.mark.parametrize("case", [("F1", "bf16", 128, 64, 1), ("F3", "bf16", 128, 64, 4),
                                  ("F2", "fp32", 64, 32, 1), ("F1A", "bf16", 64, 16, 1)])
def test_lengths(dev, case, T):
    variant, dtype, D, chunk, W = case
    inp = I.make_chunk_inputs(1, 2, T, D, D, dtype=dtype, seed=200 + T, window=W, S0_sd=0.2)
    if T == 0:
        o, S = gpu_run(dev, inp, variant, W, chunk, label="T=0")
        np.testing.assert_array_equal(to_np(S), inp.S0.astype(np.float64))
        return
    check(dev, inp, variant, W, chunk)


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("variant", ["F3", "F3A"])
def test_windows(dev, variant, W, chunk):
    inp = I.make_chunk_inputs(1, 3, 100, 64, 64, dtype="bf16", seed=300 + W, window=W,
                              halo=True)
    check(dev, inp, variant, W, chunk)


# ---- same-step pairs (k_t, v_t), the KLA / gated-delta-rule alignment ----
@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", ALL)
def test_same_step_grid(dev, variant, dtype, D, chunk):
    W = 3 if variant in ("F3", "F3A") else 1
    inp = I.make_chunk_inputs(2, 3, 150, D, D, dtype=dtype, seed=600 + D + chunk, window=W,
                              halo=True, S0_sd=0.3)
    check(dev, inp, variant, W, chunk, align="same")


@pytest.mark.parametrize("T", [1, 2, 17, 64, 65, 130])
@pytest.mark.parametrize("case", [("F1", "bf16", 128, 64, 1), ("F3", "bf16", 128, 64, 4),
                                  ("F3A", "bf16", 64, 16, 8), ("F2", "fp32", 64, 32, 1)])
def test_same_step_lengths(dev, case, T):
    variant, dtype, D, chunk, W = case
    inp = I.make_chunk_inputs(1, 2, T, D, D, dtype=dtype, seed=700 + T, window=W, halo=True,
                              S0_sd=0.2)
    check(dev, inp, variant, W, chunk, align="same")


def test_same_step_differs_from_prefix(dev):
    """The flag reaches the kernels: the two alignments give different outputs."""
    inp = I.make_chunk_inputs(1, 2, 100, 64, 64, dtype="fp32", seed=710)
    o1, _ = gpu_run(dev, inp, "F1", 1, 32)
    o2, _ = gpu_run(dev, inp, "F1", 1, 32, align="same")
    assert np.abs(to_np(o1) - to_np(o2)).max() > 1e-2


@pytest.mark.parametrize("variant", ALL)
def test_continuation(dev, variant):
    """Two calls with carried state and halo equal one call (and the oracle)."""
    import torch
    import weight_recurrent_sequence_amd as fal
    W = 4 if variant in ("F3", "F3A") else 1
    inp = I.make_chunk_inputs(2, 2, 300, 128, 128, dtype="bf16", seed=400, window=W)
    t = inp.to_torch(dev)
    T1 = 130
    announce(f"chunk_fwd continuation {variant} T=300 split {T1}")
    o1, S1 = fal.chunk_fwd(*(t[x][:, :, :T1].contiguous() for x in ("q", "k", "v", "alpha",
                                                                        "eta")),
                           variant, window=W, chunk=64)
    kp = t["k"][:, :, T1 - W:T1].contiguous()
    vp = t["v"][:, :, T1 - W + 1:T1].contiguous() if W > 1 else None
    o2, S2 = fal.chunk_fwd(*(t[x][:, :, T1:].contiguous() for x in ("q", "k", "v", "alpha",
                                                                       "eta")),
                           variant, window=W, chunk=64, S0=S1, k_prev=kp, v_prev=vp)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_run(inp, variant, W)
    o = torch.cat([o1, o2], dim=2)
    assert slice_rel_err(to_np(o), o_ref, (2, 3)) <= TOL["bf16"]
    assert slice_rel_err(to_np(S2), S_ref, (2, 3)) <= TOL["bf16"]


def test_deterministic_and_state_alias(dev):
    import torch
    import weight_recurrent_sequence_amd as fal
    inp = I.make_chunk_inputs(2, 4, 257, 128, 128, dtype="bf16", seed=500, S0_sd=0.3)
    t = inp.to_torch(dev)
    announce("chunk_fwd determinism F2 B2 H4 T257")
    runs = [fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F2", S0=t["S0"])
            for _ in range(2)]
    S_alias = t["S0"].clone()
    o3, _ = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F2", S0=S_alias,
                          S_final=S_alias)
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    assert torch.equal(o3, runs[0][0]) and torch.equal(S_alias, runs[0][1])


def test_fp32_d128_chunk64_full_tiles(dev):
    """fp32 inputs at d = 128 with 64-row tiles (the support matrix's largest
    fp32 tile): several full tiles and a ragged tail, every variant."""
    for variant in ALL:
        W = 4 if variant in ("F3", "F3A") else 1
        inp = I.make_chunk_inputs(1, 2, 333, 128, 128, dtype="fp32", seed=530 + W, window=W,
                                  halo=True, S0_sd=0.3)
        check(dev, inp, variant, W, 64, label="fp32 d128 chunk64")


# ---- the workloads at full size, in the launch configuration the benchmark
# times; the oracle recomputes every (batch, head) sequence in full ----
FULL = [
    ("falcon1_fp32_B1H1T256d64", "F1"),
    ("falcon1_bf16_B8H16T4096d128", "F1"),
    ("falcon1_bf16_B8H16T4096d128", "F1A"),
    ("falcon2_bf16_B4H32T8192d128", "F2"),
    ("falcon2_bf16_B4H32T8192d128", "F2A"),
    ("falcon3_w4_bf16_B2H16T32768d128", "F3"),
    ("falcon3_w4_bf16_B2H16T32768d128", "F3A"),
    ("falcon1_bf16_B8H16T4096d128", "F1@same"),
    ("falcon3_w4_bf16_B2H16T32768d128", "F3@same"),
]


@pytest.mark.parametrize("name,variant", FULL, ids=[f"{n}-{v}" for n, v in FULL])
def test_full_workloads_every_head(dev, name, variant):
    variant, _, align = variant.partition("@")
    align = align or "prefix"
    w = I.WORKLOADS[name]
    W = w.get("window", 1)
    inp = I.workload_inputs(name)
    o, S = gpu_run(dev, inp, variant, W, w["chunk"], label=name, align=align)
    o_np, S_np = to_np(o), to_np(S)
    del o, S
    assert np.isfinite(o_np).all() and np.isfinite(S_np).all()
    tol = TOL[inp.dtype]
    d = inp.f64()
    o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                    window=W, align=align)
    del d
    e_o = slice_rel_err(o_np, o_ref, (2, 3))
    e_S = slice_rel_err(S_np, S_ref, (2, 3))
    announce(f"{name} {variant}: max rel err o={e_o:.2e} S={e_S:.2e} over all "
             f"{w['B'] * w['H']} (batch, head) sequences")
    assert e_o <= tol and e_S <= tol, (e_o, e_S)


@pytest.mark.parametrize("case", [(2048, 128, 4), (2049, 64, 2), (3000, 128, 3), (4100, 128, 8),
                                  (12805, 64, 4)],
                         ids=lambda c: "-".join(map(str, c)))
def test_window_inner_product_segments(dev, case):
    """Falcon-3A chains of 64 tiles (2048 steps) or more run as up to four
    segments at once, each starting from the state at its first tile, formed
    from groups of 32 tiles before it: two segments at T = 2048 and 2049,
    three at 3000 and 4100 (a ragged last segment), four at 12805.  S0 and
    halos are set."""
    T, D, W = case
    inp = I.make_chunk_inputs(1, 2, T, D, D, dtype="bf16", seed=5100 + T + W, window=W, halo=True,
                              S0_sd=0.3)
    check(dev, inp, "F3A", W, 64, label="segments")


@pytest.mark.parametrize("case", [(4100, 128, 4), (2049, 64, 3)], ids=lambda c: "-".join(map(str, c)))
def test_window_inner_product_segments_same_step(dev, case):
    """Same-step pairs (k_t, v_t) through the segmented pass: the group
    kernel and the segments read each pair's key at the same lag."""
    T, D, W = case
    inp = I.make_chunk_inputs(1, 2, T, D, D, dtype="bf16", seed=5150 + T + W, window=W, halo=True,
                              S0_sd=0.3)
    check(dev, inp, "F3A", W, 64, label="segments", align="same")


def test_window_inner_product_segments_deterministic(dev):
    """The segmented chains give the same bits on every call."""
    import torch
    inp = I.make_chunk_inputs(2, 2, 4100, 128, 128, dtype="bf16", seed=5190, window=4, halo=True,
                              S0_sd=0.3)
    o1, S1 = gpu_run(dev, inp, "F3A", 4, 64, label="segments, call 1")
    o2, S2 = gpu_run(dev, inp, "F3A", 4, 64, label="segments, call 2")
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_window_inner_product_segments_state_alias(dev):
    """S_final may alias S0: the segmented pass's workgroups read S0 only
    through the copy the group kernel makes before them, so an aliased call
    gives the same bits as a separate one."""
    import torch
    import weight_recurrent_sequence_amd as fal
    inp = I.make_chunk_inputs(2, 2, 4100, 128, 128, dtype="bf16", seed=5195, window=4, halo=True,
                              S0_sd=0.3)
    o1, S1 = gpu_run(dev, inp, "F3A", 4, 64, label="segments, S_final separate")
    t = inp.to_torch(dev)
    S_alias = t["S0"].clone()
    announce("chunk_fwd F3A bf16 B2 H2 T4100 d128 W4 chunk64 segments, S_final = S0")
    o2, _ = fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F3A", window=4, chunk=64,
                          S0=S_alias, k_prev=t["k_prev"], v_prev=t["v_prev"], S_final=S_alias)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S_alias)
