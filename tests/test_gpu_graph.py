"""Chunk calls captured as a HIP graph and replayed.

The library's calls only launch kernels on the caller's stream (no
allocation, memset, copy or synchronisation of their own), so a caller may
capture them.  Each test captures one call (or a forward-and-backward step)
once, then replays it several times with new inputs copied into the captured
tensors and eager calls run between the replays; every replay must leave the
outputs the eager call on the same inputs leaves, bit for bit (the kernels
are deterministic: no atomics and a fixed order of every sum)."""
import pytest

from tests.gpu_util import announce, ensure_built
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

B, H, T, D = 2, 2, 2048, 128


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def draw(dev, variant, W, seed, state):
    x = I.make_chunk_inputs(B, H, T, D, D, dtype="bf16", seed=seed, window=W,
                            key_lognormal=variant in ("F2", "F2A"),
                            S0_sd=0.02 if state else 0.0, halo=state)
    return {k: v for k, v in x.to_torch(dev).items() if v is not None}


def run_replays(dev, tag, sets, live, call, outs):
    """Capture call(live) once; replay it on each input set in turn (copied
    into `live`), with an eager call on another set between replays, and
    compare the graph's outputs `outs` with the eager results."""
    import torch
    refs = []
    for x in sets:
        got = call(x)
        torch.cuda.synchronize()
        refs.append([t.clone() for t in got])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(live)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    announce(f"{tag}: capturing")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = call(live)
    order = [0, 1, 0, 1]
    for rep, i in enumerate(order):
        for name, t in live.items():
            t.copy_(sets[i][name])
        torch.cuda.synchronize()
        announce(f"{tag}: replay {rep} (input set {i})")
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs(captured), refs[i])):
            assert torch.equal(a, b), (rep, i, j)
        # eager work between the replays, on the other set
        other = call(sets[1 - i])
        torch.cuda.synchronize()
        for a, b in zip(other, refs[1 - i]):
            assert torch.equal(a, b), (rep, "eager")


FWD_CASES = [("F1", 1, False), ("F1", 1, True), ("F1A", 1, False), ("F2", 1, True),
             ("F3", 4, True), ("F3A", 4, False), ("F3A", 4, True)]


@pytest.mark.parametrize("variant,W,state", FWD_CASES,
                         ids=[f"{v}-W{w}-{'state' if s else 'zero'}" for v, w, s in FWD_CASES])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_forward_replayed_from_a_graph(dev, variant, W, state, entry):
    """falcon_chunk_fwd (caller's workspace) and falcon_chunk_fwd_noalloc
    (built-in scratch): the split kernels (Falcon-1, -2), the fused kernel
    (Falcon-1A), the window forms (Falcon-3) and the segmented pass with its
    group-state kernel (Falcon-3A over 64 tiles), with and without a start
    state and halo."""
    import torch
    import weight_recurrent_sequence_amd as fal
    sets = [draw(dev, variant, W, 1700 + 10 * W + s, state) for s in range(2)]
    live = {k: v.clone() for k, v in sets[0].items()}
    o = torch.empty_like(live["v"])
    Sf = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(fal.workspace_bytes(B, H, T, D, D, fal.BF16, variant, W, 64), 1),
                     dtype=torch.uint8, device=dev)

    def call(x):
        eager = x is not live
        oo = torch.empty_like(o) if eager else o
        ss = torch.empty_like(Sf) if eager else Sf
        kw = dict(window=W, S0=x.get("S0"), k_prev=x.get("k_prev"), v_prev=x.get("v_prev"),
                  o=oo, S_final=ss)
        if entry == "noalloc":
            fal.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["eta"], variant, **kw)
        else:
            fal.chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["eta"], variant, workspace=ws,
                          **kw)
        return oo, ss

    run_replays(dev, f"forward {variant} W{W} {entry} state={state}", sets, live, call,
                lambda c: c)


@pytest.mark.parametrize("variant,W", [("F1", 1), ("F2A", 1), ("F3", 4)])
def test_training_step_replayed_from_a_graph(dev, variant, W):
    """falcon_chunk_fwd_save then falcon_chunk_bwd_saved, captured as one
    step: outputs, final state and every gradient."""
    import torch
    import weight_recurrent_sequence_amd as fal
    sets = []
    for s in range(2):
        x = draw(dev, variant, W, 1900 + 10 * W + s, True)
        d_o, dS = I.make_cotangents(B, H, T, D, D, dtype="bf16", seed=1950 + s)
        x["d_o"] = torch.from_numpy(d_o).view(torch.bfloat16).to(dev)
        x["dS_final"] = torch.from_numpy(dS).to(dev)
        sets.append(x)
    live = {k: v.clone() for k, v in sets[0].items()}
    saved = torch.empty(fal.bwd_workspace_bytes(B, H, T, D, D, fal.BF16, variant, W, 64),
                        dtype=torch.uint8, device=dev)
    keys = ("dq", "dk", "dv", "dalpha", "deta", "dS0", "dk_prev", "dv_prev")

    def call(x):
        kw = dict(window=W, S0=x["S0"], k_prev=x["k_prev"], v_prev=x.get("v_prev"))
        o, Sf = fal.chunk_fwd_save(x["q"], x["k"], x["v"], x["alpha"], x["eta"], variant,
                                   saved=saved, **kw)
        g = fal.chunk_bwd_saved(x["q"], x["k"], x["v"], x["alpha"], x["eta"], x["d_o"],
                                variant, saved=saved, dS_final=x["dS_final"], **kw)
        return [o, Sf] + [g[k] for k in keys if g.get(k) is not None]

    run_replays(dev, f"training step {variant} W{W}", sets, live, call, lambda c: c)
