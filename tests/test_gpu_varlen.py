"""GPU parity of falcon_chunk_fwd_varlen (packed sequences of different
lengths) against the fp64 oracle run on each sequence on its own, and
against one batched falcon_chunk_fwd call per sequence (bitwise: the same
kernels do the same arithmetic on each sequence)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, announce, ensure_built, slice_rel_err, to_np
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

# lengths mixing empty, single-step, ragged and several-tile sequences
LENGTHS = [130, 0, 1, 63, 200, 64, 17]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


def to_dev(a, dtype, dev):
    import torch
    if a is None:
        return None
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16" and a.dtype == np.uint16:
        x = x.view(torch.bfloat16)
    return x.to(dev)


def run_varlen(dev, vi, variant, chunk, align="prefix", o_fill=None):
    import torch
    import weight_recurrent_sequence_amd as fal
    t = {n: to_dev(getattr(vi, n), vi.dtype, dev) for n in ("q", "k", "v", "k_prev", "v_prev")}
    g = {n: to_dev(getattr(vi, n), "fp32", dev) for n in ("alpha", "eta", "S0")}
    cu = torch.from_numpy(vi.cu).to(dev)
    o = None
    if o_fill is not None:
        o = torch.full(t["v"].shape, o_fill, dtype=t["v"].dtype, device=dev)
    announce(f"chunk_fwd_varlen {variant} {vi.dtype} H{vi.k.shape[0]} lengths "
             f"{np.diff(vi.cu).tolist()} W{vi.window} chunk{chunk} align={align}")
    o, S = fal.chunk_fwd_varlen(t["q"], t["k"], t["v"], g["alpha"], g["eta"], cu, variant,
                                window=vi.window, chunk=chunk, S0=g["S0"], k_prev=t["k_prev"],
                                v_prev=t["v_prev"], o=o, align=align)
    torch.cuda.synchronize()
    return o, S


CASES = [("F1", "bf16", 128, 64, 1), ("F2", "bf16", 128, 64, 1), ("F3", "bf16", 128, 64, 3),
         ("F1A", "bf16", 64, 32, 1), ("F3A", "bf16", 64, 16, 4), ("F1", "fp32", 64, 32, 1),
         ("F3", "fp32", 64, 16, 2)]


@pytest.mark.parametrize("align", ["prefix", "same"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_varlen_matches_oracle_per_sequence(dev, case, align):
    variant, dtype, D, chunk, W = case
    vi = I.make_varlen_inputs(LENGTHS, 3, D, D, dtype=dtype, seed=900 + D + W, window=W,
                              S0_sd=0.3, halo=True)
    o, S = run_varlen(dev, vi, variant, chunk, align=align)
    o_np, S_np = to_np(o), to_np(S)
    tol = TOL[dtype]
    for n in range(len(LENGTHS)):
        d = vi.sequence(n).f64()
        o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                        window=W, S0=d["S0"], k_prev=d["k_prev"],
                                        v_prev=d["v_prev"], align=align)
        a, b = vi.cu[n], vi.cu[n + 1]
        if b > a:
            assert slice_rel_err(o_np[None, :, a:b], o_ref, (2, 3)) <= tol, n
        assert slice_rel_err(S_np[n:n + 1], S_ref, (2, 3)) <= tol, n


@pytest.mark.parametrize("case", CASES[:3] + CASES[5:6], ids=lambda c: "-".join(map(str, c)))
def test_varlen_equals_one_call_per_sequence(dev, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, dtype, D, chunk, W = case
    vi = I.make_varlen_inputs(LENGTHS, 2, D, D, dtype=dtype, seed=950 + D, window=W,
                              S0_sd=0.2, halo=True)
    o, S = run_varlen(dev, vi, variant, chunk)
    for n in range(len(LENGTHS)):
        t = vi.sequence(n).to_torch(dev)
        on, Sn = fal.chunk_fwd(*(t[x].contiguous() for x in ("q", "k", "v", "alpha", "eta")),
                               variant, window=W, chunk=chunk, S0=t["S0"], k_prev=t["k_prev"],
                               v_prev=t["v_prev"])
        torch.cuda.synchronize()
        a, b = int(vi.cu[n]), int(vi.cu[n + 1])
        assert torch.equal(o[:, a:b], on[0]), n
        assert torch.equal(S[n], Sn[0]), n


def test_varlen_window_inner_product_segments(dev):
    """Falcon-3A packed calls whose longest sequence has 64 tiles or more run
    every sequence's chain in segments: long ones split, a one-tile and an
    empty sequence leave the later segments empty."""
    lengths = [2100, 0, 33, 4100, 700]
    vi = I.make_varlen_inputs(lengths, 2, 128, 128, dtype="bf16", seed=990, window=4, S0_sd=0.3,
                              halo=True)
    o, S = run_varlen(dev, vi, "F3A", 64)
    o_np, S_np = to_np(o), to_np(S)
    for n in range(len(lengths)):
        d = vi.sequence(n).f64()
        o_ref, S_ref = oracle.recurrent("F3A", d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                        window=4, S0=d["S0"], k_prev=d["k_prev"],
                                        v_prev=d["v_prev"])
        a, b = vi.cu[n], vi.cu[n + 1]
        if b > a:
            assert slice_rel_err(o_np[None, :, a:b], o_ref, (2, 3)) <= TOL["bf16"], n
        assert slice_rel_err(S_np[n:n + 1], S_ref, (2, 3)) <= TOL["bf16"], n


def test_varlen_leaves_rows_outside_sequences(dev):
    """Rows after the last sequence belong to none and are not written."""
    vi = I.make_varlen_inputs([40, 70], 2, 64, 64, dtype="bf16", seed=970, tail=33)
    o, _ = run_varlen(dev, vi, "F1", 32, o_fill=7.0)
    tail = to_np(o)[:, 110:]
    assert tail.shape[1] == 33 and np.all(tail == 7.0)


def test_varlen_full_size_sampled(dev):
    """A Falcon-1 packed batch as large as the B8 H16 T4096 workload (32768
    tokens per head), 16 sequences of mixed lengths, checked on a sample."""
    r = np.random.default_rng(5)
    lengths = r.integers(256, 3840, 15).tolist()
    lengths.append(32768 - sum(lengths))
    vi = I.make_varlen_inputs(lengths, 16, 128, 128, dtype="bf16", seed=980)
    o, S = run_varlen(dev, vi, "F1", 64)
    o_np, S_np = to_np(o), to_np(S)
    assert np.isfinite(o_np).all() and np.isfinite(S_np).all()
    for n in (0, 7, 15):
        d = vi.sequence(n).f64()
        heads = np.array([0, 9, 15])
        sl = lambda x: x[:, heads]  # noqa: E731
        o_ref, S_ref = oracle.recurrent("F1", sl(d["q"]), sl(d["k"]), sl(d["v"]),
                                        sl(d["alpha"]), sl(d["eta"]))
        a, b = vi.cu[n], vi.cu[n + 1]
        e_o = slice_rel_err(o_np[None, heads, a:b], o_ref, (2, 3))
        e_S = slice_rel_err(S_np[n:n + 1, heads], S_ref, (2, 3))
        announce(f"varlen full size seq {n} (T={b - a}): o {e_o:.2e} S {e_S:.2e}")
        assert e_o <= TOL["bf16"] and e_S <= TOL["bf16"]


# A packed plane longer than its sequences (a fixed-capacity buffer): rows
# after the last sequence belong to none.  With a feature map the intra-chunk
# kernel writes mapped copies of the keys and queries into the workspace; the
# plane is laid out so that head h's rows start at h * total_T, which for
# H >= 2 reaches beyond N * H * max_seqlen rows, the room the workspace has
# for them: the copies must be addressed per (sequence, head) instead.
TAIL_CASE = dict(lengths=[40, 70], H=3, tail=600)


def test_tail_shape_exceeds_plane_rows():
    """CPU check that the case below is the one that needs per-(sequence,
    head) rows: the last head's rows of the plane lie past the workspace's
    N * H * max_seqlen mapped rows."""
    L, H, tail = TAIL_CASE["lengths"], TAIL_CASE["H"], TAIL_CASE["tail"]
    total_T, N, max_seqlen = sum(L) + tail, len(L), max(L)
    assert (H - 1) * total_T + sum(L) > N * H * max_seqlen


@pytest.mark.parametrize("phi", ["l2", "silu"])
@pytest.mark.parametrize("case", [("F1", 1, 64), ("F3", 3, 32), ("F2A", 1, 64)],
                         ids=lambda c: "-".join(map(str, c)))
def test_varlen_feature_map_long_tail(dev, case, phi):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W, chunk = case
    L, H, tail = TAIL_CASE["lengths"], TAIL_CASE["H"], TAIL_CASE["tail"]
    vi = I.make_varlen_inputs(L, H, 128, 128, dtype="bf16", seed=990 + W, window=W,
                              S0_sd=0.2, halo=True, tail=tail)
    t = {n: to_dev(getattr(vi, n), "bf16", dev) for n in ("q", "k", "v", "k_prev", "v_prev")}
    g = {n: to_dev(getattr(vi, n), "fp32", dev) for n in ("alpha", "eta", "S0")}
    cu = torch.from_numpy(vi.cu).to(dev)
    N, maxT = len(L), max(L)
    need = fal.varlen_workspace_bytes(N, H, maxT, 128, 128, fal.BF16, variant, W, chunk, phi=phi)
    guard = 1 << 20
    ws = torch.full((need + guard,), 0x5A, dtype=torch.uint8, device=dev)
    o = torch.full(t["v"].shape, 7.0, dtype=torch.bfloat16, device=dev)
    announce(f"chunk_fwd_varlen {variant} W{W} phi={phi} lengths {L} tail {tail} H{H}")
    o, S = fal.chunk_fwd_varlen(t["q"], t["k"], t["v"], g["alpha"], g["eta"], cu, variant,
                                max_seqlen=maxT, window=W, chunk=chunk, S0=g["S0"],
                                k_prev=t["k_prev"], v_prev=t["v_prev"], o=o, phi=phi,
                                workspace=ws[:need])
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0x5A).all()), "the call wrote past its workspace"
    o_np, S_np = to_np(o), to_np(S)
    assert np.all(o_np[:, sum(L):] == 7.0)
    for n in range(N):
        d = vi.sequence(n).f64()
        o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                        window=W, S0=d["S0"], k_prev=d["k_prev"],
                                        v_prev=d["v_prev"], phi=phi)
        a, b = vi.cu[n], vi.cu[n + 1]
        assert slice_rel_err(o_np[None, :, a:b], o_ref, (2, 3)) <= TOL["bf16"], n
        assert slice_rel_err(S_np[n:n + 1], S_ref, (2, 3)) <= TOL["bf16"], n
