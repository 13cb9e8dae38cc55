"""falcon_chunk_fwd_noalloc: the forward with the library's built-in scratch
buffer instead of a caller workspace, for callers that cannot allocate.

Checked through the C ABI against falcon_chunk_fwd with a caller workspace:
the same kernels run on the same inputs, so the results must be equal bit
for bit.  Two calls in a row, the second with a smaller input (the buffer
keeps the first call's contents, which the second must not depend on), for
several variants; a call needing more than the buffer holds is rejected
before anything runs; host-side argument checks come first."""
import numpy as np
import pytest

from tests.gpu_util import announce, ensure_built
from weight_recurrent_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    ensure_built()
    return torch.device("cuda:0")


CASES = [("F1", 1, "bf16", 128, 64), ("F2", 1, "bf16", 128, 64), ("F3", 4, "bf16", 128, 64),
         ("F3A", 3, "bf16", 64, 16), ("F1", 1, "fp32", 64, 32), ("F2A", 1, "fp32", 128, 64)]


def both(fal, t, variant, W, chunk, **kw):
    import torch
    args = (t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant)
    kws = dict(window=W, chunk=chunk, S0=t["S0"], k_prev=t["k_prev"], v_prev=t["v_prev"], **kw)
    o_n, S_n = fal.chunk_fwd_noalloc(*args, **kws)
    o_w, S_w = fal.chunk_fwd(*args, **kws)
    torch.cuda.synchronize()
    return (o_n, S_n), (o_w, S_w)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_noalloc_equals_workspace_call_twice(dev, case):
    import torch
    import weight_recurrent_sequence_amd as fal
    variant, W, dtype, D, chunk = case
    for T, B, H in ((777, 3, 4), (130, 1, 2)):  # the second call is smaller
        inp = I.make_chunk_inputs(B, H, T, D, D, dtype=dtype, seed=7700 + T + W, window=W,
                                  halo=True, S0_sd=0.2)
        t = inp.to_torch(dev)
        announce(f"chunk_fwd_noalloc {variant} W{W} {dtype} d{D} chunk{chunk} B{B} H{H} T{T}")
        (o_n, S_n), (o_w, S_w) = both(fal, t, variant, W, chunk)
        assert torch.isfinite(o_n.float()).all()
        assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w), (T, B, H)


def test_noalloc_segmented_window_pass(dev):
    """Falcon-3A chains of 64 tiles or more run in segments whose group states
    and copy of S0 live in the scratch buffer: two such calls in a row, the
    second smaller, equal the workspace calls bit for bit."""
    import torch
    import weight_recurrent_sequence_amd as fal
    for T, B, H in ((2100, 2, 3), (2050, 1, 2)):
        inp = I.make_chunk_inputs(B, H, T, 128, 128, dtype="bf16", seed=7750 + T, window=4,
                                  halo=True, S0_sd=0.2)
        t = inp.to_torch(dev)
        announce(f"chunk_fwd_noalloc F3A W4 bf16 d128 chunk64 B{B} H{H} T{T} (segments)")
        (o_n, S_n), (o_w, S_w) = both(fal, t, "F3A", 4, 64)
        assert torch.isfinite(o_n.float()).all()
        assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w), (T, B, H)


def test_noalloc_feature_map_and_same_step(dev):
    import torch
    import weight_recurrent_sequence_amd as fal
    inp = I.make_chunk_inputs(2, 3, 200, 128, 128, dtype="bf16", seed=7790, window=3, halo=True,
                              S0_sd=0.2)
    t = inp.to_torch(dev)
    for align, phi in (("same", "identity"), ("prefix", "l2"), ("same", "silu")):
        announce(f"chunk_fwd_noalloc F3 W3 align={align} phi={phi}")
        (o_n, S_n), (o_w, S_w) = both(fal, t, "F3", 3, 64, align=align, phi=phi)
        assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w), (align, phi)


def test_noalloc_rejects_calls_beyond_the_buffer(dev):
    import torch
    import weight_recurrent_sequence_amd as fal
    # Falcon-2 at B4 H32 T8192 d128 needs its records and write vectors,
    # more than the 128 MiB buffer: rejected on the host, nothing launched
    B, H, T, D = 4, 32, 8192, 128
    need = fal.workspace_bytes(B, H, T, D, D, fal.BF16, "F2", 1, 64)
    assert need > fal.binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, H, T, D), dtype=torch.bfloat16, device=dev)
    g = torch.ones((B, H, T), dtype=torch.float32, device=dev)
    o = torch.full((B, H, T, D), 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fal.FalconError) as ei:
        fal.chunk_fwd_noalloc(x, x, x, g, g, "F2", chunk=64, o=o)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
    # the headline Falcon-1 workload fits
    assert fal.workspace_bytes(8, 16, 4096, D, D, fal.BF16, "F1", 1, 64) <= \
        fal.binding.NOALLOC_SCRATCH_BYTES


def test_noalloc_full_size_falcon1(dev):
    """The Falcon-1 workload B8 H16 T4096 d128 (its 114 MiB of records fill
    most of the buffer) equals the workspace call, after a smaller call."""
    import torch
    import weight_recurrent_sequence_amd as fal
    inp = I.workload_inputs("falcon1_bf16_B8H16T4096d128")
    t = inp.to_torch(dev)
    announce("chunk_fwd_noalloc F1 B8 H16 T4096 d128")
    (o_n, S_n), (o_w, S_w) = both(fal, t, "F1", 1, 64)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
    small = I.make_chunk_inputs(1, 1, 50, 128, 128, dtype="bf16", seed=7799)
    ts = small.to_torch(dev)
    (o_n, S_n), (o_w, S_w) = both(fal, ts, "F1", 1, 64)
    assert torch.equal(o_n, o_w) and torch.equal(S_n, S_w)


def test_noalloc_host_checks_first(dev):
    import torch
    import weight_recurrent_sequence_amd as fal
    L = fal.lib()
    # invalid variant / NULL inputs return their codes before the scratch is touched
    assert L.falcon_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, None, None,
                                      1, 1, 8, 64, 64, 1, 4, 1, 64, 1e-6, None) == -3
    assert L.falcon_chunk_fwd_noalloc(None, None, None, None, None, None, None, None, None, None,
                                      1, 1, 8, 64, 64, 1, 1, 1, 64, 1e-6, None) == -1
    # T = 0 copies S0 to S_final and needs no scratch
    S0 = torch.randn(1, 2, 64, 64, device=dev)
    Sf = torch.empty_like(S0)
    x = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    g = torch.empty((1, 2, 0), dtype=torch.float32, device=dev)
    fal.chunk_fwd_noalloc(x, x, x, g, g, "F1", chunk=64, S0=S0, S_final=Sf)
    torch.cuda.synchronize()
    assert torch.equal(Sf, S0)
    np.testing.assert_equal(Sf.cpu().numpy(), S0.cpu().numpy())
