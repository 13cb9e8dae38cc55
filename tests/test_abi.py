"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/falcon.h declares, and rejects invalid arguments on the host (before
any HIP call) with the documented status codes."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "falcon.h")


@pytest.fixture(scope="module")
def L():
    from weight_recurrent_sequence_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from weight_recurrent_sequence_amd import _build
        _build.build()
    return binding.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(falcon_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["falcon_chunk_fwd", "falcon_chunk_fwd_workspace",
                                           "falcon_chunk_bwd", "falcon_chunk_bwd_workspace",
                                           "falcon_chunk_bwd_varlen",
                                           "falcon_chunk_bwd_varlen_workspace",
                                           "falcon_chunk_fwd_varlen",
                                           "falcon_chunk_fwd_varlen_workspace",
                                           "falcon_chunk_fwd_save", "falcon_chunk_bwd_saved",
                                           "falcon_chunk_fwd_noalloc",
                                           "falcon_chunk_fwd_varlen_save",
                                           "falcon_chunk_bwd_varlen_saved",
                                           "falcon_decode_step", "falcon_decode_step_window",
                                           "falcon_status_string"])


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    from weight_recurrent_sequence_amd import binding
    for code in (0, -1, -2, -3, -4, -5, -6, 42):
        s = binding.status_string(code)
        assert isinstance(s, str) and s
    assert binding.status_string(99) == "unknown status"


def test_workspace_query(L):
    # one record per (batch*head, tile); a tile holds chunk // window steps
    n1 = L.falcon_chunk_fwd_workspace(8, 16, 4096, 128, 128, 1, 1, 1, 64)
    assert n1 > 0 and n1 % (8 * 16 * 64) == 0
    n3 = L.falcon_chunk_fwd_workspace(2, 16, 32768, 128, 128, 1, 3, 4, 64)
    assert n3 > 0 and n3 % (2 * 16 * (32768 // 16)) == 0
    assert L.falcon_chunk_fwd_workspace(8, 16, 0, 128, 128, 1, 1, 1, 64) == 0
    assert L.falcon_chunk_fwd_workspace(8, 16, 100, 96, 96, 1, 1, 1, 64) == 0   # rejected args
    # the inner-product family needs no triangular blocks: smaller records
    assert L.falcon_chunk_fwd_workspace(8, 16, 4096, 128, 128, 1, 11, 1, 64) < n1


def test_missing_workspace_is_rejected(L):
    assert chunk(L) == -4


P = 1 << 20  # a fake, 16-byte-aligned "device" address: never dereferenced


def chunk(L, **kw):
    a = dict(q=P, k=P, v=P, alpha=P, eta=P, S0=None, k_prev=None, v_prev=None, o=P, S_final=P,
             B=2, H=4, T=100, dk=128, dv=128, dt=1, var=1, window=1, chunk=64, eps=1e-6)
    a.update(kw)
    return L.falcon_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["eta"], a["S0"], a["k_prev"],
                              a["v_prev"], a["o"], a["S_final"], a["B"], a["H"], a["T"], a["dk"],
                              a["dv"], a["dt"], a["var"], a["window"], a["chunk"],
                              ctypes.c_float(a["eps"]), None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(var=4), -3), (dict(var=0), -3), (dict(dt=2), -3),
    (dict(B=0), -2), (dict(H=-1), -2), (dict(T=-1), -2), (dict(dk=0), -2),
    (dict(window=0), -2), (dict(window=2), -2),                 # window only for Falcon-3
    (dict(var=3, window=9), -3), (dict(chunk=48), -3), (dict(chunk=128), -3),
    (dict(dk=96, dv=96), -3), (dict(dk=64, dv=128), -3),
    (dict(dt=0, chunk=64), -4),                                  # fp32 d128 chunk64: no workspace
    (dict(eps=-1.0), -2), (dict(eps=float("nan")), -2),
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(alpha=None), -1),
    (dict(eta=None), -1), (dict(o=None), -1),
    (dict(q=P + 8), -3), (dict(S0=P + 4), -3), (dict(alpha=P + 2), -3),
    (dict(var=1 | 0x800), -3), (dict(var=0x100), -3), (dict(var=4 | 0x100), -3),  # flag bits
    (dict(var=1 | 0x100, window=2), -2),
    (dict(var=1 | 0x200 | 0x400), -3),                           # two feature maps
    (dict(var=1 | 0x200), -4), (dict(var=2 | 0x400 | 0x100), -4),  # valid flags, no workspace
])
def test_chunk_rejects(L, kw, code):
    assert chunk(L, **kw) == code


def decode(L, **kw):
    a = dict(S=P, kc=P, q=P, k=P, v=P, alpha=P, eta=P, o=P, N=4, H=2, dk=128, dv=128, dt=1,
             var=1, window=1, eps=1e-6)
    a.update(kw)
    return L.falcon_decode_step(a["S"], a["kc"], a["q"], a["k"], a["v"], a["alpha"], a["eta"],
                                a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dt"], a["var"],
                                a["window"], ctypes.c_float(a["eps"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(var=3), -3), (dict(var=13), -3), (dict(var=5), -3), (dict(dt=7), -3),
    (dict(N=0), -2), (dict(H=0), -2), (dict(window=0), -2), (dict(window=2), -3),
    (dict(dk=32, dv=32), -3), (dict(dk=128, dv=64), -3), (dict(eps=-2.0), -2),
    (dict(S=None), -1), (dict(kc=None), -1), (dict(o=None), -1), (dict(eta=None), -1),
    (dict(S=P + 8), -3),
    (dict(var=3 | 0x100), -3), (dict(var=1 | 0x800), -3), (dict(var=0x100), -3),
    (dict(var=1 | 0x600), -3),
])
def test_decode_rejects(L, kw, code):
    assert decode(L, **kw) == code


def decode_window(L, **kw):
    a = dict(S=P, kc=P, vc=P, q=P, k=P, v=P, alpha=P, eta=P, o=P, N=4, H=2, dk=128, dv=128, dt=1,
             var=3, window=4, eps=1e-6)
    a.update(kw)
    return L.falcon_decode_step_window(a["S"], a["kc"], a["vc"], a["q"], a["k"], a["v"],
                                       a["alpha"], a["eta"], a["o"], a["N"], a["H"], a["dk"],
                                       a["dv"], a["dt"], a["var"], a["window"],
                                       ctypes.c_float(a["eps"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(var=1), -3), (dict(var=11), -3), (dict(var=2), -3), (dict(dt=5), -3),
    (dict(N=0), -2), (dict(H=0), -2), (dict(window=0), -2), (dict(window=9), -3),
    (dict(dk=32, dv=32), -3), (dict(dk=128, dv=64), -3), (dict(eps=-1.0), -2),
    (dict(S=None), -1), (dict(kc=None), -1), (dict(vc=None), -1), (dict(o=None), -1),
    (dict(alpha=None), -1), (dict(S=P + 4), -3), (dict(eta=P + 2), -3),
    (dict(var=1 | 0x100), -3), (dict(var=3 | 0x1000), -3), (dict(var=3 | 0x600), -3),
])
def test_decode_window_rejects(L, kw, code):
    assert decode_window(L, **kw) == code


def test_python_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    import weight_recurrent_sequence_amd as fal
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(TypeError):
        fal.chunk_fwd(q.double(), q.double(), q.double(), torch.zeros(1, 1, 4),
                      torch.zeros(1, 1, 4), "F1")
    with pytest.raises(ValueError):
        fal.chunk_fwd(q, q, q[:, :, :3], torch.zeros(1, 1, 4), torch.zeros(1, 1, 4), "F1")


def test_package_has_no_cpu_fallback():
    """The binding only marshals arguments: it imports neither the oracle nor
    any CPU implementation of the recurrence."""
    pkg = os.path.join(ROOT, "weight_recurrent_sequence_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "import oracle" not in src and "from oracle" not in src, fn


def test_same_step_flag_keeps_the_workspace_size(L):
    """The alignment flag changes which key each pair reads, not the records."""
    for var in (1, 2, 3, 11, 12, 13):
        W = 4 if var in (3, 13) else 1
        a = L.falcon_chunk_fwd_workspace(2, 3, 1000, 128, 128, 1, var, W, 64)
        b = L.falcon_chunk_fwd_workspace(2, 3, 1000, 128, 128, 1, var | 0x100, W, 64)
        assert a == b and a > 0


def varlen(L, **kw):
    a = dict(q=P, k=P, v=P, alpha=P, eta=P, S0=None, k_prev=None, v_prev=None, o=P, S_final=P,
             cu=P, N=3, H=4, Ttot=300, maxT=150, dk=128, dv=128, dt=1, var=1, window=1,
             chunk=64, eps=1e-6)
    a.update(kw)
    return L.falcon_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["alpha"], a["eta"], a["S0"],
                                     a["k_prev"], a["v_prev"], a["o"], a["S_final"], a["cu"],
                                     a["N"], a["H"], a["Ttot"], a["maxT"], a["dk"], a["dv"],
                                     a["dt"], a["var"], a["window"], a["chunk"],
                                     ctypes.c_float(a["eps"]), None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), -1), (dict(cu=P + 2), -3), (dict(N=0), -2), (dict(H=0), -2),
    (dict(Ttot=-1), -2), (dict(maxT=-1), -2), (dict(var=4), -3), (dict(window=2), -2),
    (dict(dk=96, dv=96), -3), (dict(q=None), -1), (dict(o=None), -1), (dict(eps=-1.0), -2),
    (dict(), -4),                                                   # no workspace given
])
def test_varlen_rejects(L, kw, code):
    assert varlen(L, **kw) == code


def test_varlen_workspace_matches_batched_layout(L):
    """Records are per (sequence, head) with the longest sequence's tile count,
    followed by 256-byte-aligned room for 2N+1 ints (the schedule) and a job
    table of 16 bytes per record slot."""
    a = L.falcon_chunk_fwd_varlen_workspace(3, 4, 150, 128, 128, 1, 1, 1, 64)
    b = L.falcon_chunk_fwd_workspace(3, 4, 150, 128, 128, 1, 1, 1, 64)
    assert b > 0 and a == b + 256 + 3 * 4 * 3 * 16
    assert L.falcon_chunk_fwd_varlen_workspace(1000, 4, 150, 128, 128, 1, 1, 1, 64) == \
        L.falcon_chunk_fwd_workspace(1000, 4, 150, 128, 128, 1, 1, 1, 64) + 8192 + 1000 * 4 * 3 * 16


def test_feature_map_workspace_holds_the_mapped_inputs(L):
    """With a feature map the workspace also holds the mapped keys and queries
    (B*H*T*dk entries each, 256-byte aligned) and the mapped halo keys.  The
    scalar rule's records are the same with and without a map; the window
    rules with a map run the split kernels, whose records are at least the
    collapsed form's that the call without a map sizes."""
    B, H, T, d = 2, 3, 1000, 128
    es = 2
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    for var, W in ((1, 1), (3, 4), (13, 3)):
        base = L.falcon_chunk_fwd_workspace(B, H, T, d, d, 1, var, W, 64)
        sizes = set()
        for flag in (0x200, 0x400, 0x200 | 0x100):
            got = L.falcon_chunk_fwd_workspace(B, H, T, d, d, 1, var | flag, W, 64)
            rec = got - 2 * al(B * H * T * d * es) - al(B * H * W * d * es)
            assert rec % 256 == 0 and rec >= base, (var, flag)
            if W == 1:
                assert rec == al(base)
            sizes.add(got)
        assert len(sizes) == 1  # the map and the alignment do not change the size


def test_window_forward_workspace_is_the_collapsed_forms(L):
    """The window rules at bf16 without a feature map size the forward's
    workspace by the collapsed form's records (and the segmented pass's group
    states), not by the split kernels' records that the backward's checkpoint
    runs need (its workspace query includes those)."""
    for var in (3, 13):
        fwd = L.falcon_chunk_fwd_workspace(2, 16, 32768, 128, 128, 1, var, 4, 64)
        fp32 = L.falcon_chunk_fwd_workspace(2, 16, 32768, 128, 128, 0, var, 4, 64)
        mapped = L.falcon_chunk_fwd_workspace(2, 16, 32768, 128, 128, 1, var | 0x200, 4, 64)
        bwd = L.falcon_chunk_bwd_workspace(2, 16, 32768, 128, 128, 1, var, 4, 64)
        assert 0 < fwd < fp32 and fwd < mapped and fwd < bwd, var


def bwd(L, fn="falcon_chunk_bwd", **kw):
    a = dict(q=P, k=P, v=P, alpha=P, eta=P, S0=None, k_prev=None, v_prev=None, do=P, dS=None,
             dq=P, dk=P, dv=P, dal=P, det=P, dS0=None, dkp=None, dvp=None, B=2, H=4, T=100,
             dk_=128, dv_=128, dt=1, var=1, window=1, chunk=64, eps=1e-6, ws=None, wsn=0)
    a.update(kw)
    return getattr(L, fn)(a["q"], a["k"], a["v"], a["alpha"], a["eta"], a["S0"], a["k_prev"],
                              a["v_prev"], a["do"], a["dS"], a["dq"], a["dk"], a["dv"], a["dal"],
                              a["det"], a["dS0"], a["dkp"], a["dvp"], a["B"], a["H"], a["T"],
                              a["dk_"], a["dv_"], a["dt"], a["var"], a["window"], a["chunk"],
                              ctypes.c_float(a["eps"]), a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(var=4), -3), (dict(dt=0), -3), (dict(chunk=32), -3), (dict(var=2, chunk=16), -3),
    (dict(var=12, dt=0), -3), (dict(var=3, window=9), -3), (dict(dk_=96, dv_=96), -3),
    (dict(var=2), -4), (dict(var=12 | 0x100), -4),
    (dict(var=3, window=2), -4), (dict(var=13, window=8), -4),
    (dict(B=0), -2), (dict(T=-1), -2), (dict(eps=-1.0), -2),
    (dict(q=None), -1), (dict(do=None), -1), (dict(dq=None), -1), (dict(dk=None), -1),
    (dict(dv=None), -1), (dict(dal=None), -1), (dict(det=None), -1),
    (dict(dq=P + 8), -3), (dict(dal=P + 2), -3), (dict(dS0=P + 4), -3),
    (dict(var=1 | 0x800), -3), (dict(var=1 | 0x600), -3),
    (dict(), -4), (dict(var=11 | 0x100 | 0x200), -4), (dict(var=3, window=1), -4),
])
def test_bwd_rejects(L, kw, code):
    assert bwd(L, **kw) == code
    # the backward from saved checkpoints checks its arguments the same way
    assert bwd(L, fn="falcon_chunk_bwd_saved", **kw) == code


def fwd_save(L, **kw):
    a = dict(q=P, k=P, v=P, alpha=P, eta=P, S0=None, k_prev=None, v_prev=None, o=P, S=None,
             B=2, H=4, T=100, dk_=128, dv_=128, dt=1, var=1, window=1, chunk=64, eps=1e-6,
             ws=None, wsn=0)
    a.update(kw)
    return L.falcon_chunk_fwd_save(a["q"], a["k"], a["v"], a["alpha"], a["eta"], a["S0"],
                                   a["k_prev"], a["v_prev"], a["o"], a["S"], a["B"], a["H"],
                                   a["T"], a["dk_"], a["dv_"], a["dt"], a["var"], a["window"],
                                   a["chunk"], ctypes.c_float(a["eps"]), a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(var=4), -3), (dict(dt=0), -3), (dict(chunk=32), -3), (dict(dk_=96, dv_=96), -3),
    (dict(var=3, window=9), -3), (dict(B=0), -2), (dict(eps=-1.0), -2),
    (dict(q=None), -1), (dict(o=None), -1),
    (dict(), -4), (dict(ws=P, wsn=1024), -4), (dict(var=13, window=4), -4),
])
def test_fwd_save_rejects(L, kw, code):
    """The saving forward takes the forward's arguments, the backward's
    support matrix and a buffer of the backward's workspace size."""
    assert fwd_save(L, **kw) == code


def test_fwd_save_with_nothing_to_do(L):
    # no steps and no final state: nothing to write, no buffer needed
    assert fwd_save(L, T=0) == 0


def test_bwd_workspace_sizes(L):
    """The forward's workspace, then the state at every tile start and the
    state gradient at every tile end (bf16, d x d each) and Delta (bf16,
    d x chunk), each 256-byte aligned."""
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    for var in (1, 11, 1 | 0x100, 11 | 0x200):
        B, H, T, d = 2, 3, 1000, 128
        fwd = L.falcon_chunk_fwd_workspace(B, H, T, d, d, 1, var, 1, 64)
        nt = (T + 63) // 64
        want = al(fwd) + 2 * al(B * H * nt * d * d * 2) + al(B * H * nt * d * 64 * 2)
        assert L.falcon_chunk_bwd_workspace(B, H, T, d, d, 1, var, 1, 64) == want
    # windows: tiles of 64 // W steps, and room for the per-row target and key
    # gradients; the forward part is the split kernels' records (those of a
    # call with a feature map, less the mapped inputs), which the checkpoint
    # runs use, not the collapsed form's that the forward alone sizes
    B, H, T, d, W = 2, 3, 1000, 128, 4
    fwd = (L.falcon_chunk_fwd_workspace(B, H, T, d, d, 1, 3 | 0x200, W, 64)
           - 2 * al(B * H * T * d * 2) - al(B * H * W * d * 2))
    assert fwd > L.falcon_chunk_fwd_workspace(B, H, T, d, d, 1, 3, W, 64)
    nt = (T + 64 // W - 1) // (64 // W)
    want = al(fwd) + 2 * al(B * H * nt * d * d * 2) + 3 * al(B * H * nt * d * 64 * 2)
    assert L.falcon_chunk_bwd_workspace(B, H, T, d, d, 1, 3, W, 64) == want
    assert L.falcon_chunk_bwd_workspace(2, 3, 1000, 128, 128, 1, 2, 1, 32) == 0   # unsupported
    assert L.falcon_chunk_bwd_workspace(2, 3, 1000, 128, 128, 0, 1, 1, 32) == 0
    assert L.falcon_chunk_bwd_workspace(2, 3, 0, 128, 128, 1, 1, 1, 64) == 0


def test_bwd_varlen_workspace(L):
    """The packed forward's workspace, then the same checkpoint room as a
    batched call of N sequences of max_seqlen steps."""
    al = lambda n: (n + 255) // 256 * 256  # noqa: E731
    for var, W in ((1, 1), (13, 4), (2 | 0x200, 1)):
        N, H, mx, d = 5, 3, 300, 128
        fwd = L.falcon_chunk_fwd_varlen_workspace(N, H, mx, d, d, 1, var, W, 64)
        if W > 1:
            # the split kernels' records, as in test_bwd_workspace_sizes
            fwd = (L.falcon_chunk_fwd_varlen_workspace(N, H, mx, d, d, 1, var | 0x200, W, 64)
                   - 2 * al(N * H * mx * d * 2) - al(N * H * W * d * 2))
        nt = (mx + 64 // W - 1) // (64 // W)
        want = al(fwd) + 2 * al(N * H * nt * d * d * 2) + al(N * H * nt * d * 64 * 2)
        if W > 1:
            want += 2 * al(N * H * nt * d * 64 * 2)
        assert L.falcon_chunk_bwd_varlen_workspace(N, H, mx, d, d, 1, var, W, 64) == want
    assert L.falcon_chunk_bwd_varlen_workspace(5, 3, 300, 128, 128, 0, 1, 1, 32) == 0
