"""The algorithmic work bench.py divides by time, checked against the counts
written out from the method's definition (no GPU): bytes a call must move at
least once, and the flops of the chunk form on full tiles."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_chunk_bytes(bench):
    # q, k, v, o in bf16 (4 x 256 B per token-head at d = 128), alpha and eta
    # (2 x 4 B), plus the fp32 final state of every (batch, head)
    B, H, T, d = 8, 16, 4096, 128
    per_token_head = 4 * d * 2 + 2 * 4
    assert per_token_head == 1032
    want = B * H * T * per_token_head + B * H * d * d * 4
    assert bench.chunk_bytes(B, H, T, d) == want == 549_453_824


def test_chunk_flops(bench):
    # per 64-row tile of the delta family: the Gram blocks (A, P: 2 C^2 d each,
    # plus the write-vector products, 2 C^2 (3 d_k + 2 d_v) in all), the two
    # C x d products per side of the state and the update (6 C d^2), and the
    # triangular solve (2 C^3 / 3)
    C, d = 64, 128
    per_tile = 2 * C * C * (3 * d + 2 * d) + 6 * C * d * d + 2 * C ** 3 / 3
    assert bench.chunk_flops(8, 16, 4096, d, C) == pytest.approx(8 * 16 * 64 * per_tile)
    assert bench.chunk_flops(8, 16, 4096, d, C) == pytest.approx(95.92e9, rel=1e-3)
    # the inner-product family has no solve and no residual product
    per_tile_a = 2 * C * C * (d + d) + 4 * C * d * d
    assert bench.chunk_flops(8, 16, 4096, d, C, delta=False) == pytest.approx(8 * 16 * 64 * per_tile_a)


def test_decode_bytes(bench):
    # per head-step: the fp32 state read and written (2 x 64 KiB), q, k, v, o,
    # the key cache read and rewritten, alpha and eta
    N, H, d = 256, 32, 128
    per = 2 * d * d * 4 + 3 * d * 2 + 2 * d * 2 + 2 * 4 + d * 2
    assert per == 132_616
    assert bench.decode_bytes(N, H, d) == N * H * per
    assert bench.decode_bytes(N, H, d) == pytest.approx(1.086e9, rel=1e-3)


def test_decode_window_bytes(bench):
    # the window step also reads and rewrites W key-cache slots and W-1
    # value-cache slots
    N, H, d, W = 256, 32, 128, 4
    per = 2 * d * d * 4 + 4 * d * 2 + 2 * W * d * 2 + 2 * (W - 1) * d * 2 + 2 * 4
    assert bench.decode_window_bytes(N, H, d, W) == N * H * per


def test_bwd_bytes(bench):
    # q, k, v, d_o read and dq, dk, dv written once (bf16), the gates and their
    # gradients (fp32), dS_final read and dS0 written (fp32)
    B, H, T, d = 8, 16, 4096, 128
    want = B * H * T * (7 * d * 2 + 4 * 4) + 2 * B * H * d * d * 4
    assert bench.bwd_bytes(B, H, T, d) == want


def test_window_flops(bench):
    # Falcon-3 / Falcon-3A with W = 4 on chunks of C = 64 steps: E = C + W - 1
    # = 67 distinct keys serve CW = 256 virtual examples.  Falcon-3: the
    # extended key Gram (E^2 entries of d-long dot products), the query-key
    # products (C x E), the CW x CW triangular solve, the transformed keys and
    # targets (CW x CW times d_k + d_v), the residual product (CW x d_k x d_v),
    # the state read by the queries (C x d_k x d_v), the intra-chunk outputs
    # (C x CW x d_v) and the state update over the E keys (E x d_k x d_v),
    # two flops per multiply-add.
    C, W, d = 64, 4, 128
    E, Cv = C + W - 1, C * W
    per = (2 * E * E * d + 2 * C * E * d + 2 * Cv ** 3 / 3 + 2 * Cv * Cv * 2 * d
           + 2 * Cv * d * d + 2 * C * d * d + 2 * C * Cv * d + 2 * E * d * d)
    assert per == pytest.approx(63.86e6, rel=1e-3)
    chunks = 2 * 16 * (32768 // C)
    assert bench.window_flops(2, 16, 32768, d, C, W) == pytest.approx(chunks * per)
    assert bench.window_flops(2, 16, 32768, d, C, W) == pytest.approx(1.046e12, rel=1e-3)
    # Falcon-3A: the banded outputs over the E keys (C x E times d_k + d_v),
    # the state read and the update
    per_a = 2 * C * E * (d + d) + 2 * C * d * d + 2 * E * d * d
    assert bench.window_flops(2, 16, 32768, d, C, W, delta=False) == pytest.approx(chunks * per_a)
    assert bench.window_flops(2, 16, 32768, d, C, W, delta=False) == pytest.approx(106.3e9, rel=1e-2)
