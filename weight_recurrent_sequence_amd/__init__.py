"""Falcon fast-weight recurrence on AMD Instinct MI355X (gfx950).

The computation runs in libfalcon.so (hand-written HIP kernels behind the C
ABI of include/falcon.h); this package is its Python binding plus the seeded
input generators used by tests and benchmarks.
"""
from .binding import (BF16, F1, F1A, F2, F2A, F3, F3A, FP32, SAME_STEP, VARIANTS, FalconError,  # noqa: F401
                      bwd_varlen_workspace_bytes, bwd_workspace_bytes, chunk_bwd,
                      chunk_bwd_saved, chunk_bwd_varlen, chunk_bwd_varlen_saved, chunk_fwd,
                      chunk_fwd_noalloc,
                      chunk_fwd_save, chunk_fwd_varlen, chunk_fwd_varlen_save, decode_step,
                      decode_step_window, lib,
                      status_string, varlen_workspace_bytes, workspace_bytes)
