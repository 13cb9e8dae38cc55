"""Helpers shared by the GPU parity tests (no test functions here)."""
import os
import sys

import numpy as np

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def announce(msg):
    """Name the case before each GPU step (a fault may end the process)."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def slice_rel_err(got, ref, axes):
    """Max over slices of max|got - ref| / max|ref| (slice = the leading
    axes not in `axes`); the acceptance metric for outputs and states."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def ensure_built():
    from weight_recurrent_sequence_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from weight_recurrent_sequence_amd import _build
        _build.build()


def to_np(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)
