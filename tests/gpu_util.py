"""Shared helpers of the GPU parity tests (HIP path vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np

REL_TOL = 2e-3   # |y - y_ref| <= REL_TOL * sum_k |w x| + ABS_TOL per element
ABS_TOL = 1e-5


def announce(*parts) -> None:
    """Name the case on stdout before a GPU step (a fault then still says which)."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def assert_within(y_gpu, y_ref, a_ref, what: str) -> float:
    """Acceptance bound per element; returns max |err| / a_ref for the log."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (what, y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite outputs" % what
    err = np.abs(y_gpu - y_ref)
    bound = REL_TOL * a_ref + ABS_TOL
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: gpu=%r ref=%r a=%r"
                             % (what, int(bad.sum()), err.size, i, y_gpu[i], y_ref[i], a_ref[i]))
    ratio = float(np.max(err / np.maximum(a_ref, 1e-30))) if err.size else 0.0
    print("[parity] %s: max |err|/a_ref = %.3e over %d outputs" % (what, ratio, err.size), flush=True)
    return ratio
