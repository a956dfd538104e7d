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


def assert_within(y_gpu, y_ref, a_ref, what: str, fp16_out: bool = False) -> float:
    """Acceptance bound per element; returns max |err| / a_ref for the log.

    fp16_out: the result was rounded once more, to fp16 (nearest even), which
    adds at most half an fp16 ulp: 2^-11 |y| in the normal range, 2^-25 below
    it."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    assert y_gpu.shape == y_ref.shape, (what, y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), "%s: non-finite outputs" % what
    err = np.abs(y_gpu - y_ref)
    bound = REL_TOL * a_ref + ABS_TOL
    if fp16_out:
        bound = bound + 2.0 ** -11 * np.abs(y_ref) + 2.0 ** -25
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d outside tolerance; worst at %s: gpu=%r ref=%r a=%r"
                             % (what, int(bad.sum()), err.size, i, y_gpu[i], y_ref[i], a_ref[i]))
    ratio = float(np.max(err / np.maximum(a_ref, 1e-30))) if err.size else 0.0
    print("[parity] %s: max |err|/a_ref = %.3e over %d outputs" % (what, ratio, err.size), flush=True)
    return ratio


def glu_bound(g_ref, a_g, u_ref, a_u):
    """Acceptance bound for h = silu(g) * u from the bounds of g and u.

    With |dg| <= eg = REL_TOL * a_g + ABS_TOL (same for u) and |silu'| <= 1.1
    everywhere, |silu(g + dg)(u + du) - silu(g) u| <= 1.1 eg (|u| + eu) +
    |silu(g)| eu; fp32 evaluation of the exponential, division and product
    adds a few ulp of |h| (bounded here by 1e-5 |h| + 1e-7)."""
    import oracle
    eg = REL_TOL * a_g + ABS_TOL
    eu = REL_TOL * a_u + ABS_TOL
    sg = oracle.silu(g_ref)
    return 1.1 * eg * (np.abs(u_ref) + eu) + np.abs(sg) * eu + 1e-5 * np.abs(sg * u_ref) + 1e-7
