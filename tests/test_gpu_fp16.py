"""Unquantized fp16 weights (bits 16) on the GPU vs the CPU oracle: exact
cases and the scale/min pointers that this format does not read."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu


def _words(h):
    # fp16 patterns [n][k] -> words, k = 2j in the low half of word j.
    h = np.asarray(h, dtype=np.uint32)
    return (h[:, 0::2] | (h[:, 1::2] << 16)).astype(np.uint32)


def _matrix(w_f16):
    n, k = w_f16.shape
    return {"w": _words(w_f16.view(np.uint16)), "scales": None, "mins": None,
            "n": n, "k": k, "bits": 16, "group": 64}


def _run(q, x, m=None, tile=None, qmm_override=None):
    import torch
    from gemm_qmm_gemv_amd import tensors
    if tile is not None:
        qmm_override("QMM_GEMM_TILE_M", tile)
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    y = tensors.gemv(dq, xd) if m is None else tensors.gemm(dq, xd)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("m", (None, 2, 5, 100, 300))
def test_fp16_exact_integer(m, qmm_override):
    # Integer weights in [-8, 8] and activations in [-2, 2]: every partial
    # sum is an integer below 2^24, so GEMV and GEMM are exact.
    n, k = 333, 2048
    rng = inputs.rng_for(90, 0 if m is None else m)
    wi = rng.integers(-8, 9, size=(n, k)).astype(np.float16)
    xi = rng.integers(-2, 3, size=(1 if m is None else m, k)).astype(np.float16)
    q = _matrix(wi)
    x = xi[0] if m is None else xi
    announce("fp16-exact", m)
    y = _run(q, x, m)
    y_ref, _ = oracle.qmm(q["w"], None, None, x, n, k, 16, 64)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_fp16_gemv_one_hot():
    n, k = 150, 1024
    q = inputs.quantized_matrix(n, k, 16, 64, key=(91,))
    for j in (0, 1, 2, 31, 32, 33, 511, 1023):
        x = np.zeros(k, dtype=np.float16)
        x[j] = 1.0
        announce("fp16-one-hot", j)
        y = _run(q, x)
        y_ref, _ = oracle.qmm(q["w"], None, None, x, n, k, 16, 64)
        assert np.array_equal(y, y_ref.astype(np.float32)), j


@pytest.mark.parametrize("tile", (32, 64, 128))
def test_fp16_gemm_identity_rows(tile, qmm_override):
    # X = the first rows of I_K: row i of Y is column i of W, exactly.
    n, k, m = 200, 256, 70
    q = inputs.quantized_matrix(n, k, 16, 64, key=(92,))
    x = np.eye(m, k, dtype=np.float16)
    announce("fp16-identity", tile)
    y = _run(q, x, m, tile, qmm_override)
    y_ref, _ = oracle.qmm(q["w"], None, None, x, n, k, 16, 64)
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_fp16_ignores_scale_pointers():
    # Non-null scale and min pointers (to garbage) change nothing.
    import torch
    from gemm_qmm_gemv_amd import tensors
    n, k = 500, 1024
    q = inputs.quantized_matrix(n, k, 16, 64, key=(93,))
    x = inputs.activation_rows(1, k, key=(93,))[0]
    dq = tensors.upload_matrix(q)
    junk = torch.full((n * k // 64,), 12345, dtype=torch.int16, device="cuda")
    xd = tensors.device_tensor(x)
    announce("fp16-junk-scales")
    y0 = tensors.gemv(dq, xd)
    y1 = tensors.gemv(dict(dq, scales=junk, mins=junk), xd)
    torch.cuda.synchronize()
    assert np.array_equal(y0.cpu().numpy(), y1.cpu().numpy())
    y_ref, a_ref = oracle.qmm(q["w"], None, None, x, n, k, 16, 64)
    assert_within(y0.cpu().numpy(), y_ref, a_ref, "fp16 gemv 500x1024")
