"""Decode GEMV with the residual add fused (qmm_gemv_residual) on the GPU vs
the CPU oracle: y = r + W x."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import ABS_TOL, REL_TOL, announce

pytestmark = pytest.mark.gpu


def _case(n, k, bits, group, seed):
    q = inputs.quantized_matrix(n, k, bits, group, key=(97, seed, n, k, bits, group))
    x = inputs.activation_rows(1, k, key=(97, seed, n, k, bits, group))[0]
    r = inputs.activation_rows(1, n, key=(98, seed, n, k))[0].astype(np.float32) * 4
    return q, x, r


def _check(y, q, x, r, what):
    n, k, bits, group = q["n"], q["k"], q["bits"], q["group"]
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
    want = r.astype(np.float64) + y_ref
    # The GEMV's own bound, plus one more fp32 rounding for the add.
    bound = REL_TOL * a_ref + ABS_TOL + 2.0 ** -23 * (np.abs(r) + np.abs(y_ref))
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), what
    bad = np.abs(y - want) > bound
    assert not bad.any(), "%s: %d outside" % (what, int(bad.sum()))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
@pytest.mark.parametrize("n,k,group", [(3072, 1024, 64), (1000, 3072, 64), (77, 512, 32),
                                       (129, 16384, 128), (1, 64, 64)])
def test_residual_parity(bits, n, k, group):
    import torch
    from gemm_qmm_gemv_amd import tensors
    q, x, r = _case(n, k, bits, group, 1)
    announce("gemv-residual", bits, n, k, group)
    dq = tensors.upload_matrix(q)
    y = tensors.gemv_residual(dq, tensors.device_tensor(x), torch.from_numpy(r).cuda())
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), q, x, r, "residual b%d %dx%d g%d" % (bits, n, k, group))


@pytest.mark.parametrize("n,k", [(3072, 1024), (2048, 8192), (40, 16384)])
def test_residual_in_place(n, k):
    # y += W x: the residual buffer is the output.
    import torch
    from gemm_qmm_gemv_amd import tensors
    q, x, r = _case(n, k, 4, 64, 2)
    announce("gemv-residual-in-place", n, k)
    dq = tensors.upload_matrix(q)
    y = torch.from_numpy(r.copy()).cuda()
    tensors.gemv_residual(dq, tensors.device_tensor(x), y, y)
    torch.cuda.synchronize()
    _check(y.cpu().numpy(), q, x, r, "residual in place %dx%d" % (n, k))


def test_residual_zero_equals_plain_gemv():
    # r = 0 adds exactly nothing: same bits as qmm_gemv.
    import torch
    from gemm_qmm_gemv_amd import tensors
    q, x, _ = _case(3072, 1024, 4, 64, 3)
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    announce("gemv-residual-zero")
    y0 = tensors.gemv_residual(dq, xd, torch.zeros(3072, dtype=torch.float32, device="cuda"))
    y1 = tensors.gemv(dq, xd)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
