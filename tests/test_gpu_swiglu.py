"""Fused gate/up projection (qmm_gemv_swiglu) on the GPU vs the CPU oracle:
h = silu(Wg x) * (Wu x)."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import announce, glu_bound

pytestmark = pytest.mark.gpu


def _pair(n, k, bits, group, seed):
    g = inputs.quantized_matrix(n, k, bits, group, key=(95, seed, 0, n, k, bits, group))
    u = inputs.quantized_matrix(n, k, bits, group, key=(95, seed, 1, n, k, bits, group))
    x = inputs.activation_rows(1, k, key=(95, seed, n, k, bits, group))[0]
    return g, u, x


def _run(g, u, x):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dg, du = tensors.upload_matrix(g), tensors.upload_matrix(u)
    h = tensors.gemv_swiglu(dg, du, tensors.device_tensor(x))
    torch.cuda.synchronize()
    return h.cpu().numpy()


def _check(h, g, u, x, what):
    n, k, bits, group = g["n"], g["k"], g["bits"], g["group"]
    g_ref, a_g = oracle.qmm(g["w"], g["scales"], g["mins"], x, n, k, bits, group)
    u_ref, a_u = oracle.qmm(u["w"], u["scales"], u["mins"], x, n, k, bits, group)
    h_ref = oracle.silu(g_ref) * u_ref
    bound = glu_bound(g_ref, a_g, u_ref, a_u)
    err = np.abs(h.astype(np.float64) - h_ref)
    assert np.all(np.isfinite(h)), what
    bad = err > bound
    assert not bad.any(), "%s: %d outside; worst %r" % (what, int(bad.sum()), float(np.max(err - bound)))
    print("[parity] %s: max err/bound = %.3e" % (what, float(np.max(err / bound))), flush=True)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
@pytest.mark.parametrize("n,k,group", [(3072, 1024, 64), (1000, 3072, 64), (8192, 2048, 64),
                                       (77, 512, 32), (129, 4096, 128), (1, 64, 64), (33, 8192, 64)])
def test_swiglu_parity(bits, n, k, group):
    if bits == 16 and k > 4096:
        pytest.skip("fp16 weights: one pass covers k <= 4096 (see the unsupported-size test)")
    g, u, x = _pair(n, k, bits, group, 1)
    announce("swiglu", bits, n, k, group)
    _check(_run(g, u, x), g, u, x, "swiglu b%d %dx%d g%d" % (bits, n, k, group))


def test_swiglu_matches_separate_gemvs():
    # Same arithmetic as two qmm_gemv launches followed by silu * product.
    import torch
    from gemm_qmm_gemv_amd import tensors
    n, k = 3072, 1024
    g, u, x = _pair(n, k, 4, 64, 2)
    dg, du = tensors.upload_matrix(g), tensors.upload_matrix(u)
    xd = tensors.device_tensor(x)
    announce("swiglu-vs-gemv")
    h = tensors.gemv_swiglu(dg, du, xd)
    yg, yu = tensors.gemv(dg, xd), tensors.gemv(du, xd)
    torch.cuda.synchronize()
    yg, yu = yg.cpu().numpy().astype(np.float64), yu.cpu().numpy().astype(np.float64)
    sep = oracle.silu(yg) * yu
    assert np.allclose(h.cpu().numpy(), sep, rtol=1e-4, atol=1e-5)


def test_swiglu_saturation():
    # Large |g|: silu -> g for g >> 0 and -> 0 for g << 0, no NaN or Inf.
    n, k = 64, 256
    g, u, x = _pair(n, k, 8, 64, 3)
    g = dict(g, scales=(g["scales"].astype(np.float32) * 40).astype(np.float16),
             mins=(g["mins"].astype(np.float32) * 40).astype(np.float16))
    announce("swiglu-saturation")
    h = _run(g, u, x)
    _check(h, g, u, x, "swiglu large gate")


def test_swiglu_unsupported_k():
    from gemm_qmm_gemv_amd import QmmError
    g, u, x = _pair(16, 16384, 4, 64, 4)
    with pytest.raises(QmmError, match="more than one pass"):
        _run(g, u, x)
