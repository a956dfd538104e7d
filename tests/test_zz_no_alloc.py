"""qmm_gemm_noalloc (the prefill GEMM that allocates nothing) through the C
ABI: bit-identical to qmm_gemm run with its preferred workspace, on two calls
in a row with the second one smaller, over the plans that use the scratch
array differently (split summed in the kernel with arrival counters, split
summed by a second kernel, no split, and the small-m route that needs none).
"""
import numpy as np
import pytest
import torch

import gemm_qmm_gemv_amd as qmm
from gemm_qmm_gemv_amd import inputs, tensors
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

BITS, GROUP = 4, 64

# (first call, second call): each (m, n, k); the second is smaller.
SEQUENCES = [
    ((128, 4096, 2048), (96, 2048, 1024)),    # two-way split summed in the kernel, then a smaller one
    ((128, 2048, 2048), (64, 512, 2048)),     # split summed by a second kernel
    ((512, 8192, 2048), (2, 256, 1024)),      # no split, then the multi-row GEMV route
    ((2048, 256, 2048), (200, 1024, 3072)),   # in-kernel split at 2048 tokens, then a ragged m
]


def _case(m, n, k, key):
    q = inputs.quantized_matrix(n, k, BITS, GROUP, key=key)
    x = inputs.activation_rows(m, k, key=key)
    return tensors.upload_matrix(q), tensors.device_tensor(x)


def _noalloc(dq, xd):
    m = xd.shape[0]
    y = torch.full((m, dq["n"]), float("nan"), dtype=torch.float32, device="cuda")
    qmm.qmm_gemm_noalloc(dq["w"], dq["scales"], dq["mins"], xd, y, m, dq["n"], dq["k"], dq["bits"],
                         dq["group"])
    return y


def _with_workspace(dq, xd):
    m = xd.shape[0]
    y = torch.full((m, dq["n"]), float("nan"), dtype=torch.float32, device="cuda")
    return tensors.gemm(dq, xd, y=y)


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_equals_qmm_gemm_twice(seq):
    for call, (m, n, k) in enumerate(SEQUENCES[seq]):
        announce("qmm_gemm_noalloc", "sequence", seq, "call", call, "m n k", m, n, k)
        dq, xd = _case(m, n, k, key=(40, seq, call))
        plan = qmm.qmm_get_plan(1, m, n, k, BITS, GROUP, workspace_bytes=1 << 40)
        need = qmm.qmm_gemm_workspace_bytes(m, n, k, BITS, GROUP)
        assert need <= qmm.QMM_NOALLOC_SCRATCH_BYTES
        y_na = _noalloc(dq, xd)
        y_ws = _with_workspace(dq, xd)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert np.isfinite(a).all(), "unwritten outputs (m=%d n=%d k=%d)" % (m, n, k)
        assert np.array_equal(a, b), "noalloc differs from qmm_gemm at m=%d n=%d k=%d split=%d" % (
            m, n, k, plan["split_k"])
        print("[noalloc] m=%d n=%d k=%d split=%d tile=%d equal" % (m, n, k, plan["split_k"], plan["tile_m"]),
              flush=True)


def test_noalloc_repeated_calls_reset_the_counters():
    # The same split shape five times in a row on one stream: every call
    # finds its arrival counters at zero (each resets the ones it uses).
    dq, xd = _case(128, 8192, 2048, key=(41, 0, 0))
    announce("qmm_gemm_noalloc repeated", 128, 8192, 2048)
    ref = _with_workspace(dq, xd)
    for _ in range(5):
        y = _noalloc(dq, xd)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)


def test_noalloc_rejects_a_split_beyond_the_scratch(qmm_override):
    # Forcing 16 splits of 512 x 8192 fp32 partial sums asks for 256 MiB,
    # more than the array holds: the call fails on the host and writes
    # nothing.
    qmm_override("QMM_GEMM_SPLIT", 16)
    m, n, k = 512, 8192, 8192
    assert qmm.qmm_gemm_workspace_bytes(m, n, k, BITS, GROUP) > qmm.QMM_NOALLOC_SCRATCH_BYTES
    dq, xd = _case(m, n, k, key=(42, 0, 0))
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_gemm_noalloc(dq["w"], dq["scales"], dq["mins"], xd, y, m, n, k, BITS, GROUP)
    assert e.value.status == qmm.QMM_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
