"""Empty work through the C ABI: no rows, no columns, no (token, expert)
pairs.  Each call must succeed and leave its output buffer untouched.  The
buffers are real device allocations, so only the sizes are degenerate."""
import numpy as np
import pytest

import gemm_qmm_gemv_amd as qmm
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

SENTINEL = -7.0


def _dense(n=96, k=256, bits=4, group=64):
    from gemm_qmm_gemv_amd import tensors
    q = inputs.quantized_matrix(n, k, bits, group, key=(91, n, k, bits))
    x = tensors.device_tensor(inputs.activation_rows(4, k, key=(91, n, k, bits)))
    return tensors.upload_matrix(q), x


def _untouched(y):
    import torch
    torch.cuda.synchronize()
    assert bool((y == SENTINEL).all())


def test_gemm_with_no_rows_or_no_columns_writes_nothing():
    import torch
    dq, x = _dense()
    y = torch.full((4, dq["n"]), SENTINEL, dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    for m, n in ((0, dq["n"]), (4, 0)):
        announce("gemm-empty", m, n)
        for fn in (qmm.qmm_gemm, qmm.qmm_gemm_f16out):
            fn(dq["w"], dq["scales"], dq["mins"], x, y, m, n, dq["k"], dq["bits"], dq["group"],
               workspace=ws, workspace_bytes=ws.numel())
    _untouched(y)
    assert bool((ws == 0).all())


def test_grouped_gemm_with_no_rows_writes_nothing():
    import torch
    dq, x = _dense()
    ys = [torch.full((4, dq["n"]), SENTINEL, dtype=torch.float32, device="cuda") for _ in range(2)]
    members = [(dq["w"], dq["scales"], dq["mins"], y, dq["n"]) for y in ys]
    announce("gemm-grouped-empty", 0)
    qmm.qmm_gemm_grouped(members, x, 0, dq["k"], dq["bits"], dq["group"])
    for y in ys:
        _untouched(y)


@pytest.mark.parametrize("combine", (False, True), ids=("rows", "combine"))
def test_moe_with_no_pairs_writes_nothing(combine):
    import torch
    from gemm_qmm_gemv_amd import tensors
    e, n, k = 4, 64, 256
    st = inputs.stacked_experts(e, n, k, 4, 64, key=(92,))
    dst = tensors.upload_matrix(st)
    x = tensors.device_tensor(inputs.activation_rows(2, k, key=(92, k)))
    off = tensors.device_tensor(np.zeros(e + 1, dtype=np.int32))
    rows = tensors.device_tensor(np.zeros(2, dtype=np.int32))
    y = torch.full((2, n), SENTINEL, dtype=torch.float32, device="cuda")
    announce("moe-empty", combine)
    if combine:
        tok = tensors.device_tensor(np.zeros(2, dtype=np.int32))
        wgt = torch.ones(2, dtype=torch.float32, device="cuda")
        qmm.qmm_moe_combine(dst["w"], dst["scales"], dst["mins"], x, rows, 2, off, tok, wgt, y, 2, 0,
                            e, n, k, 4, 64)
    else:
        qmm.qmm_moe_gemm(dst["w"], dst["scales"], dst["mins"], x, rows, 2, off, y, 0, e, n, k, 4, 64)
    _untouched(y)
