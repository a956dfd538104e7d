"""Entry points captured in a HIP graph and replayed several times, with the
program's own eager work and synchronizations between replays: every replay
must reproduce the eager result bit for bit (the K-split GEMM's arrival
counters reset themselves; nothing here records a memset)."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu


def _replays(fn, out, eager, n=5):
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(n):
        out.fill_(float("nan"))
        noise.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager result" % r


@pytest.mark.parametrize("m,n,k", [(128, 4096, 2048), (128, 2048, 2048), (512, 1024, 2048)])
def test_split_gemm_graph_replays(m, n, k):
    # Two-way splits reduce inside the kernel, four-way in a second kernel.
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    q = inputs.quantized_matrix(n, k, 4, 64, key=(120, m, n, k))
    x = inputs.activation_rows(m, k, key=(120, m, n, k))
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    pl = qmm.qmm_get_plan(1, m, n, k, 4, 64, workspace_bytes=ws.numel())
    assert pl["split_k"] > 1
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    announce("graph-gemm", m, n, k, pl["split_k"])
    tensors.gemm(dq, xd, y, workspace=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    rn = np.arange(0, n, 97)
    rows = np.repeat(np.arange(0, m, 31), len(rn))
    cols = np.tile(rn, len(np.arange(0, m, 31)))
    y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, 4, 64, rows, cols)
    assert_within(eager.cpu().numpy()[rows, cols], y_ref, a_ref, "graph gemm eager")
    _replays(lambda: tensors.gemm(dq, xd, y, workspace=ws), y, eager)


def test_batched_gemv_graph_replays():
    import torch
    from gemm_qmm_gemv_amd import tensors
    shapes = [(2048, 1024), (1024, 1024), (3072, 1024), (1024, 3072), (20000, 1024)]
    items = []
    for i, (n, k) in enumerate(shapes):
        q = inputs.quantized_matrix(n, k, 4, 64, key=(121, i))
        x = inputs.activation_rows(1, k, key=(121, i))[0]
        items.append((tensors.upload_matrix(q), tensors.device_tensor(x),
                      torch.empty(n, dtype=torch.float32, device="cuda")))
    batch = tensors.GemvBatch(items, 4, 64)
    announce("graph-batched")
    batch()
    torch.cuda.synchronize()
    ys = [it[2] for it in items]
    eager = torch.cat([y.clone() for y in ys])

    class Cat:
        def fill_(self, v):
            for y in ys:
                y.fill_(v)

    out = Cat()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        batch()
    for r in range(5):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(ys), eager), "replay %d differs" % r
