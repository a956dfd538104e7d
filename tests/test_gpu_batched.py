"""Batched decode GEMVs (qmm_gemv_batched) on the GPU vs the CPU oracle."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu


def _run_batch(shapes, bits, group, seed):
    import torch
    from gemm_qmm_gemv_amd import tensors
    qs, items = [], []
    for i, (n, k) in enumerate(shapes):
        q = inputs.quantized_matrix(n, k, bits, group, key=(80, seed, i, bits))
        x = inputs.activation_rows(1, k, key=(80, seed, i, bits))[0]
        dq = tensors.upload_matrix(q)
        y = torch.full((max(n, 1),), -3.0, dtype=torch.float32, device="cuda")
        items.append((dq, tensors.device_tensor(x), y))
        qs.append((q, x))
    batch = tensors.GemvBatch(items, bits, group)
    batch()
    torch.cuda.synchronize()
    return qs, [it[2].cpu().numpy() for it in items]


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
def test_batched_mixed_shapes(bits):
    shapes = [(2048, 1024), (0, 1024), (1, 64), (1000, 1024), (37, 1024), (513, 512), (3, 1024)]
    announce("batched-mixed", bits)
    qs, ys = _run_batch(shapes, bits, 64, 1)
    for (q, x), y, (n, k) in zip(qs, ys, shapes):
        if n == 0:
            assert np.all(y == -3.0)
            continue
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
        assert_within(y[:n], y_ref, a_ref, "batched b%d %dx%d" % (bits, n, k))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
def test_batched_mixed_k_one_launch(bits):
    # Different K per descriptor in one launch: each gets its own lane layout
    # (16, 32 or 64 lanes per row; two units per lane for K = 8192).
    shapes = [(300, 1024), (129, 2048), (77, 3072), (1000, 1024), (5, 768), (40, 8192), (64, 4096),
              (1, 64), (33, 2048)]
    if bits == 16:
        # fp16 rows use 32-code units: a batched launch covers K <= 4096.
        from gemm_qmm_gemv_amd import QmmError
        with pytest.raises(QmmError, match="too large for a batched launch"):
            _run_batch(shapes, bits, 64, 4)
        shapes = [s for s in shapes if s[1] <= 4096]
    announce("batched-mixed-k", bits)
    qs, ys = _run_batch(shapes, bits, 64, 4)
    for (q, x), y, (n, k) in zip(qs, ys, shapes):
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
        assert_within(y[:n], y_ref, a_ref, "batched mixed-k b%d %dx%d" % (bits, n, k))


@pytest.mark.parametrize("count", (257, 3000, 17000))
def test_batched_many_descriptors(count):
    # The launch finds each wave's first descriptor through a 256-entry
    # index of the work list: one descriptor per entry up to 256, a block of
    # ceil(count / 256) per entry above (searched by one round of 64 lanes),
    # and past 16384 blocks wider than a round (finished by the walk from
    # descriptor to descriptor).  Small matrices of mixed K, empty ones
    # among them; every row of every output checked.
    rng = np.random.default_rng(count)
    ks = (64, 1024, 2048, 3072)
    shapes = [(int(rng.integers(0, 9)) if i % 7 else 0, int(ks[rng.integers(0, 4)])) for i in range(count)]
    shapes[-1] = (5, 1024)
    announce("batched-many", count)
    qs, ys = _run_batch(shapes, 4, 64, 5)
    for i, ((q, x), y, (n, k)) in enumerate(zip(qs, ys, shapes)):
        if n == 0:
            assert np.all(y == -3.0), i
            continue
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, 4, 64)
        assert_within(y[:n], y_ref, a_ref, "batched many %d: descriptor %d" % (count, i))


@pytest.mark.parametrize("k", (2048, 3072))
def test_batched_layer_like(k):
    # Many matrices of one K, as in one launch of the decode set.
    shapes = [(1024, k)] * 6 + [(3072, k)] * 3 + [(20000, k)]
    announce("batched-layer", k)
    qs, ys = _run_batch(shapes, 4, 64, 2)
    for (q, x), y, (n, kk) in zip(qs, ys, shapes):
        rn = np.unique(np.linspace(0, n - 1, 300).astype(np.int64))
        y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, kk, 4, 64,
                                         np.zeros_like(rn), rn)
        assert_within(y[rn], y_ref, a_ref, "batched %dx%d" % (n, kk))


def test_batched_equals_single_launches():
    # Same kernel arithmetic per row as qmm_gemv with the same lane split:
    # compare to the oracle and to each other within the bound.
    import torch
    from gemm_qmm_gemv_amd import tensors
    shapes = [(3072, 1024), (1024, 1024), (2048, 1024)]
    qs, ys = _run_batch(shapes, 4, 64, 3)
    for (q, x), y, (n, k) in zip(qs, ys, shapes):
        dq = tensors.upload_matrix(q)
        ys_single = tensors.gemv(dq, tensors.device_tensor(x))
        torch.cuda.synchronize()
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, 4, 64)
        assert_within(ys_single.cpu().numpy(), y_ref, a_ref, "single")
        assert_within(y, y_ref, a_ref, "batched")


def test_batched_rejects_unprepared_descriptors():
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    q = inputs.quantized_matrix(64, 1024, 4, 64, key=(81,))
    dq = tensors.upload_matrix(q)
    x = torch.zeros(1024, dtype=torch.float16, device="cuda")
    y = torch.zeros(64, dtype=torch.float32, device="cuda")
    b = tensors.GemvBatch([(dq, x, y)], 4, 64)
    b.host[0].first_item = 5
    with pytest.raises(qmm.QmmError):
        b()
