"""Exact pins on every GEMV-family kernel, through the C ABI.

Two special cases make the product exact, so the GPU must equal the oracle
bit for bit and a layout or indexing mistake cannot hide inside the 2e-3
tolerance:

* exact integers: scale 1, min 0 (or integer fp16 weights) and integer
  activations in [-2, 2]; every product and partial sum is an integer below
  2^24, so any summation order gives the same fp32 value;
* one-hot activations x = e_j: every output is s*q[n][j] + m of its own
  weight, one rounding to fp32 of an exact value -- a wrong code position,
  group, scale or min shows up directly.

Covered here: the batched launch (mixed K: 16, 32 and 64 lanes per row, two
units per lane), the expert-rows kernel (one and two activation rows per
batch), the m = 2 GEMM route (the same kernel), the residual variant
(r = 0 and integer r), and the fused gate/up kernels, single and expert
rows (a gate sum of at least 32, where silu is the identity in fp32)."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import inputs
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8, 16)


def _exact_matrix(n, k, bits, key):
    """Scale 1, min 0 codes (or small-integer fp16 weights for bits 16)."""
    rng = inputs.rng_for(*key)
    if bits == 16:
        v = rng.integers(-3, 4, size=(n, k)).astype(np.float16)
        w = v.view(np.uint16).reshape(n, k // 2, 2)
        words = (w[:, :, 0].astype(np.uint32) | (w[:, :, 1].astype(np.uint32) << 16))
        return {"w": np.ascontiguousarray(words), "scales": None, "mins": None, "n": n, "k": k,
                "bits": 16, "group": 64}
    return {"w": inputs.packed_words(rng, n, k, bits), "scales": np.ones((n, k // 64), np.float16),
            "mins": np.zeros((n, k // 64), np.float16), "n": n, "k": k, "bits": bits, "group": 64}


def _int_x(rows, k, key):
    return inputs.rng_for(*key).integers(-2, 3, size=(rows, k)).astype(np.float16)


def _batch(items, bits):
    """items: [(q, x [k])]; one batched launch; outputs as numpy."""
    import torch
    from gemm_qmm_gemv_amd import tensors
    dev = []
    for q, x in items:
        y = torch.full((q["n"],), float("nan"), dtype=torch.float32, device="cuda")
        dev.append((tensors.upload_matrix(q), tensors.device_tensor(x), y))
    tensors.GemvBatch(dev, bits, 64)()
    torch.cuda.synchronize()
    return [d[2].cpu().numpy() for d in dev]


# 16, 32 and 64 lanes per row (K = 1024, 2048, 3072) and two units per lane
# (K = 8192); K = 768 leaves lanes of a 16-lane row idle.
MIXED = [(300, 1024), (129, 2048), (77, 3072), (5, 768), (40, 8192), (64, 4096), (33, 2048)]


def _mixed(bits):
    return [s for s in MIXED if bits != 16 or s[1] <= 4096]


@pytest.mark.parametrize("bits", BITS)
def test_batched_exact_integer(bits):
    items = []
    for i, (n, k) in enumerate(_mixed(bits)):
        items.append((_exact_matrix(n, k, bits, (90, bits, i)), _int_x(1, k, (91, bits, i))[0]))
    announce("batched-exact-int", bits)
    ys = _batch(items, bits)
    for (q, x), y in zip(items, ys):
        y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, q["n"], q["k"], bits, 64)
        assert np.array_equal(y.astype(np.float64), y_ref.reshape(-1)), (bits, q["n"], q["k"])


@pytest.mark.parametrize("bits", BITS)
def test_batched_one_hot(bits):
    # Each descriptor gets its own one-hot position: first, last and
    # group-boundary codes across the mixed lane layouts.
    items = []
    for i, (n, k) in enumerate(_mixed(bits)):
        q = inputs.quantized_matrix(n, k, bits, 64, key=(92, bits, i))
        x = np.zeros(k, np.float16)
        x[(0, k - 1, 63, 64, k // 2 + 31, 32, 1)[i % 7]] = 1.0
        items.append((q, x))
    announce("batched-one-hot", bits)
    ys = _batch(items, bits)
    for (q, x), y in zip(items, ys):
        y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, q["n"], q["k"], bits, 64)
        assert np.array_equal(y, y_ref.reshape(-1).astype(np.float32)), (bits, q["n"], q["k"])


@pytest.mark.parametrize("bits", (2, 4, 5, 8, 16))
def test_batched_equals_single_launches_bitwise(bits):
    # Same lane layout and the same per-row arithmetic as qmm_gemv: the
    # batched launch gives the single launches' results bit for bit.
    import torch
    from gemm_qmm_gemv_amd import tensors
    shapes = [(3072, 1024), (1024, 1024), (2048, 1024), (500, 1024)]
    items = [(inputs.quantized_matrix(n, k, bits, 64, key=(93, bits, i)),
              inputs.activation_rows(1, k, key=(93, bits, i))[0]) for i, (n, k) in enumerate(shapes)]
    announce("batched-vs-single", bits)
    ys = _batch(items, bits)
    for (q, x), y in zip(items, ys):
        single = tensors.gemv(tensors.upload_matrix(q), tensors.device_tensor(x))
        torch.cuda.synchronize()
        assert np.array_equal(y, single.cpu().numpy()), (bits, q["n"])


def _moe(st, x, x_rows, offsets, p_rows):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dst = tensors.upload_matrix(st)
    xd = tensors.device_tensor(x)
    xr = tensors.device_tensor(np.asarray(x_rows, np.int32)) if x_rows is not None else None
    off = tensors.device_tensor(np.asarray(offsets, np.int32))
    y = torch.full((p_rows, st["n"]), float("nan"), dtype=torch.float32, device="cuda")
    tensors.moe(dst, xd, xr, off, p_rows, y=y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _exact_stack(e, n, k, bits, key):
    qs = [_exact_matrix(n, k, bits, (*key, i)) for i in range(e)]
    st = {"w": np.stack([q["w"] for q in qs]), "n_experts": e, "n": n, "k": k, "bits": bits, "group": 64,
          "scales": None if bits == 16 else np.stack([q["scales"] for q in qs]),
          "mins": None if bits == 16 else np.stack([q["mins"] for q in qs])}
    return st


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("per_expert", (1, 3), ids=("one_row", "rows_pairs"))
def test_moe_exact_integer(bits, per_expert):
    # One row per expert runs one activation row per batch; three rows per
    # expert run two per batch and a ragged last batch.
    import gemm_qmm_gemv_amd as qmm
    e, n, k = 6, 130, 1024
    st = _exact_stack(e, n, k, bits, (94, bits))
    counts = [per_expert] * e
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    x = _int_x(4, k, (95, bits))
    x_rows = inputs.rng_for(96, bits).integers(0, 4, size=p).astype(np.int32)
    plan = qmm.qmm_get_plan(2, per_expert, n, k, bits, 64)
    announce("moe-exact-int", bits, per_expert, "rows per batch", plan["rows_per_iter"])
    y = _moe(st, x, x_rows, offsets, p)
    y_ref, _ = oracle.moe(st["w"], st["scales"], st["mins"], x, x_rows, offsets, e, n, k, bits, 64)
    assert np.array_equal(y.astype(np.float64), y_ref), (bits, per_expert)


@pytest.mark.parametrize("bits", BITS)
def test_moe_one_hot(bits):
    e, n, k = 5, 96, 2048
    st = inputs.stacked_experts(e, n, k, bits, 64, key=(97, bits))
    counts = [2, 1, 0, 3, 2]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    x = np.zeros((p, k), np.float16)
    for r in range(p):
        x[r, (r * 677 + 5) % k] = 1.0
    announce("moe-one-hot", bits)
    y = _moe(st, x, None, offsets, p)
    y_ref, _ = oracle.moe(st["w"], st["scales"], st["mins"], x, None, offsets, e, n, k, bits, 64)
    assert np.array_equal(y, y_ref.astype(np.float32)), bits


@pytest.mark.parametrize("bits", BITS)
def test_gemm_two_rows_exact(bits):
    # qmm_gemm at m = 2 takes the multi-row GEMV kernel: exact integers and
    # one-hot rows, bit for bit.
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    n, k = 333, 2048
    assert qmm.qmm_get_plan(1, 2, n, k, bits, 64)["variant"] == 1
    q = _exact_matrix(n, k, bits, (98, bits))
    x = _int_x(2, k, (99, bits))
    announce("gemm-m2-exact", bits)
    y = tensors.gemm(tensors.upload_matrix(q), tensors.device_tensor(x))
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    q = inputs.quantized_matrix(n, k, bits, 64, key=(100, bits))
    x = np.zeros((2, k), np.float16)
    x[0, 0] = 1.0
    x[1, k - 65] = 1.0
    y = tensors.gemm(tensors.upload_matrix(q), tensors.device_tensor(x))
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy(), y_ref.astype(np.float32))


@pytest.mark.parametrize("bits", BITS)
def test_residual_exact(bits):
    # r = 0: the fused residual GEMV equals the plain GEMV bit for bit; with
    # exact-integer data and an integer residual, y = r + W x exactly.
    import torch
    from gemm_qmm_gemv_amd import tensors
    n, k = 1000, 3072
    q = inputs.quantized_matrix(n, k, bits, 64, key=(101, bits))
    x = inputs.activation_rows(1, k, key=(101, bits))[0]
    dq, xd = tensors.upload_matrix(q), tensors.device_tensor(x)
    announce("residual-exact", bits)
    plain = tensors.gemv(dq, xd)
    zero = torch.zeros(n, dtype=torch.float32, device="cuda")
    fused = tensors.gemv_residual(dq, xd, zero)
    torch.cuda.synchronize()
    assert np.array_equal(fused.cpu().numpy(), plain.cpu().numpy())
    qe = _exact_matrix(n, k, bits, (102, bits))
    xe = _int_x(1, k, (103, bits))[0]
    r = inputs.rng_for(104, bits).integers(-1000, 1000, size=n).astype(np.float32)
    ye = tensors.gemv_residual(tensors.upload_matrix(qe), tensors.device_tensor(xe), tensors.device_tensor(r))
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(qe["w"], qe["scales"], qe["mins"], xe, n, k, bits, 64)
    assert np.array_equal(ye.cpu().numpy().astype(np.float64), y_ref.reshape(-1) + r.astype(np.float64))


@pytest.mark.parametrize("bits", (2, 3, 4, 8))
def test_staged_single_gemv_exact_and_residual(bits):
    # 64-lane rows with many batches per wave take the LDS-staged sweep:
    # exact integers bit for bit, the fused residual added at the flush
    # (in place), ragged row count.
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    n, k = 8195, 4096
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64, cu_count=256)
    assert pl["staged"] and pl["lanes_per_row"] == 64
    qe = _exact_matrix(n, k, bits, (105, bits))
    xe = _int_x(1, k, (106, bits))[0]
    announce("staged-exact", bits)
    dq, xd = tensors.upload_matrix(qe), tensors.device_tensor(xe)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemv(dq, xd, y)
    r = inputs.rng_for(107, bits).integers(-1000, 1000, size=n).astype(np.float32)
    rd = tensors.device_tensor(r)
    tensors.gemv_residual(dq, xd, rd, rd)
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(qe["w"], qe["scales"], qe["mins"], xe, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref.reshape(-1))
    assert np.array_equal(rd.cpu().numpy().astype(np.float64), y_ref.reshape(-1) + r.astype(np.float64))


# Fused gate/up: lanes per row x units per lane for each K.
GLU_SHAPES = [(1029, 1024, (16, 1)), (1000, 2048, (32, 1)), (1029, 3072, (16, 3)), (515, 4096, (64, 1)),
              (515, 8192, (64, 2))]


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8))
@pytest.mark.parametrize("n,k,layout", GLU_SHAPES)
def test_swiglu_exact(bits, n, k, layout):
    # Exact integers with non-negative activations x in {0, 1, 2}: both sums
    # are integers below 2^24, and the gate sum is at least 32, where
    # exp(-g) vanishes beside 1 in fp32, so silu(g) = g / 1 = g exactly and
    # h = g * u rounds once: the fused kernel must match fp32(g * u) bit for
    # bit.  A dropped or misplaced unit, group or row changes g or u by an
    # integer and h by at least u or g.
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64, cu_count=256)
    assert (pl["lanes_per_row"], pl["units_per_lane"], pl["multipass"]) == layout + (False,)
    g = _exact_matrix(n, k, bits, (108, bits, k))
    u = _exact_matrix(n, k, bits, (109, bits, k))
    x = inputs.rng_for(110, bits, k).integers(0, 3, size=k).astype(np.float16)
    g_ref, _ = oracle.qmm(g["w"], g["scales"], g["mins"], x, n, k, bits, 64)
    u_ref, _ = oracle.qmm(u["w"], u["scales"], u["mins"], x, n, k, bits, 64)
    assert g_ref.min() >= 32
    announce("swiglu-exact", bits, n, k)
    h = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemv_swiglu(tensors.upload_matrix(g), tensors.upload_matrix(u), tensors.device_tensor(x), h)
    torch.cuda.synchronize()
    h_ref = (g_ref.reshape(-1) * u_ref.reshape(-1)).astype(np.float32)
    assert np.array_equal(h.cpu().numpy(), h_ref)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8))
@pytest.mark.parametrize("k", (1024, 2048))
@pytest.mark.parametrize("per_expert", (1, 3), ids=("one_row", "rows_pairs"))
def test_moe_swiglu_exact(bits, k, per_expert):
    # The fused gate/up rows with exact integers and activations in {0, 1, 2}:
    # every gate sum is at least 32, where silu is the identity in fp32, so
    # each output must equal fp32(g * u) bit for bit (16 and 32 lanes per
    # row; one and two activation rows per batch, a ragged last batch).
    import torch
    from gemm_qmm_gemv_amd import tensors
    e, n = 6, 130
    gs = _exact_stack(e, n, k, bits, (111, bits, k))
    us = _exact_stack(e, n, k, bits, (112, bits, k))
    offsets = np.concatenate([[0], np.cumsum([per_expert] * e)]).astype(np.int32)
    p = int(offsets[-1])
    x = inputs.rng_for(113, bits, k).integers(0, 3, size=(4, k)).astype(np.float16)
    x_rows = inputs.rng_for(114, bits, k).integers(0, 4, size=p).astype(np.int32)
    g_ref, _ = oracle.moe(gs["w"], gs["scales"], gs["mins"], x, x_rows, offsets, e, n, k, bits, 64)
    u_ref, _ = oracle.moe(us["w"], us["scales"], us["mins"], x, x_rows, offsets, e, n, k, bits, 64)
    assert g_ref.min() >= 32
    announce("moe-swiglu-exact", bits, k, per_expert)
    h = torch.full((p, n), float("nan"), dtype=torch.float32, device="cuda")
    tensors.moe_swiglu(tensors.upload_matrix(gs), tensors.upload_matrix(us), tensors.device_tensor(x),
                       tensors.device_tensor(x_rows), tensors.device_tensor(offsets), p, h=h)
    torch.cuda.synchronize()
    assert np.array_equal(h.cpu().numpy(), (g_ref * u_ref).astype(np.float32))
