"""Decode GEMV (qmm_gemv) and code unpacking on the GPU vs the CPU oracle."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
PARITY_BITS = BITS + (16,)  # 16: fp16 weights


def _torch():
    import torch
    return torch


def _run_gemv(q, x):
    torch = _torch()
    from gemm_qmm_gemv_amd import tensors
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    y = tensors.gemv(dq, xd)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("n,k", [(1, 64), (3, 128), (17, 192), (1000, 1024), (257, 3072),
                                 (64, 8192), (33, 16384), (5, 768)])
def test_unpack_bit_exact(bits, n, k):
    from gemm_qmm_gemv_amd import tensors
    torch = _torch()
    q = inputs.quantized_matrix(n, k, bits, 64, key=(50, n, k, bits))
    announce("unpack", bits, n, k)
    dq = tensors.upload_matrix(q)
    codes = tensors.unpack(dq)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.unpack(q["w"], n, k, bits))


@pytest.mark.parametrize("bits", PARITY_BITS)
@pytest.mark.parametrize("n,k,group", [
    (1, 64, 64), (7, 64, 32), (17, 192, 64), (3072, 1024, 64), (1000, 3072, 64),
    (300, 2048, 128), (129, 768, 64), (96, 8192, 64), (40, 16384, 64), (50, 96, 32),
    (61, 4160, 64), (1031, 1024, 64)])
def test_gemv_parity(bits, n, k, group):
    q = inputs.quantized_matrix(n, k, bits, group, key=(51, n, k, bits, group))
    x = inputs.activation_rows(1, k, key=(51, n, k, bits, group))[0]
    announce("gemv", bits, n, k, group)
    y = _run_gemv(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
    assert_within(y, y_ref, a_ref, "gemv b%d %dx%d g%d" % (bits, n, k, group))


@pytest.mark.parametrize("bits", BITS)
def test_gemv_exact_integer(bits):
    # scale 1, min 0, integer x in [-2, 2]: every partial sum is an integer
    # below 2^24, so the GPU result must equal the oracle exactly.
    n, k = 300, 4096
    rng = inputs.rng_for(52, bits)
    w = inputs.packed_words(rng, n, k, bits)
    s = np.ones((n, k // 64), dtype=np.float16)
    mn = np.zeros((n, k // 64), dtype=np.float16)
    x = rng.integers(-2, 3, size=k).astype(np.float16)
    q = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
    announce("gemv-exact-int", bits)
    y = _run_gemv(q, x)
    y_ref, _ = oracle.qmm(w, s, mn, x, n, k, bits, 64)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("bits", BITS)
def test_gemv_one_hot(bits):
    # x = e_j: y[n] = s*q[n,j] + m, one rounding to fp32 of an exact value.
    n, k = 200, 1024
    q = inputs.quantized_matrix(n, k, bits, 64, key=(53, bits))
    for j in (0, 1, 5, 31, 32, 63, 64, 500, 1023):
        x = np.zeros(k, dtype=np.float16)
        x[j] = 1.0
        announce("gemv-one-hot", bits, j)
        y = _run_gemv(q, x)
        y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
        assert np.array_equal(y, y_ref.astype(np.float32)), (bits, j)


@pytest.mark.parametrize("bits", (3, 4, 8))
def test_gemv_exact_invariants_and_determinism(bits):
    # Exact for this kernel: scale and min enter only through fused
    # multiply-adds after the packed dot products, so scaling both by 2 or
    # negating both scales and negates y exactly.  Negating x goes through the
    # packed fp16 dot-product instruction, whose rounding is not symmetric
    # under a sign change, so that one is checked to the acceptance bound.
    n, k = 500, 2048
    q = inputs.quantized_matrix(n, k, bits, 64, key=(54, bits))
    x = inputs.activation_rows(1, k, key=(54, bits))[0]
    announce("gemv-invariants", bits)
    y = _run_gemv(q, x)
    y_again = _run_gemv(q, x)
    assert np.array_equal(y, y_again)
    q2 = dict(q)
    q2["scales"] = (q["scales"].astype(np.float32) * 2).astype(np.float16)
    q2["mins"] = (q["mins"].astype(np.float32) * 2).astype(np.float16)
    assert np.array_equal(_run_gemv(q2, x), 2 * y)
    q3 = dict(q, scales=-q["scales"], mins=-q["mins"])
    assert np.array_equal(_run_gemv(q3, x), -y)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], -x, n, k, bits, 64)
    assert_within(_run_gemv(q, -x), y_ref, a_ref, "gemv -x b%d" % bits)


def test_gemv_constant_codes_closed_form():
    # Codes all equal c: y = sum_g (c s_g + m_g) sum_{k in g} x_k.
    n, k, group = 64, 1024, 64
    rng = inputs.rng_for(55)
    s, mn = inputs.scales_mins(rng, n, k, group)
    x = inputs.activations(rng, 1, k)[0]
    xs = x.astype(np.float64).reshape(k // group, group).sum(axis=1)
    for bits in BITS:
        for c in (0, (1 << bits) - 1):
            w = oracle.pack(np.full((n, k), c, dtype=np.uint8), bits)
            q = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": group}
            announce("gemv-constant", bits, c)
            y = _run_gemv(q, x)
            y_cf = (c * s.astype(np.float64) + mn.astype(np.float64)) @ xs
            a = np.abs(c * s.astype(np.float64) + mn.astype(np.float64)) @ np.abs(
                x.astype(np.float64).reshape(k // group, group)).sum(axis=1)
            assert_within(y, y_cf, a, "constant b%d c%d" % (bits, c))


def test_gemv_single_q4_config():
    """The single Q4 GEMV workload, full size, every output checked."""
    c = configs.SINGLE_Q4
    q = inputs.quantized_matrix(c["n"], c["k"], 4, configs.GROUP, key=(configs.CFG_SINGLE, 0, 0, 4))
    x = inputs.activation_rows(1, c["k"], key=(configs.CFG_SINGLE, 0, 0, 4))[0]
    announce("gemv-config-single", c)
    y = _run_gemv(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, c["n"], c["k"], 4, configs.GROUP)
    assert_within(y, y_ref, a_ref, "single q4 3072x1024")


def test_gemv_zero_rows_is_noop():
    torch = _torch()
    from gemm_qmm_gemv_amd import qmm_gemv
    y = torch.full((4,), 7.0, device="cuda")
    x = torch.zeros(64, dtype=torch.float16, device="cuda")
    w = torch.zeros(64, dtype=torch.int32, device="cuda")
    s = torch.zeros(4, dtype=torch.float16, device="cuda")
    qmm_gemv(w, s, s, x, y, 0, 64, 4, 64)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("bits", PARITY_BITS)
@pytest.mark.parametrize("n,k", [(257, 3072), (64, 768), (33, 6144)])
def test_gemv_three_units_per_lane(qmm_override, bits, n, k):
    """16 lanes per row with three units each (forced): parity, and exact
    integers bit for bit."""
    import gemm_qmm_gemv_amd as qmm
    qmm_override("QMM_GEMV_LPR", 16)
    qmm_override("QMM_GEMV_XC", 3)
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64)
    assert (pl["lanes_per_row"], pl["units_per_lane"]) == (16, 3)
    q = inputs.quantized_matrix(n, k, bits, 64, key=(54, n, k, bits))
    x = inputs.activation_rows(1, k, key=(54, n, k, bits))[0]
    announce("gemv-16x3", bits, n, k, "multipass", pl["multipass"])
    y = _run_gemv(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y, y_ref, a_ref, "gemv 16x3 b%d %dx%d" % (bits, n, k))
    if bits != 16:
        rng = inputs.rng_for(55, n, k, bits)
        w = inputs.packed_words(rng, n, k, bits)
        s = np.ones((n, k // 64), dtype=np.float16)
        mn = np.zeros((n, k // 64), dtype=np.float16)
        xi = rng.integers(-2, 3, size=k).astype(np.float16)
        qe = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
        ye = _run_gemv(qe, xi)
        y_ref, _ = oracle.qmm(w, s, mn, xi, n, k, bits, 64)
        assert np.array_equal(ye.astype(np.float64), y_ref)


@pytest.mark.parametrize("bits", (2, 3, 4, 8))
def test_gemv_k3072_takes_16x3_exact_and_residual(bits):
    """K = 3072 rows (48 units) are planned as 16 lanes x 3 units with the
    activation units in LDS: exact integers bit for bit, and the fused
    residual added in place, on a ragged row count."""
    import gemm_qmm_gemv_amd as qmm
    torch = _torch()
    from gemm_qmm_gemv_amd import tensors
    n, k = 1029, 3072
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64)
    assert (pl["lanes_per_row"], pl["units_per_lane"], pl["multipass"]) == (16, 3, False)
    rng = inputs.rng_for(56, n, k, bits)
    w = inputs.packed_words(rng, n, k, bits)
    s = np.ones((n, k // 64), dtype=np.float16)
    mn = np.zeros((n, k // 64), dtype=np.float16)
    xi = rng.integers(-2, 3, size=k).astype(np.float16)
    qe = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
    announce("gemv-k3072-16x3", bits, n, k)
    dq, xd = tensors.upload_matrix(qe), tensors.device_tensor(xi)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemv(dq, xd, y)
    r = rng.integers(-1000, 1000, size=n).astype(np.float32)
    rd = tensors.device_tensor(r)
    tensors.gemv_residual(dq, xd, rd, rd)
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(w, s, mn, xi, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref.reshape(-1))
    assert np.array_equal(rd.cpu().numpy().astype(np.float64), y_ref.reshape(-1) + r.astype(np.float64))


@pytest.mark.parametrize("bits", (2, 3, 4, 8))
@pytest.mark.parametrize("staged", (0, 1))
def test_gemv_16x3_staged_and_unstaged_exact(qmm_override, bits, staged):
    """The 16 x 3 layout through both loops -- row sums staged in LDS (Q4 and
    wider) and stored per batch -- with every output NaN-prefilled: exact
    integers bit for bit, the residual added in place."""
    import gemm_qmm_gemv_amd as qmm
    torch = _torch()
    from gemm_qmm_gemv_amd import tensors
    qmm_override("QMM_GEMV_STAGED", staged)
    n, k = 8195, 3072
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64)
    assert (pl["lanes_per_row"], pl["units_per_lane"]) == (16, 3)
    assert pl["staged"] == (bool(staged) and bits >= 4)
    rng = inputs.rng_for(57, n, k, bits)
    w = inputs.packed_words(rng, n, k, bits)
    s = np.ones((n, k // 64), dtype=np.float16)
    mn = np.zeros((n, k // 64), dtype=np.float16)
    xi = rng.integers(-2, 3, size=k).astype(np.float16)
    qe = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
    announce("gemv-16x3-staged", staged, bits)
    dq, xd = tensors.upload_matrix(qe), tensors.device_tensor(xi)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemv(dq, xd, y)
    r = rng.integers(-1000, 1000, size=n).astype(np.float32)
    rd = tensors.device_tensor(r)
    tensors.gemv_residual(dq, xd, rd, rd)
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(w, s, mn, xi, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref.reshape(-1))
    assert np.array_equal(rd.cpu().numpy().astype(np.float64), y_ref.reshape(-1) + r.astype(np.float64))
    q = inputs.quantized_matrix(n, k, bits, 64, key=(58, bits))
    x = inputs.activation_rows(1, k, key=(58, bits))[0]
    yq = _run_gemv(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(yq, y_ref, a_ref, "gemv 16x3 staged=%d b%d" % (staged, bits))


@pytest.mark.parametrize("late", (0, 1))
@pytest.mark.parametrize("n,k", ((5, 1024), (777, 128), (3075, 1024), (1029, 2048), (20011, 1024)))
def test_gemv_q4_late_unit_build_exact(qmm_override, late, n, k):
    """Q4 rows of one unit per lane (K up to 2048) with the activation units
    built before or after the first weight loads, including launches where
    most waves have no rows (every wave still reaches the LDS barrier) and
    two rows per slot: exact integers bit for bit on NaN-prefilled outputs,
    the residual added in place, and seeded inputs within tolerance."""
    import gemm_qmm_gemv_amd as qmm
    torch = _torch()
    from gemm_qmm_gemv_amd import tensors
    bits = 4
    qmm_override("QMM_GEMV_LATE", late)
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, 64)
    assert pl["units_per_lane"] == 1 and pl["lanes_per_row"] <= 32 and not pl["multipass"]
    assert pl["late"] == bool(late)
    rng = inputs.rng_for(61, n, k, bits)
    w = inputs.packed_words(rng, n, k, bits)
    s = np.ones((n, k // 64), dtype=np.float16)
    mn = np.zeros((n, k // 64), dtype=np.float16)
    xi = rng.integers(-2, 3, size=k).astype(np.float16)
    qe = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
    announce("gemv-q4-late", late, n, k)
    dq, xd = tensors.upload_matrix(qe), tensors.device_tensor(xi)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemv(dq, xd, y)
    r = rng.integers(-1000, 1000, size=n).astype(np.float32)
    rd = tensors.device_tensor(r)
    tensors.gemv_residual(dq, xd, rd, rd)
    torch.cuda.synchronize()
    y_ref, _ = oracle.qmm(w, s, mn, xi, n, k, bits, 64)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref.reshape(-1))
    assert np.array_equal(rd.cpu().numpy().astype(np.float64), y_ref.reshape(-1) + r.astype(np.float64))
    q = inputs.quantized_matrix(n, k, bits, 64, key=(62, n, k))
    x = inputs.activation_rows(1, k, key=(62, n, k))[0]
    yq = _run_gemv(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(yq, y_ref, a_ref, "gemv q4 late=%d %dx%d" % (late, n, k))
