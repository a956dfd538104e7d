"""Prefill GEMM with the weights dequantized into LDS (gemm_wl.hip), forced
through the launch-plan override on every tile shape, against the CPU oracle:
tolerance on random data, bit-exact on the exact cases (integer products,
identity activations), K splits summed in the kernel and by the separate
reduction, fp16 output, and the full-size prefill shapes with every output
prefilled with NaN so that an unwritten tile cannot pass."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8, 16)
TILES = ((128, 128), (256, 128), (128, 256), (256, 256))


def _force(qmm_override, tm, tn, split=0):
    qmm_override("QMM_GEMM_KERNEL", 1)
    qmm_override("QMM_GEMM_TILE_M", tm)
    qmm_override("QMM_GEMM_TILE_N", tn)
    if split:
        qmm_override("QMM_GEMM_SPLIT", split)


def _run(q, x, out_fp16=False, workspace="auto"):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    m = x.shape[0]
    y = torch.full((m, q["n"]), float("nan"), dtype=torch.float16 if out_fp16 else torch.float32,
                   device="cuda")
    ws = None
    if workspace is None:
        ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    tensors.gemm(dq, xd, y=y, workspace=ws, out_fp16=out_fp16)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _plan(m, n, k, bits, group=64):
    import gemm_qmm_gemv_amd as qmm
    return qmm.qmm_get_plan(1, m, n, k, bits, group, workspace_bytes=1 << 40)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("tm,tn", TILES)
@pytest.mark.parametrize("m,n,k,group", [(100, 300, 1024, 64), (257, 200, 2048, 64), (300, 130, 352, 32),
                                         (3, 70, 4096, 128)])
def test_wl_parity(qmm_override, bits, tm, tn, m, n, k, group):
    _force(qmm_override, tm, tn)
    pl = _plan(m, n, k, bits, group)
    assert pl["variant"] == 4 and (pl["tile_m"], pl["tile_n"]) == (tm, tn)
    q = inputs.quantized_matrix(n, k, bits, group, key=(70, m, n, k, bits, group))
    x = inputs.activation_rows(m, k, key=(70, m, n, k, bits, group))
    announce("gemm-wl", tm, tn, bits, m, n, k, group, "split", pl["split_k"])
    y = _run(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
    assert_within(y, y_ref, a_ref, "gemm-wl %dx%d b%d m%d %dx%d g%d" % (tm, tn, bits, m, n, k, group))


@pytest.mark.parametrize("tm,tn", TILES)
def test_wl_exact_integer(qmm_override, tm, tn):
    # s = 1, m = 0, integer x in [-2, 2]: every product and partial sum is an
    # integer below 2^24, so the result equals the oracle bit for bit.
    _force(qmm_override, tm, tn)
    for bits in BITS[:-1]:
        m, n, k = 150, 200, 2048
        rng = inputs.rng_for(71, bits)
        w = inputs.packed_words(rng, n, k, bits)
        s = np.ones((n, k // 64), dtype=np.float16)
        mn = np.zeros((n, k // 64), dtype=np.float16)
        x = rng.integers(-2, 3, size=(m, k)).astype(np.float16)
        q = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
        announce("gemm-wl-exact-int", tm, tn, bits)
        y = _run(q, x)
        y_ref, _ = oracle.qmm(w, s, mn, x, n, k, bits, 64)
        assert np.array_equal(y.astype(np.float64), y_ref), (tm, tn, bits)


@pytest.mark.parametrize("tm,tn", TILES)
@pytest.mark.parametrize("bits", BITS)
def test_wl_identity_activation_gives_fp16_weights(qmm_override, tm, tn, bits):
    # X = I: Y = fp16(s*q + m)^T exactly -- every weight lands at its own k
    # (a wrong permute, block or lane-half assignment moves it).
    _force(qmm_override, tm, tn)
    k, n = 512, 160
    q = inputs.quantized_matrix(n, k, bits, 64, key=(72, bits))
    x = np.eye(k, dtype=np.float16)
    announce("gemm-wl-identity", tm, tn, bits)
    y = _run(q, x)
    # The oracle's exact product with X = I is W^T in fp64; one rounding to
    # fp16 is what the kernel stages (fp16 weights: already exact).
    y_ref, _ = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert np.array_equal(y, y_ref.astype(np.float16).astype(np.float32))


@pytest.mark.parametrize("split", (2, 3, 4))
@pytest.mark.parametrize("tm,tn", ((128, 128), (256, 128), (256, 256)))
def test_wl_splits(qmm_override, tm, tn, split):
    # Two splits are summed in the kernel, more by the separate reduction;
    # both within the bound, deterministic, and the fp16 output is the fp32
    # result rounded once.
    _force(qmm_override, tm, tn, split)
    m, n, k, bits = 200, 520, 3072, 4
    assert _plan(m, n, k, bits)["split_k"] == split
    q = inputs.quantized_matrix(n, k, bits, 64, key=(73, split))
    x = inputs.activation_rows(m, k, key=(73, split))
    announce("gemm-wl-split", tm, tn, split)
    y1 = _run(q, x)
    y2 = _run(q, x)
    h = _run(q, x, out_fp16=True)
    assert np.array_equal(y1, y2)
    assert np.array_equal(h.view(np.uint16), y1.astype(np.float16).view(np.uint16))
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y1, y_ref, a_ref, "gemm-wl split%d %dx%d" % (split, tm, tn))


@pytest.mark.parametrize("m", configs.PREFILL_M + (configs.PREFILL_M_LONG,))
@pytest.mark.parametrize("proj", configs.LLAMA32_1B_PROJ, ids=[p[0] for p in configs.LLAMA32_1B_PROJ])
def test_wl_prefill_config_sampled(qmm_override, m, proj):
    """Full-size Llama-3.2-1B prefill shapes on the LDS kernel with its own
    tile and split choice; 256 sampled outputs against the oracle and every
    output written (NaN prefill)."""
    qmm_override("QMM_GEMM_KERNEL", 1)
    name, n, k = proj
    j = [p[0] for p in configs.LLAMA32_1B_PROJ].index(name)
    q = inputs.quantized_matrix(n, k, 4, configs.GROUP, key=(configs.CFG_PREFILL, 0, j, 4))
    x = inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, j, 4, m))
    pl = _plan(m, n, k, 4)
    announce("gemm-wl-prefill", m, name, pl["tile_m"], pl["tile_n"], pl["split_k"])
    y = _run(q, x)
    assert np.all(np.isfinite(y)), "unwritten outputs"
    rng = np.random.default_rng(9)
    rm = rng.integers(0, m, 256)
    rn = rng.integers(0, n, 256)
    rm[:4] = [0, m - 1, 0, m - 1]
    rn[:4] = [0, 0, n - 1, n - 1]
    y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, 4, configs.GROUP, rm, rn)
    assert_within(y[rm, rn], y_ref, a_ref, "gemm-wl prefill m%d %s" % (m, name))


@pytest.mark.parametrize("bits", (2, 4, 5, 16))
@pytest.mark.parametrize("tm,tn", TILES)
@pytest.mark.parametrize("m,ns,k", [(200, [300, 77, 130], 1024), (64, [512, 128, 128], 2048),
                                    (300, [256, 520], 512)])
def test_wl_grouped_parity(qmm_override, bits, tm, tn, m, ns, k):
    """Grouped launches on the LDS kernel (one launch forced): every member
    against the oracle, K splits summed in the kernel, outputs NaN-prefilled."""
    import torch
    from gemm_qmm_gemv_amd import tensors
    _force(qmm_override, tm, tn)
    qmm_override("QMM_GEMM_GROUPED", 1)
    qs = [inputs.quantized_matrix(n, k, bits, 64, key=(74, m, k, bits, i, n)) for i, n in enumerate(ns)]
    x = inputs.activation_rows(m, k, key=(74, m, k, bits))
    announce("gemm-wl-grouped", tm, tn, bits, m, ns, k)
    dqs = [tensors.upload_matrix(q) for q in qs]
    ys = [torch.full((m, q["n"]), float("nan"), dtype=torch.float32, device="cuda") for q in qs]
    tensors.gemm_grouped(dqs, tensors.device_tensor(x), ys=ys)
    ys2 = [torch.full((m, q["n"]), float("nan"), dtype=torch.float32, device="cuda") for q in qs]
    tensors.gemm_grouped(dqs, tensors.device_tensor(x), ys=ys2)
    torch.cuda.synchronize()
    for i, (q, y, y2) in enumerate(zip(qs, ys, ys2)):
        yh = y.cpu().numpy()
        assert np.array_equal(yh, y2.cpu().numpy()), "member %d not deterministic" % i
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, q["n"], k, bits, 64)
        assert_within(yh, y_ref, a_ref, "gemm-wl grouped %dx%d b%d member %d" % (tm, tn, bits, i))
