"""Prefill GEMM (qmm_gemm) on the GPU vs the CPU oracle."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 5, 6, 8)
PARITY_BITS = BITS + (16,)  # 16: fp16 weights


def _run_gemm(q, x, workspace="auto"):
    # Outputs start as NaN, so a tile the kernel never writes cannot pass.
    import torch
    from gemm_qmm_gemv_amd import tensors
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    ws = None if workspace == "auto" else workspace
    if workspace is None:
        ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    y = torch.full((x.shape[0], q["n"]), float("nan"), dtype=torch.float32, device="cuda")
    tensors.gemm(dq, xd, y=y, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("bits", PARITY_BITS)
@pytest.mark.parametrize("m,n,k,group", [
    (2, 130, 256, 64), (3, 64, 128, 64), (5, 200, 1024, 64), (64, 128, 512, 64),
    (100, 300, 1024, 64), (128, 512, 2048, 64), (130, 257, 320, 64), (256, 640, 768, 32),
    (17, 129, 4096, 128)])
def test_gemm_parity(bits, m, n, k, group):
    q = inputs.quantized_matrix(n, k, bits, group, key=(60, m, n, k, bits, group))
    x = inputs.activation_rows(m, k, key=(60, m, n, k, bits, group))
    announce("gemm", bits, m, n, k, group)
    y = _run_gemm(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, group)
    assert_within(y, y_ref, a_ref, "gemm b%d m%d %dx%d g%d" % (bits, m, n, k, group))


@pytest.mark.parametrize("bits", PARITY_BITS)
@pytest.mark.parametrize("tile", (32, 64, 128))
@pytest.mark.parametrize("m,n,k", [(100, 300, 1024), (130, 257, 320), (257, 384, 2048)])
def test_gemm_parity_every_tile(qmm_override, bits, tile, m, n, k):
    # Each tile height on shapes the planner would give another one.
    qmm_override("QMM_GEMM_TILE_M", tile)
    q = inputs.quantized_matrix(n, k, bits, 64, key=(62, m, n, k, bits))
    x = inputs.activation_rows(m, k, key=(62, m, n, k, bits))
    announce("gemm-tile", tile, bits, m, n, k)
    y = _run_gemm(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y, y_ref, a_ref, "gemm tile%d b%d m%d %dx%d" % (tile, bits, m, n, k))


@pytest.mark.parametrize("bits", (4, 8))
def test_gemm_without_workspace_matches_split(bits):
    # Same product with and without a K split: both within tolerance, and the
    # unsplit result is deterministic run to run.
    m, n, k = 128, 512, 4096
    q = inputs.quantized_matrix(n, k, bits, 64, key=(61, bits))
    x = inputs.activation_rows(m, k, key=(61, bits))
    announce("gemm-split-vs-none", bits)
    y_split = _run_gemm(q, x)
    y_none = _run_gemm(q, x, workspace=None)
    y_none2 = _run_gemm(q, x, workspace=None)
    assert np.array_equal(y_none, y_none2)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y_split, y_ref, a_ref, "gemm split b%d" % bits)
    assert_within(y_none, y_ref, a_ref, "gemm no-split b%d" % bits)


def test_gemm_split_workspace_reuse():
    # One zeroed workspace across a sequence of split GEMMs of different
    # shapes (and splits, with fp16 output too): each result within the bound,
    # each repeat bit-identical (the partial sums are added in split order),
    # and the arrival counters at the workspace's start back at zero after
    # every call.
    import torch
    import gemm_qmm_gemv_amd as qmm
    from gemm_qmm_gemv_amd import tensors
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    # Splits of 2 are added up inside the GEMM kernel, larger ones by a
    # separate reduction kernel: both kinds, and odd N, in one sequence.
    cases = [(128, 4096, 2048, 4), (128, 2048, 2048, 4), (512, 1024, 2048, 3), (64, 512, 8192, 4),
             (128, 2048, 8192, 8), (96, 300, 1024, 4), (128, 4100, 2048, 5), (128, 2052, 2048, 4),
             (200, 1000, 4096, 2)]
    for m, n, k, bits in cases:
        pl = qmm.qmm_get_plan(1, m, n, k, bits, 64, workspace_bytes=ws.numel())
        assert pl["split_k"] > 1, (m, n, k)
        q = inputs.quantized_matrix(n, k, bits, 64, key=(66, m, n, k, bits))
        x = inputs.activation_rows(m, k, key=(66, m, n, k))
        dq = tensors.upload_matrix(q)
        xd = tensors.device_tensor(x)
        announce("gemm-split-reuse", m, n, k, bits, pl["split_k"])
        y1 = tensors.gemm(dq, xd, workspace=ws)
        y2 = tensors.gemm(dq, xd, workspace=ws)
        h = tensors.gemm(dq, xd, workspace=ws, out_fp16=True)
        torch.cuda.synchronize()
        assert not torch.any(ws[:4096]), "arrival counters not reset"  # the partial sums follow
        assert torch.equal(y1, y2)
        y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
        assert_within(y1.cpu().numpy(), y_ref, a_ref, "split reuse %dx%dx%d" % (m, n, k))
        assert np.array_equal(h.cpu().numpy(), y1.cpu().numpy().astype(np.float16))


def test_gemm_exact_integer():
    # scale 1, min 0, integer x: fp16 weights are exact small integers, MFMA
    # products and fp32 sums stay below 2^24 -> exact.
    for bits in BITS:
        m, n, k = 96, 160, 2048
        rng = inputs.rng_for(62, bits)
        w = inputs.packed_words(rng, n, k, bits)
        s = np.ones((n, k // 64), dtype=np.float16)
        mn = np.zeros((n, k // 64), dtype=np.float16)
        x = rng.integers(-2, 3, size=(m, k)).astype(np.float16)
        q = {"w": w, "scales": s, "mins": mn, "n": n, "k": k, "bits": bits, "group": 64}
        announce("gemm-exact-int", bits)
        y = _run_gemm(q, x)
        y_ref, _ = oracle.qmm(w, s, mn, x, n, k, bits, 64)
        assert np.array_equal(y.astype(np.float64), y_ref), bits


def test_gemm_identity_activation_gives_fp16_weights():
    # X = I: Y = fp16(s*q + m)^T, the dequantized tile exactly as staged.
    k, n, bits = 128, 96, 4
    q = inputs.quantized_matrix(n, k, bits, 64, key=(63,))
    x = np.eye(k, dtype=np.float16)
    announce("gemm-identity")
    y = _run_gemm(q, x)
    wd = oracle.dequant(q["w"], q["scales"], q["mins"], n, k, bits, 64)
    assert np.array_equal(y, wd.T.astype(np.float16).astype(np.float32))


def test_gemm_rows_match_gemv():
    # Row i of a GEMM is the GEMV of x[i] (within tolerance of each other and
    # of the oracle; different kernels, so not bit-identical).
    import torch
    from gemm_qmm_gemv_amd import tensors
    m, n, k, bits = 4, 300, 1024, 4
    q = inputs.quantized_matrix(n, k, bits, 64, key=(64,))
    x = inputs.activation_rows(m, k, key=(64,))
    announce("gemm-rows-vs-gemv")
    dq = tensors.upload_matrix(q)
    y = tensors.gemm(dq, tensors.device_tensor(x))
    ys = [tensors.gemv(dq, tensors.device_tensor(x[i])) for i in range(m)]
    torch.cuda.synchronize()
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    for i in range(m):
        assert_within(ys[i].cpu().numpy(), y_ref[i], a_ref[i], "gemv row %d" % i)
    assert_within(y.cpu().numpy(), y_ref, a_ref, "gemm rows")


@pytest.mark.parametrize("m", configs.PREFILL_M)
@pytest.mark.parametrize("proj", configs.LLAMA32_1B_PROJ, ids=[p[0] for p in configs.LLAMA32_1B_PROJ])
def test_gemm_prefill_config_sampled(m, proj):
    """Llama-3.2-1B-shaped prefill at full size, in the launch configuration the
    benchmark times; 256 sampled outputs checked against the oracle."""
    name, n, k = proj
    j = [p[0] for p in configs.LLAMA32_1B_PROJ].index(name)
    q = inputs.quantized_matrix(n, k, 4, configs.GROUP, key=(configs.CFG_PREFILL, 0, j, 4))
    x = inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, j, 4, m))
    announce("gemm-prefill", m, name, n, k)
    y = _run_gemm(q, x)
    rng = np.random.default_rng(7)
    rm = rng.integers(0, m, 256)
    rn = rng.integers(0, n, 256)
    rm[:4] = [0, m - 1, 0, m - 1]
    rn[:4] = [0, 0, n - 1, n - 1]
    y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, 4, configs.GROUP, rm, rn)
    assert_within(y[rm, rn], y_ref, a_ref, "prefill m%d %s" % (m, name))
    assert np.all(np.isfinite(y))


def _run_gemm_f16(q, x, workspace="auto"):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    ws = None if workspace == "auto" else workspace
    if workspace is None:
        ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    y = torch.full((x.shape[0], q["n"]), float("nan"), dtype=torch.float16, device="cuda")
    tensors.gemm(dq, xd, y=y, workspace=ws, out_fp16=True)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("bits", (2, 4, 8, 16))
@pytest.mark.parametrize("tile", (32, 64, 128))
@pytest.mark.parametrize("m,n,k", [(1, 300, 1024), (2, 129, 512), (100, 300, 1024), (257, 384, 2048),
                                   (130, 640, 4096)])
def test_gemm_f16out_parity(qmm_override, bits, tile, m, n, k):
    qmm_override("QMM_GEMM_TILE_M", tile)
    q = inputs.quantized_matrix(n, k, bits, 64, key=(63, m, n, k, bits))
    x = inputs.activation_rows(m, k, key=(63, m, n, k, bits))
    announce("gemm-f16out", tile, bits, m, n, k)
    y = _run_gemm_f16(q, x)
    assert y.dtype == np.float16
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y, y_ref, a_ref, "gemm f16out tile%d b%d m%d %dx%d" % (tile, bits, m, n, k),
                  fp16_out=True)


@pytest.mark.parametrize("bits", (4, 16))
@pytest.mark.parametrize("split", (1, 3))
def test_gemm_f16out_is_the_rounded_fp32_result(qmm_override, bits, split):
    # Same plan, same sums: the fp16 output is the fp32 output rounded to
    # nearest even, bit for bit (with and without a K split).
    qmm_override("QMM_GEMM_SPLIT", split)
    m, n, k = 200, 520, 3072
    q = inputs.quantized_matrix(n, k, bits, 64, key=(64, bits))
    x = inputs.activation_rows(m, k, key=(64, bits))
    announce("gemm-f16out-vs-fp32", bits, split)
    y32 = _run_gemm(q, x)
    y16 = _run_gemm_f16(q, x)
    assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("out_fp16", (False, True), ids=("fp32_out", "fp16_out"))
@pytest.mark.parametrize("proj", configs.LLAMA32_1B_PROJ, ids=[p[0] for p in configs.LLAMA32_1B_PROJ])
def test_gemm_long_prefill_sampled(proj, out_fp16):
    """2048-token prefill on the Llama-3.2-1B projections, full size, in the
    benchmark's launch configuration; sampled outputs against the oracle."""
    m = configs.PREFILL_M_LONG
    name, n, k = proj
    j = [p[0] for p in configs.LLAMA32_1B_PROJ].index(name)
    q = inputs.quantized_matrix(n, k, 4, configs.GROUP, key=(configs.CFG_PREFILL, 0, j, 4))
    x = inputs.activation_rows(m, k, key=(configs.CFG_PREFILL, 0, j, 4, m))
    announce("gemm-prefill-long", m, name, out_fp16)
    y = _run_gemm_f16(q, x) if out_fp16 else _run_gemm(q, x)
    rng = np.random.default_rng(8)
    rm = rng.integers(0, m, 256)
    rn = rng.integers(0, n, 256)
    rm[:4] = [0, m - 1, 0, m - 1]
    rn[:4] = [0, 0, n - 1, n - 1]
    y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, 4, configs.GROUP, rm, rn)
    assert_within(y[rm, rn], y_ref, a_ref, "prefill m%d %s" % (m, name), fp16_out=out_fp16)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("bits", (2, 4, 5, 8, 16))
@pytest.mark.parametrize("tile", (64, 128))
@pytest.mark.parametrize("m,n,k", [(100, 300, 1024), (257, 600, 2048), (130, 520, 3072)])
def test_gemm_parity_wide_tile(qmm_override, bits, tile, m, n, k):
    # 256-column tiles (eight waves along N taking whole steps), with and
    # without the wide scale loads (K a multiple of 512 or not).
    qmm_override("QMM_GEMM_TILE_M", tile)
    qmm_override("QMM_GEMM_TILE_N", 256)
    q = inputs.quantized_matrix(n, k, bits, 64, key=(65, m, n, k, bits))
    x = inputs.activation_rows(m, k, key=(65, m, n, k, bits))
    announce("gemm-wide-tile", tile, bits, m, n, k)
    y = _run_gemm(q, x)
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
    assert_within(y, y_ref, a_ref, "gemm tile%dx256 b%d m%d %dx%d" % (tile, bits, m, n, k))
