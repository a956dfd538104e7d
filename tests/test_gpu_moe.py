"""Mixture-of-experts projections (qmm_moe_gemm) on the GPU vs the CPU oracle."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu


def _run_moe(st, x, x_rows, offsets, p_rows):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dst = tensors.upload_matrix(st)
    xd = tensors.device_tensor(x)
    xr = tensors.device_tensor(np.asarray(x_rows, dtype=np.int32)) if x_rows is not None else None
    off = tensors.device_tensor(np.asarray(offsets, dtype=np.int32))
    y = torch.full((p_rows, st["n"]), -7.0, dtype=torch.float32, device="cuda")
    tensors.moe(dst, xd, xr, off, p_rows, y=y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("tokens", configs.MOE["tokens"])
@pytest.mark.parametrize("proj", configs.MOE_PROJ, ids=[p[0] for p in configs.MOE_PROJ])
def test_moe_config(tokens, proj):
    """Qwen3-30B-A3B-shaped experts, top-8 of 128, full size, every output."""
    name, n, k = proj
    j = [p[0] for p in configs.MOE_PROJ].index(name)
    e, top = configs.MOE["n_experts"], configs.MOE["top_k"]
    st = inputs.stacked_experts(e, n, k, 4, configs.GROUP, key=(configs.CFG_MOE, j))
    r = inputs.routing(tokens, e, top, key=(configs.CFG_MOE, tokens))
    p = tokens * top
    if name == "down_proj":
        # The down projection reads one activation row per (token, expert) pair.
        x = inputs.activation_rows(p, k, key=(configs.CFG_MOE, tokens, 9))
        x_rows = None
    else:
        x = inputs.activation_rows(tokens, k, key=(configs.CFG_MOE, tokens))
        x_rows = r["pair_token"]
    announce("moe", tokens, name)
    y = _run_moe(st, x, x_rows, r["offsets"], p)
    y_ref, a_ref = oracle.moe(st["w"], st["scales"], st["mins"], x, x_rows, r["offsets"],
                              e, n, k, 4, configs.GROUP)
    assert_within(y, y_ref, a_ref, "moe T%d %s" % (tokens, name))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
def test_moe_uneven_segments(bits):
    # Experts with 0, 1, 2, 5 and 9 rows, ragged N, an out-of-range index.
    e, n, k = 7, 70, 320
    st = inputs.stacked_experts(e, n, k, bits, 64, key=(70, bits))
    counts = [0, 1, 2, 0, 5, 9, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    t = 6
    x = inputs.activation_rows(t, k, key=(70, bits))
    rng = inputs.rng_for(70, bits, 1)
    x_rows = rng.integers(0, t, size=p).astype(np.int32)
    announce("moe-uneven", bits)
    y = _run_moe(st, x, x_rows, offsets, p)
    y_ref, a_ref = oracle.moe(st["w"], st["scales"], st["mins"], x, x_rows, offsets, e, n, k, bits, 64)
    assert_within(y, y_ref, a_ref, "moe uneven b%d" % bits)
    # An activation index out of range gives a NaN row and nothing else changes.
    bad = x_rows.copy()
    bad[3] = t + 5
    y_bad = _run_moe(st, x, bad, offsets, p)
    assert np.all(np.isnan(y_bad[3]))
    keep = np.ones(p, bool)
    keep[3] = False
    assert np.array_equal(y_bad[keep], y[keep])


def test_moe_rows_equal_per_expert_gemv():
    # Each MoE row equals qmm_gemv on that expert's matrix (same kernel family,
    # both checked against the oracle).
    import torch
    from gemm_qmm_gemv_amd import tensors
    e, n, k, tokens = 16, 256, 2048, 3
    st = inputs.stacked_experts(e, n, k, 4, 64, key=(71,))
    r = inputs.routing(tokens, e, 4, key=(71,))
    x = inputs.activation_rows(tokens, k, key=(71,))
    p = tokens * 4
    announce("moe-vs-gemv")
    y = _run_moe(st, x, r["pair_token"], r["offsets"], p)
    y_ref, a_ref = oracle.moe(st["w"], st["scales"], st["mins"], x, r["pair_token"], r["offsets"],
                              e, n, k, 4, 64)
    assert_within(y, y_ref, a_ref, "moe small")
    for pi in range(p):
        ex = int(r["pair_expert"][pi])
        q = {"w": st["w"][ex], "scales": st["scales"][ex], "mins": st["mins"][ex],
             "n": n, "k": k, "bits": 4, "group": 64}
        dq = tensors.upload_matrix(q)
        yg = tensors.gemv(dq, tensors.device_tensor(x[r["pair_token"][pi]]))
        torch.cuda.synchronize()
        assert_within(yg.cpu().numpy(), y_ref[pi], a_ref[pi], "gemv expert %d" % ex)


def test_moe_more_row_batches_than_grid_rows():
    # 140000 (token, expert) pairs over three experts: more row batches than
    # one launch grid has work-group rows, so each row of work-groups takes
    # several batches in turn.
    e, n, k = 3, 16, 64
    st = inputs.stacked_experts(e, n, k, 4, 64, key=(72,))
    counts = [60000, 0, 80000]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    x = inputs.activation_rows(p, k, key=(72,))
    announce("moe-many-pairs", p)
    y = _run_moe(st, x, None, offsets, p)
    y_ref, a_ref = oracle.moe(st["w"], st["scales"], st["mins"], x, None, offsets, e, n, k, 4, 64)
    assert_within(y, y_ref, a_ref, "moe many pairs")


def _run_moe_glu(sg, su, x, x_rows, offsets, p_rows):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dg, du = tensors.upload_matrix(sg), tensors.upload_matrix(su)
    xd = tensors.device_tensor(x)
    xr = tensors.device_tensor(np.asarray(x_rows, dtype=np.int32)) if x_rows is not None else None
    off = tensors.device_tensor(np.asarray(offsets, dtype=np.int32))
    h = torch.full((p_rows, sg["n"]), -7.0, dtype=torch.float32, device="cuda")
    tensors.moe_swiglu(dg, du, xd, xr, off, p_rows, h=h)
    torch.cuda.synchronize()
    return h.cpu().numpy()


def _check_glu(h, sg, su, x, x_rows, offsets, what):
    from tests.gpu_util import glu_bound
    e, n, k, bits, group = sg["n_experts"], sg["n"], sg["k"], sg["bits"], sg["group"]
    g, ag = oracle.moe(sg["w"], sg["scales"], sg["mins"], x, x_rows, offsets, e, n, k, bits, group)
    u, au = oracle.moe(su["w"], su["scales"], su["mins"], x, x_rows, offsets, e, n, k, bits, group)
    ref = oracle.silu(g) * u
    bound = glu_bound(g, ag, u, au)
    assert np.all(np.isfinite(h)), what
    err = np.abs(h.astype(np.float64) - ref)
    assert np.all(err <= bound), "%s: %d outside" % (what, int((err > bound).sum()))
    print("[parity] %s: max err/bound = %.3e" % (what, float(np.max(err / bound))), flush=True)


@pytest.mark.parametrize("tokens", configs.MOE["tokens"])
def test_moe_swiglu_config(tokens):
    """Qwen3-30B-A3B-shaped gate and up experts fused with the SiLU-gated
    product, top-8 of 128, full size, every output."""
    e, top = configs.MOE["n_experts"], configs.MOE["top_k"]
    _, n, k = configs.MOE_PROJ[0]
    sg = inputs.stacked_experts(e, n, k, 4, configs.GROUP, key=(configs.CFG_MOE, 0))
    su = inputs.stacked_experts(e, n, k, 4, configs.GROUP, key=(configs.CFG_MOE, 1))
    r = inputs.routing(tokens, e, top, key=(configs.CFG_MOE, tokens))
    x = inputs.activation_rows(tokens, k, key=(configs.CFG_MOE, tokens))
    announce("moe-swiglu", tokens)
    h = _run_moe_glu(sg, su, x, r["pair_token"], r["offsets"], tokens * top)
    _check_glu(h, sg, su, x, r["pair_token"], r["offsets"], "moe swiglu T%d" % tokens)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
def test_moe_swiglu_uneven_segments(bits):
    e, n, k = 7, 70, 320
    sg = inputs.stacked_experts(e, n, k, bits, 64, key=(71, bits, 0))
    su = inputs.stacked_experts(e, n, k, bits, 64, key=(71, bits, 1))
    counts = [0, 1, 2, 0, 5, 9, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    t = 6
    x = inputs.activation_rows(t, k, key=(71, bits))
    x_rows = inputs.rng_for(71, bits, 2).integers(0, t, size=p).astype(np.int32)
    announce("moe-swiglu-uneven", bits)
    h = _run_moe_glu(sg, su, x, x_rows, offsets, p)
    _check_glu(h, sg, su, x, x_rows, offsets, "moe swiglu uneven b%d" % bits)
    bad = x_rows.copy()
    bad[4] = -1
    h_bad = _run_moe_glu(sg, su, x, bad, offsets, p)
    assert np.all(np.isnan(h_bad[4]))
    keep = np.ones(p, bool)
    keep[4] = False
    assert np.array_equal(h_bad[keep], h[keep])


def test_moe_swiglu_unsupported_k():
    from gemm_qmm_gemv_amd import QmmError
    sg = inputs.stacked_experts(2, 16, 16384, 4, 64, key=(72, 0))
    su = inputs.stacked_experts(2, 16, 16384, 4, 64, key=(72, 1))
    x = inputs.activation_rows(2, 16384, key=(72,))
    with pytest.raises(QmmError, match="more than one pass"):
        _run_moe_glu(sg, su, x, None, [0, 1, 2], 2)
