"""Expert projection with the routing-weighted combine (qmm_moe_combine) on the
GPU vs the CPU oracle: y[token(p)] += weight(p) * W_e(p) x[row(p)]."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import ABS_TOL, REL_TOL, announce

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    from gemm_qmm_gemv_amd import tensors
    return tensors.device_tensor(np.asarray(a, dtype=dtype))


def _run(st, x, x_rows, offsets, pair_token, pair_weight, y0):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dst = tensors.upload_matrix(st)
    y = torch.from_numpy(np.asarray(y0, dtype=np.float32).copy()).cuda()
    xr = _dev(x_rows, np.int32) if x_rows is not None else None
    tensors.moe_combine(dst, tensors.device_tensor(x), xr, _dev(offsets, np.int32),
                        _dev(pair_token, np.int32), _dev(pair_weight, np.float32),
                        len(pair_token), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check(y, st, x, x_rows, offsets, pair_token, pair_weight, y0, what):
    e, n, k, bits, group = st["n_experts"], st["n"], st["k"], st["bits"], st["group"]
    yp, ap = oracle.moe(st["w"], st["scales"], st["mins"], x, x_rows, offsets, e, n, k, bits, group)
    t = y0.shape[0]
    want, a = oracle.moe_combine(yp, ap, pair_token, pair_weight, t, y0)
    # Magnitude of the terms each element sums, and how many adds it takes.
    mag, _ = oracle.moe_combine(np.abs(yp), np.zeros_like(ap), pair_token, np.abs(pair_weight), t,
                                   np.abs(y0))
    per_tok = np.bincount(np.asarray(pair_token)[(pair_token >= 0) & (pair_token < t)], minlength=t)
    wsum = oracle.moe_combine(np.ones_like(yp), np.zeros_like(ap), pair_token, np.abs(pair_weight),
                              t)[0]
    # Each pair's rows carry the projection bound, scaled by |weight|; every
    # product and atomic add rounds once more in fp32.
    bound = REL_TOL * a + ABS_TOL * wsum + (per_tok[:, None] + 2) * 2.0 ** -24 * mag + 1e-30
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), what
    bad = np.abs(y - want) > bound
    assert not bad.any(), "%s: %d outside; worst %r" % (what, int(bad.sum()),
                                                       float(np.max(np.abs(y - want) - bound)))
    print("[parity] %s: max err/bound = %.3e" % (what, float(np.max(np.abs(y - want) / bound))),
          flush=True)


@pytest.mark.parametrize("tokens", configs.MOE["tokens"])
def test_combine_down_proj_config(tokens):
    """Qwen3-30B-A3B down projection (2048 x 768 per expert, top-8 of 128),
    combined into a residual stream, every output checked."""
    e, top = configs.MOE["n_experts"], configs.MOE["top_k"]
    j = [p[0] for p in configs.MOE_PROJ].index("down_proj")
    _, n, k = configs.MOE_PROJ[j]
    st = inputs.stacked_experts(e, n, k, 4, configs.GROUP, key=(configs.CFG_MOE, j))
    r = inputs.routing(tokens, e, top, key=(configs.CFG_MOE, tokens))
    p = tokens * top
    x = inputs.activation_rows(p, k, key=(configs.CFG_MOE, tokens, 9))
    y0 = inputs.activation_rows(tokens, n, key=(configs.CFG_MOE, tokens, 10)).astype(np.float64)
    announce("moe-combine", tokens)
    y = _run(st, x, None, r["offsets"], r["pair_token"], r["pair_weight"], y0)
    _check(y, st, x, None, r["offsets"], r["pair_token"], r["pair_weight"], y0,
           "combine T%d" % tokens)


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
def test_combine_uneven_segments(bits):
    # Experts with 0, 1, 2, 5 and 9 rows, ragged N, rows read through an index.
    e, n, k, t = 7, 70, 320, 6
    st = inputs.stacked_experts(e, n, k, bits, 64, key=(72, bits))
    counts = [0, 1, 2, 0, 5, 9, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = int(offsets[-1])
    rng = inputs.rng_for(72, bits, 1)
    x = inputs.activation_rows(t, k, key=(72, bits))
    x_rows = rng.integers(0, t, size=p).astype(np.int32)
    pair_token = rng.integers(0, t, size=p).astype(np.int32)
    pair_weight = rng.uniform(-1, 1, size=p).astype(np.float32)
    y0 = inputs.activation_rows(t, n, key=(72, bits, 2)).astype(np.float64)
    announce("moe-combine-uneven", bits)
    y = _run(st, x, x_rows, offsets, pair_token, pair_weight, y0)
    _check(y, st, x, x_rows, offsets, pair_token, pair_weight, y0, "combine uneven b%d" % bits)


def test_combine_bad_indices():
    # A token index out of range adds nothing; an activation index out of
    # range adds NaN to its token's row (and only there).
    e, n, k, t = 3, 40, 256, 4
    st = inputs.stacked_experts(e, n, k, 4, 64, key=(73,))
    offsets = np.array([0, 3, 5, 8], dtype=np.int32)
    x = inputs.activation_rows(t, k, key=(73,))
    x_rows = np.array([0, 1, 2, 3, 0, 1, 2, 3], dtype=np.int32)
    pair_token = np.array([0, 1, 2, 3, 0, 1, 2, 3], dtype=np.int32)
    pair_weight = np.full(8, 0.5, dtype=np.float32)
    y0 = np.zeros((t, n))
    tok_bad = pair_token.copy()
    tok_bad[[2, 6]] = [t, -1]  # token 2 loses both of its pairs
    announce("moe-combine-bad-token")
    y = _run(st, x, x_rows, offsets, tok_bad, pair_weight, y0)
    assert np.all(y[2] == 0.0)
    _check(y, st, x, x_rows, offsets, tok_bad, pair_weight, y0, "combine bad token")
    xr_bad = x_rows.copy()
    xr_bad[3] = t  # pair 3 belongs to token 3
    announce("moe-combine-bad-row")
    y = _run(st, x, xr_bad, offsets, pair_token, pair_weight, y0)
    assert np.all(np.isnan(y[3]))
    assert np.all(np.isfinite(y[[0, 1, 2]]))


def test_combine_matches_unfused():
    # Same as qmm_moe_gemm followed by the weighted scatter-add on the host.
    import torch
    from gemm_qmm_gemv_amd import tensors
    e, top, t = 16, 4, 5
    n, k = 512, 768
    st = inputs.stacked_experts(e, n, k, 4, 64, key=(74,))
    r = inputs.routing(t, e, top, key=(74,))
    p = t * top
    x = inputs.activation_rows(p, k, key=(74, 1))
    dst = tensors.upload_matrix(st)
    yp = tensors.moe(dst, tensors.device_tensor(x), None, _dev(r["offsets"], np.int32), p)
    torch.cuda.synchronize()
    yp = yp.cpu().numpy().astype(np.float64)
    y0 = np.zeros((t, n))
    announce("moe-combine-vs-unfused")
    y = _run(st, x, None, r["offsets"], r["pair_token"], r["pair_weight"], y0)
    sep, _ = oracle.moe_combine(yp, np.zeros_like(yp), r["pair_token"], r["pair_weight"], t)
    mag, _ = oracle.moe_combine(np.abs(yp), np.zeros_like(yp), r["pair_token"],
                                np.abs(r["pair_weight"]), t)
    assert np.all(np.abs(y - sep) <= (top + 2) * 2.0 ** -24 * mag + 1e-30)


def test_combine_no_tokens_is_noop():
    import torch
    from gemm_qmm_gemv_amd import qmm_moe_combine
    z = torch.zeros(64, dtype=torch.int32, device="cuda")
    y = torch.full((1, 8), 3.0, device="cuda")
    qmm_moe_combine(z, z, z, z, None, 8, z, z, z, y, 0, 8, 2, 8, 64, 4, 64)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
