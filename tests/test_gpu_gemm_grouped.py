"""Grouped prefill GEMM (qmm_gemm_grouped) on the GPU vs the CPU oracle:
several weight matrices sharing X in one launch."""
import numpy as np
import pytest

import oracle
from gemm_qmm_gemv_amd import configs, inputs
from tests.gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu


def _members(ns, k, bits, seed):
    return [inputs.quantized_matrix(n, k, bits, 64, key=(130, seed, i, n, k, bits)) for i, n in enumerate(ns)]


def _run(qs, x, workspace=None):
    import torch
    from gemm_qmm_gemv_amd import tensors
    dqs = [tensors.upload_matrix(q) for q in qs]
    # Outputs start as NaN, so a tile no member's work-group writes cannot pass.
    ys = [torch.full((x.shape[0], q["n"]), float("nan"), dtype=torch.float32, device="cuda") for q in qs]
    tensors.gemm_grouped(dqs, tensors.device_tensor(x), ys=ys, workspace=workspace)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def _check(ys, qs, x, what, sample=None):
    m, k = x.shape
    for i, (y, q) in enumerate(zip(ys, qs)):
        n, bits = q["n"], q["bits"]
        if sample is None:
            y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, n, k, bits, 64)
            assert_within(y, y_ref, a_ref, "%s member %d" % (what, i))
        else:
            rng = np.random.default_rng(i)
            rm = rng.integers(0, m, sample)
            rn = rng.integers(0, n, sample)
            rm[:2], rn[:2] = [0, m - 1], [n - 1, 0]
            y_ref, a_ref = oracle.qmm_sample(q["w"], q["scales"], q["mins"], x, k, bits, 64, rm, rn)
            assert_within(y[rm, rn], y_ref, a_ref, "%s member %d (sampled)" % (what, i))
            assert np.all(np.isfinite(y))


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
@pytest.mark.parametrize("m,ns,k", [(3, [300, 77], 512), (64, [256, 128, 128], 1024),
                                    (128, [512, 128, 128], 2048), (200, [384, 96, 200, 64], 1024)])
def test_grouped_parity(bits, m, ns, k):
    qs = _members(ns, k, bits, 1)
    x = inputs.activation_rows(m, k, key=(131, m, k, bits))
    announce("gemm-grouped", bits, m, ns, k)
    _check(_run(qs, x), qs, x, "grouped b%d m%d" % (bits, m))


@pytest.mark.parametrize("force_one_launch", [False, True])
@pytest.mark.parametrize("m", tuple(configs.PREFILL_M) + (2048,))
@pytest.mark.parametrize("group", ["qkv", "gate_up"])
def test_grouped_prefill_layer_sampled(qmm_override, m, group, force_one_launch):
    """The Llama-3.2-1B layer's q|k|v and gate|up groups at full size, as the
    benchmark launches them (and forced into one launch where the library
    would launch the members separately); sampled outputs of every member."""
    if force_one_launch:
        qmm_override("QMM_GEMM_GROUPED", 1)
    names = ["q_proj", "k_proj", "v_proj"] if group == "qkv" else ["gate_proj", "up_proj"]
    projs = {p[0]: (j, p) for j, p in enumerate(configs.LLAMA32_1B_PROJ)}
    qs = []
    for name in names:
        j, (_, n, k) = projs[name]
        qs.append(inputs.quantized_matrix(n, k, 4, configs.GROUP, key=(configs.CFG_PREFILL, 0, j, 4)))
    j0 = projs[names[0]][0]
    x = inputs.activation_rows(m, qs[0]["k"], key=(configs.CFG_PREFILL, 0, j0, 4, m))
    announce("gemm-grouped-layer", m, group)
    _check(_run(qs, x), qs, x, "grouped %s m%d" % (group, m), sample=256)


def test_grouped_deterministic_and_counters_reset():
    import torch
    from gemm_qmm_gemv_amd import tensors
    import gemm_qmm_gemv_amd as qmm
    m, k = 128, 2048
    qs = _members([2048, 512, 512], k, 4, 2)
    x = inputs.activation_rows(m, k, key=(132,))
    dqs = [tensors.upload_matrix(q) for q in qs]
    xd = tensors.device_tensor(x)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    members = [(d["w"], d["scales"], d["mins"], None, d["n"]) for d in dqs]
    assert qmm.qmm_gemm_grouped_workspace_bytes(members, m, k, 4, 64) > 4096  # plans a K split
    announce("gemm-grouped-repeat")
    a = tensors.gemm_grouped(dqs, xd, workspace=ws)
    b = tensors.gemm_grouped(dqs, xd, workspace=ws)
    torch.cuda.synchronize()
    assert not torch.any(ws[:4096]), "arrival counters not reset"
    for ya, yb in zip(a, b):
        assert torch.equal(ya, yb)
    _check([y.cpu().numpy() for y in a], qs, x, "grouped repeat")


def test_grouped_skips_empty_members_and_matches_plain():
    import torch
    from gemm_qmm_gemv_amd import tensors
    m, k = 96, 1024
    q = _members([640], k, 4, 3)[0]
    x = inputs.activation_rows(m, k, key=(133,))
    dq = tensors.upload_matrix(q)
    xd = tensors.device_tensor(x)
    empty = dict(dq, n=0)
    announce("gemm-grouped-empty")
    y_empty = torch.full((1, 1), 5.0, device="cuda")
    ys = tensors.gemm_grouped([empty, dq], xd, ys=[y_empty, torch.empty((m, 640), device="cuda")])
    y_plain = tensors.gemm(dq, xd)
    torch.cuda.synchronize()
    assert float(y_empty[0, 0]) == 5.0
    y_ref, a_ref = oracle.qmm(q["w"], q["scales"], q["mins"], x, 640, k, 4, 64)
    assert_within(ys[1].cpu().numpy(), y_ref, a_ref, "grouped one member")
    assert_within(y_plain.cpu().numpy(), y_ref, a_ref, "plain")
