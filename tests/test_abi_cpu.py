"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, rejects bad arguments before touching a device, and plans launches
from integers alone."""
import ctypes
import os
import re

import pytest

import gemm_qmm_gemv_amd as qmm
from gemm_qmm_gemv_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")

A16 = 0x10000  # a 16-byte aligned stand-in address; never dereferenced here


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qmm.library_path()):
        from gemm_qmm_gemv_amd import build
        build.build()
    return qmm.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^QMM_API\s+[\w\s\*]+?\b(qmm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_python_surface():
    assert sorted(qmm.EXPORTED_SYMBOLS) == header_functions()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert qmm.qmm_abi_version() == 3


def test_exports_are_only_the_abi(lib):
    # nm -D lists the dynamic symbols; every qmm_ symbol must be declared.
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qmm.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if " T qmm_" in ln})
    assert exported == header_functions()


def test_status_strings(lib):
    assert qmm.qmm_status_string(0) == "QMM_OK"
    assert qmm.qmm_status_string(3) == "QMM_ERR_MISALIGNED"
    assert qmm.qmm_status_string(99) == "QMM_ERR_UNKNOWN"


def _gemv(lib, w=A16, s=A16, m=A16, x=A16, y=A16, n=64, k=128, bits=4, g=64):
    p = ctypes.c_void_p
    return lib.qmm_gemv(p(w), p(s), p(m), p(x), p(y), n, k, bits, g, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(bits=7), qmm.QMM_ERR_UNSUPPORTED),
    (dict(bits=1), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(bits=9), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(bits=17), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(g=48), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(g=0), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(k=96, g=64), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(k=0), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(n=-1), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(w=0), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(x=0), qmm.QMM_ERR_INVALID_ARGUMENT),
    (dict(w=A16 + 4), qmm.QMM_ERR_MISALIGNED),
    (dict(x=A16 + 8), qmm.QMM_ERR_MISALIGNED),
    (dict(y=A16 + 4), qmm.QMM_ERR_MISALIGNED),
    (dict(s=A16 + 1), qmm.QMM_ERR_MISALIGNED),
    (dict(n=0, w=0, x=0), qmm.QMM_OK),
])
def test_gemv_argument_checks(lib, kwargs, status):
    assert _gemv(lib, **kwargs) == status
    if status != qmm.QMM_OK:
        assert qmm.qmm_last_error() != ""


def test_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _gemv(lib) == qmm.QMM_ERR_DEVICE
    assert "device" in qmm.qmm_last_error()


def test_gemm_and_moe_argument_checks(lib):
    p = ctypes.c_void_p
    g = lib.qmm_gemm
    assert g(p(A16), p(A16), p(A16), p(A16), p(A16), -1, 64, 128, 4, 64, None, 0, None) == \
        qmm.QMM_ERR_INVALID_ARGUMENT
    assert g(p(A16), p(A16), p(A16), p(A16), p(A16), 0, 64, 128, 4, 64, None, 0, None) == qmm.QMM_OK
    assert g(p(A16), p(A16), p(A16), p(A16), p(A16), 8, 64, 128, 4, 64, None, 64, None) == \
        qmm.QMM_ERR_INVALID_ARGUMENT  # bytes without a buffer
    assert g(p(A16), p(A16), p(A16), p(A16), p(A16), 8, 64, 128, 4, 64, p(A16 + 4), 64, None) == \
        qmm.QMM_ERR_MISALIGNED
    na = lib.qmm_gemm_noalloc
    assert na(p(A16), p(A16), p(A16), p(A16), p(A16), -1, 64, 128, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert na(p(A16), p(A16), p(A16), p(A16), p(A16), 0, 64, 128, 4, 64, None) == qmm.QMM_OK
    assert na(p(A16), p(A16), p(A16), p(A16), p(A16 + 4), 8, 64, 128, 4, 64, None) == qmm.QMM_ERR_MISALIGNED
    assert na(p(A16), p(A16), p(A16), None, p(A16), 8, 64, 128, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert na(p(A16), p(A16), p(A16), p(A16), p(A16), 8, 64, 128, 7, 64, None) == qmm.QMM_ERR_UNSUPPORTED
    mo = lib.qmm_moe_gemm
    assert mo(p(A16), p(A16), p(A16), p(A16), None, 4, p(A16), p(A16), 8, 2, 64, 128, 4, 64, None) == \
        qmm.QMM_ERR_INVALID_ARGUMENT  # no index and too few x rows
    assert mo(p(A16), p(A16), p(A16), p(A16), None, 8, None, p(A16), 8, 2, 64, 128, 4, 64, None) == \
        qmm.QMM_ERR_INVALID_ARGUMENT  # no offsets
    assert mo(p(A16), p(A16), p(A16), p(A16), None, 8, p(A16 + 2), p(A16), 8, 2, 64, 128, 4, 64,
              None) == qmm.QMM_ERR_MISALIGNED
    assert mo(p(A16), p(A16), p(A16), p(A16), None, 8, p(A16), p(A16), 0, 2, 64, 128, 4, 64, None) == \
        qmm.QMM_OK
    assert lib.qmm_unpack(p(A16), p(A16 + 8), 4, 64, 4, None) == qmm.QMM_ERR_MISALIGNED
    assert lib.qmm_unpack(p(A16), p(A16), 4, 64, 7, None) == qmm.QMM_ERR_UNSUPPORTED
    # fp16 weights (bits 16) hold no codes to unpack.
    assert lib.qmm_unpack(p(A16), p(A16), 4, 64, 16, None) == qmm.QMM_ERR_UNSUPPORTED


def test_swiglu_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.qmm_gemv_swiglu
    args = [p(A16)] * 6 + [p(A16), p(A16)]
    assert f(*args, 64, 128, 4, 64, None) in (qmm.QMM_ERR_DEVICE, qmm.QMM_OK)
    assert f(*args, 0, 128, 4, 64, None) == qmm.QMM_OK
    assert f(*([p(A16)] * 6), p(A16), None, 64, 128, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert f(*([p(A16)] * 6), p(A16), p(A16 + 4), 64, 128, 4, 64, None) == qmm.QMM_ERR_MISALIGNED
    bad_up = [p(A16)] * 3 + [None] + [p(A16)] * 2 + [p(A16), p(A16)]
    assert f(*bad_up, 64, 128, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert f(*args, 64, 128, 7, 64, None) == qmm.QMM_ERR_UNSUPPORTED


def test_combine_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.qmm_moe_combine
    w3 = [p(A16)] * 3

    def call(tok=A16, wgt=A16, y=A16, n_tokens=4, p_rows=8, bits=4, k=128):
        return f(*w3, p(A16), None, 8, p(A16), p(tok) if tok else None, p(wgt) if wgt else None,
                 p(y), n_tokens, p_rows, 2, 64, k, bits, 64, None)
    assert call() in (qmm.QMM_ERR_DEVICE, qmm.QMM_OK)
    assert call(n_tokens=0) == qmm.QMM_OK
    assert call(p_rows=0) == qmm.QMM_OK
    assert call(tok=0) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(wgt=0) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(tok=A16 + 2) == qmm.QMM_ERR_MISALIGNED
    assert call(wgt=A16 + 1) == qmm.QMM_ERR_MISALIGNED
    assert call(y=A16 + 4) == qmm.QMM_ERR_MISALIGNED
    assert call(n_tokens=-1) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(bits=7) == qmm.QMM_ERR_UNSUPPORTED
    assert call(k=100) == qmm.QMM_ERR_INVALID_ARGUMENT


def test_residual_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.qmm_gemv_residual
    w4 = [p(A16)] * 4
    assert f(*w4, p(A16), p(A16), 64, 128, 4, 64, None) in (qmm.QMM_ERR_DEVICE, qmm.QMM_OK)
    assert f(*w4, p(A16), p(A16), 0, 128, 4, 64, None) == qmm.QMM_OK
    assert f(*w4, None, p(A16), 64, 128, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert f(*w4, p(A16 + 2), p(A16), 64, 128, 4, 64, None) == qmm.QMM_ERR_MISALIGNED
    assert f(*w4, p(A16), p(A16 + 4), 64, 128, 4, 64, None) == qmm.QMM_ERR_MISALIGNED
    assert f(*w4, p(A16), p(A16), 64, 128, 7, 64, None) == qmm.QMM_ERR_UNSUPPORTED
    assert f(*w4, p(A16), p(A16), 64, 100, 4, 64, None) == qmm.QMM_ERR_INVALID_ARGUMENT


def test_fp16_weights_need_no_scales(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    # NULL scales and mins pass the checks for bits 16 (and only for 16).
    assert _gemv(lib, s=0, m=0, bits=16) == qmm.QMM_ERR_DEVICE
    assert _gemv(lib, s=0, m=0, bits=8) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert _gemv(lib, s=A16 + 1, bits=16) == qmm.QMM_ERR_DEVICE  # not read, not checked
    assert _gemv(lib, bits=12) == qmm.QMM_ERR_INVALID_ARGUMENT
    pl = qmm.qmm_get_plan(0, 1, 4096, 4096, 16, 64, cu_count=256)
    assert pl["unit_codes"] == 32


# ---- launch planning (host integer logic) -----------------------------------------

ALL_DECODE_SHAPES = sorted({(n, k) for _, n, k in configs.QWEN3_06B_PROJ + [configs.QWEN3_06B_LM_HEAD]}
                           | {(n, k) for _, n, k in configs.LLAMA32_3B_PROJ}
                           | {(configs.SINGLE_Q4["n"], configs.SINGLE_Q4["k"])}
                           | {(n, k) for _, n, k in configs.MOE_PROJ})


@pytest.mark.parametrize("bits", (2, 3, 4, 5, 6, 8, 16))
@pytest.mark.parametrize("n,k", ALL_DECODE_SHAPES + [(5, 16384), (7, 96), (1, 64)])
@pytest.mark.parametrize("group", (64, 32, 128))
def test_gemv_plan_covers_the_row(lib, bits, n, k, group):
    if k % group:
        pytest.skip("k not a multiple of the group")
    pl = qmm.qmm_get_plan(0, 1, n, k, bits, group, cu_count=256)
    unit = pl["unit_codes"]
    assert unit == (64 if group % 64 == 0 and bits != 16 else 32)
    assert pl["block"] == 256
    cover = pl["lanes_per_row"] * pl["units_per_lane"] * unit
    assert pl["multipass"] == (cover < k)
    assert 64 % pl["lanes_per_row"] == 0
    slots = 64 // pl["lanes_per_row"]
    rows_per_block = 4 * slots * pl["rows_per_iter"]
    # Enough work-groups to cover the rows, no more than the row batches need.
    assert 1 <= pl["grid"] <= (n + rows_per_block - 1) // rows_per_block + 1
    # Weight bytes in flight per lane per iteration stay modest.
    assert pl["rows_per_iter"] * pl["units_per_lane"] * unit * bits // 8 <= 256


def test_gemv_plan_small_vs_large(lib):
    small = qmm.qmm_get_plan(0, 1, 3072, 1024, 4, 64, cu_count=256)
    large = qmm.qmm_get_plan(0, 1, 151936, 1024, 4, 64, cu_count=256)
    assert small["rows_per_iter"] == 1      # latency-bound: widest grid
    assert large["rows_per_iter"] > 1       # bandwidth-bound: more bytes per lane
    assert large["grid"] <= 256 * 32 // 4   # persistent-sized grid


def _expected_tile(m, n, k, cus=256):
    # 64-row tiles unless they would need more work-groups than CUs, or K is
    # long (64 steps of 128 or more) with more than one 128-row tile; above
    # 64 rows, 32-row tiles where the 64-row grid underfills the CUs and K
    # is short.
    if m <= 32:
        return 32
    if m <= 64:
        return 64
    tiles64 = -(-m // 64) * -(-n // 128)
    long_k = -(-k // 128) >= 64
    if tiles64 <= cus and not (long_k and m > 128):
        return 32 if tiles64 < cus and not long_k else 64
    return 128


@pytest.mark.parametrize("m", (3, 64, 128, 512, 1000))
@pytest.mark.parametrize("n,k", [(512, 2048), (2048, 2048), (8192, 2048), (2048, 8192)])
def test_gemm_plan(lib, m, n, k):
    unlimited = 1 << 40
    pl = qmm.qmm_get_plan(1, m, n, k, 4, 64, cu_count=256, workspace_bytes=unlimited)
    assert pl["variant"] == 2
    assert pl["tile_m"] == _expected_tile(m, n, k)
    # 256-column tiles exactly where a 128-row grid of them fills the CUs.
    wide = pl["tile_m"] == 128 and -(-m // 128) * -(-n // 256) >= 256
    assert pl["tile_n"] == (256 if wide else 128)
    assert pl["block"] == (256 if pl["tile_m"] == 32 else 512)
    tiles = -(-m // pl["tile_m"]) * -(-n // pl["tile_n"])
    assert pl["grid"] >= tiles * pl["split_k"]
    assert 1 <= pl["split_k"] <= 16
    # Every split keeps at least four K steps of 128.
    assert pl["split_k"] == 1 or -(-k // 128) // pl["split_k"] >= 4
    if tiles >= 256:
        assert pl["split_k"] == 1
    none = qmm.qmm_get_plan(1, m, n, k, 4, 64, cu_count=256, workspace_bytes=0)
    assert none["split_k"] == 1


def test_gemm_plan_on_the_prefill_shapes(lib):
    # The measured choices: (m, n, k) -> (tile_m, split_k).
    want = {(128, 2048, 2048): (32, 4), (128, 512, 2048): (32, 4), (128, 8192, 2048): (32, 1),
            (128, 2048, 8192): (64, 8), (512, 2048, 2048): (32, 1), (512, 512, 2048): (32, 4),
            (512, 8192, 2048): (128, 1), (512, 2048, 8192): (128, 4)}
    for (m, n, k), (tile, split) in want.items():
        pl = qmm.qmm_get_plan(1, m, n, k, 4, 64, cu_count=256, workspace_bytes=1 << 40)
        assert (pl["tile_m"], pl["split_k"]) == (tile, split), (m, n, k)


def test_gemm_tile_override(lib, qmm_override):
    qmm_override("QMM_GEMM_TILE_M", 128)
    assert qmm.qmm_get_plan(1, 100, 512, 1024, 4, 64, cu_count=256)["tile_m"] == 128
    qmm_override("QMM_GEMM_TILE_M", 32)
    pl = qmm.qmm_get_plan(1, 100, 512, 1024, 4, 64, cu_count=256)
    assert pl["tile_m"] == 32 and pl["block"] == 256


def test_unknown_override_is_rejected(lib):
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_set_override("QMM_NO_SUCH_KNOB", 1)
    assert e.value.status == qmm.QMM_ERR_INVALID_ARGUMENT


def _plans():
    return [qmm.qmm_get_plan(1, 100, 512, 1024, 4, 64, cu_count=256),
            qmm.qmm_get_plan(0, 1, 3072, 1024, 4, 64, cu_count=256),
            qmm.qmm_get_plan(2, 16, 768, 2048, 4, 64, cu_count=256),
            qmm.qmm_get_plan(3, 1, 200000, 3072, 4, 64, cu_count=256)]


def test_environment_after_load_changes_no_plan(lib, monkeypatch):
    # The library reads its overrides once, at load: setting them in the
    # environment afterwards changes nothing.
    before = _plans()
    for name, value in (("QMM_GEMM_TILE_M", "32"), ("QMM_GEMM_SPLIT", "3"), ("QMM_GEMV_LPR", "16"),
                        ("QMM_GEMV_XC", "1"), ("QMM_GEMV_U", "2"), ("QMM_ROWS_MR", "1"),
                        ("QMM_UNIT", "32"), ("QMM_BATCH_U", "2"), ("QMM_GEMV_WAVES_PER_CU", "4")):
        monkeypatch.setenv(name, value)
    assert _plans() == before


def test_environment_at_load_is_read(lib):
    # A fresh process with the override in its environment at load time.
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r); import gemm_qmm_gemv_amd as q; q.load(); "
            "print(q.qmm_get_plan(1, 100, 512, 1024, 4, 64, cu_count=256)['tile_m'])" % ROOT)
    env = dict(os.environ, QMM_GEMM_TILE_M="32")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
    assert out.stdout.strip().splitlines()[-1] == "32"


def test_small_m_routes(lib):
    assert qmm.qmm_get_plan(1, 1, 256, 1024, 4, 64, cu_count=256)["variant"] == 0
    assert qmm.qmm_get_plan(1, 2, 256, 1024, 4, 64, cu_count=256)["variant"] == 1
    assert qmm.qmm_get_plan(1, 3, 256, 1024, 4, 64, cu_count=256)["variant"] == 2
    assert qmm.qmm_get_plan(2, 16, 768, 2048, 4, 64, cu_count=256)["variant"] == 1


def test_sizes_beyond_32bit_offsets_are_rejected(lib):
    # One packed matrix or one activation block of 4 GiB or more cannot be
    # addressed with the kernels' 32-bit buffer offsets.
    assert _gemv(lib, n=1 << 20, k=1 << 15) == qmm.QMM_ERR_UNSUPPORTED
    assert "4 GiB" in qmm.qmm_last_error()
    p = ctypes.c_void_p
    assert lib.qmm_gemm(p(A16), p(A16), p(A16), p(A16), p(A16), 1 << 20, 64, 1 << 12, 4, 64,
                        None, 0, None) == qmm.QMM_ERR_UNSUPPORTED
    assert "activation" in qmm.qmm_last_error()
    # Just below the limit the checks pass on to the device (none here).
    import torch
    if not torch.cuda.is_available():
        assert _gemv(lib, n=(1 << 20) - 64, k=1 << 13) == qmm.QMM_ERR_DEVICE


def test_ceiling_library_exports():
    # The measurement kernels bench.py times beside the spec peaks (not part
    # of the qmm.h interface): the library loads and argument checks run on
    # the host.
    import os
    from gemm_qmm_gemv_amd import build as qbuild
    if not os.path.exists(qbuild.CEILING_LIB):
        pytest.skip("libqmm_ceiling.so not built")
    cl = ctypes.CDLL(qbuild.CEILING_LIB)
    p, u64, ci = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
    cl.qmm_ceiling_read.argtypes = [p, u64, ci, p, p]
    cl.qmm_ceiling_mfma.argtypes = [ci, ci, p, p]
    assert cl.qmm_ceiling_read(None, 16, 1, p(A16), None) == 1
    assert cl.qmm_ceiling_read(p(A16), 15, 1, p(A16), None) == 1
    assert cl.qmm_ceiling_mfma(0, 10, p(A16), None) == 1


def test_grouped_argument_checks(lib):
    p = ctypes.c_void_p
    import gemm_qmm_gemv_amd as q
    f = lib.qmm_gemm_grouped

    def call(members, count=None, x=A16, m=64, k=128, bits=4, ws=None, wsb=0):
        arr = (q.GemmMember * max(len(members), 1))()
        for d, (w, y, n) in zip(arr, members):
            d.w_packed, d.scales, d.mins, d.y, d.n = w, A16, A16, y, n
        return f(ctypes.addressof(arr), len(members) if count is None else count, p(x) if x else None,
                 m, k, bits, 64, p(ws) if ws else None, wsb, None)
    good = [(A16, A16, 128), (A16, A16, 64)]
    assert call(good) in (qmm.QMM_ERR_DEVICE, qmm.QMM_OK)
    assert call(good, count=0) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(good * 3, count=5) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(good, m=0) == qmm.QMM_OK
    assert call([(A16, A16, 0)]) == qmm.QMM_OK  # nothing to compute
    assert call([(A16, A16 + 4, 128)]) == qmm.QMM_ERR_MISALIGNED
    assert call([(A16, 0, 128)]) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(good, x=A16 + 2) == qmm.QMM_ERR_MISALIGNED
    assert call(good, bits=7) == qmm.QMM_ERR_UNSUPPORTED
    assert call(good, k=100) == qmm.QMM_ERR_INVALID_ARGUMENT
    assert call(good, ws=A16 + 8, wsb=1024) == qmm.QMM_ERR_MISALIGNED
    assert f(None, 2, p(A16), 64, 128, 4, 64, None, 0, None) == qmm.QMM_ERR_INVALID_ARGUMENT


def test_grouped_workspace_follows_the_launch_decision(lib):
    # Without a device the planner assumes 256 compute units.  q|k|v of a
    # Llama-3.2-1B layer at 128 tokens underfill the GPU alone: one grouped
    # launch of 4 x 24 tiles (32 rows), K split in two (three fitted, two
    # after rounding each split to whole blocks of four steps; counters,
    # then the partial sums of all three members).  gate|up at 2048 tokens
    # fill it alone: separate launches without a split need no workspace.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")

    def members(ns):
        return [(A16, A16, A16, A16, n) for n in ns]
    need = qmm.qmm_gemm_grouped_workspace_bytes(members([2048, 512, 512]), 128, 2048, 4, 64)
    assert need == 4096 + 2 * 128 * 3072 * 4
    assert qmm.qmm_gemm_grouped_workspace_bytes(members([8192, 8192]), 2048, 2048, 4, 64) == 0
    # A member with n = 0 is skipped; an empty group needs nothing.
    assert qmm.qmm_gemm_grouped_workspace_bytes(members([2048, 0, 512, 512]), 128, 2048, 4, 64) == need
    assert qmm.qmm_gemm_grouped_workspace_bytes(members([0]), 128, 2048, 4, 64) == 0
