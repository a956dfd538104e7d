"""Python binding of libqmm (quantized GEMV / GEMM with inline dequantization
for AMD MI355X, gfx950).

The functions here carry the C ABI's names (``include/qmm.h``) and only
marshal arguments: every step of the computation runs in the HIP kernels of
``libqmm.so``.  PyTorch supplies device memory and streams.  There is no
fallback: if the library is missing or fails to load, every call raises.

Arguments that are device buffers may be given as torch tensors (their
``data_ptr()`` is passed) or as raw integer addresses.  ``stream`` defaults to
torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "QmmError", "library_path", "load",
    "qmm_gemv", "qmm_gemm", "qmm_gemm_workspace_bytes", "qmm_moe_gemm", "qmm_unpack",
    "qmm_gemv_batch_prepare", "qmm_gemv_batched", "GemvDesc", "GemmMember", "qmm_gemv_swiglu",
    "qmm_gemm_f16out",
    "qmm_moe_swiglu", "qmm_gemv_residual", "qmm_moe_combine", "qmm_gemm_grouped",
    "qmm_gemm_grouped_workspace_bytes", "qmm_gemm_noalloc", "qmm_set_override", "overrides",
    "QMM_NOALLOC_SCRATCH_BYTES",
    "qmm_get_plan", "qmm_status_string", "qmm_last_error", "qmm_abi_version",
    "QMM_OK", "QMM_ERR_INVALID_ARGUMENT", "QMM_ERR_UNSUPPORTED", "QMM_ERR_MISALIGNED",
    "QMM_ERR_DEVICE", "EXPORTED_SYMBOLS",
]

QMM_OK = 0
QMM_ERR_INVALID_ARGUMENT = 1
QMM_ERR_UNSUPPORTED = 2
QMM_ERR_MISALIGNED = 3
QMM_ERR_DEVICE = 4
QMM_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # include/qmm.h

EXPORTED_SYMBOLS = (
    "qmm_gemv", "qmm_gemm", "qmm_gemm_workspace_bytes", "qmm_moe_gemm", "qmm_unpack",
    "qmm_gemv_batch_prepare", "qmm_gemv_batched", "qmm_gemv_swiglu", "qmm_gemm_f16out",
    "qmm_moe_swiglu", "qmm_gemv_residual", "qmm_moe_combine", "qmm_gemm_grouped",
    "qmm_gemm_grouped_workspace_bytes", "qmm_gemm_noalloc", "qmm_set_override",
    "qmm_get_plan", "qmm_status_string", "qmm_last_error", "qmm_abi_version",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libqmm.so"
_lib = None


class QmmError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__("%s failed with status %d: %s" % (func, status, detail))


class _Plan(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("lanes_per_row", ctypes.c_int32),
        ("units_per_lane", ctypes.c_int32),
        ("rows_per_iter", ctypes.c_int32),
        ("unit_codes", ctypes.c_int32),
        ("split_k", ctypes.c_int32),
        ("tile_m", ctypes.c_int32),
        ("tile_n", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 5),
    ]


class GemvDesc(ctypes.Structure):
    """qmm_gemv_desc: one GEMV of a batched launch (64 bytes)."""
    _fields_ = [
        ("w_packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("mins", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("first_item", ctypes.c_int64),
    ]


assert ctypes.sizeof(GemvDesc) == 64


class GemmMember(ctypes.Structure):
    """qmm_gemm_member: one weight matrix of a grouped GEMM and its output."""
    _fields_ = [
        ("w_packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("mins", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("n", ctypes.c_int64),
    ]


assert ctypes.sizeof(GemmMember) == 40


def library_path() -> str:
    """In-tree libqmm.so, or the file named by $QMM_LIBRARY (tuning builds)."""
    return os.environ.get("QMM_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def load():
    """Load libqmm.so (built in-tree by ``python -m gemm_qmm_gemv_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            "libqmm.so is not built (%s); run `python -m gemm_qmm_gemv_amd.build`" % path)
    try:
        # torch first: its HIP runtime is then the one the library binds to.
        import torch  # noqa: F401
    except Exception:
        pass
    lib = ctypes.CDLL(path)
    p, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.qmm_gemv.argtypes = [p, p, p, p, p, i64, i64, ci, ci, p]
    lib.qmm_gemm.argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, p, sz, p]
    lib.qmm_gemv_swiglu.argtypes = [p, p, p, p, p, p, p, p, i64, i64, ci, ci, p]
    lib.qmm_gemv_residual.argtypes = [p, p, p, p, p, p, i64, i64, ci, ci, p]
    lib.qmm_gemm_f16out.argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, p, sz, p]
    lib.qmm_gemm_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, ci, ci, p]
    lib.qmm_set_override.argtypes = [ctypes.c_char_p, ci]
    lib.qmm_gemm_workspace_bytes.argtypes = [i64, i64, i64, ci, ci]
    lib.qmm_gemm_workspace_bytes.restype = sz
    lib.qmm_moe_gemm.argtypes = [p, p, p, p, p, i64, p, p, i64, i64, i64, i64, ci, ci, p]
    lib.qmm_moe_swiglu.argtypes = [p, p, p, p, p, p, p, p, i64, p, p, i64, i64, i64, i64, ci, ci, p]
    lib.qmm_moe_combine.argtypes = [p, p, p, p, p, i64, p, p, p, p, i64, i64, i64, i64, i64, ci, ci, p]
    lib.qmm_gemm_grouped.argtypes = [p, ci, p, i64, i64, ci, ci, p, ctypes.c_size_t, p]
    lib.qmm_gemm_grouped_workspace_bytes.argtypes = [p, ci, i64, i64, ci, ci]
    lib.qmm_gemm_grouped_workspace_bytes.restype = ctypes.c_size_t
    lib.qmm_unpack.argtypes = [p, p, i64, i64, ci, p]
    lib.qmm_gemv_batch_prepare.argtypes = [p, i64, ci, ci]
    lib.qmm_gemv_batched.argtypes = [p, p, i64, ci, ci, p]
    lib.qmm_get_plan.argtypes = [ci, i64, i64, i64, ci, ci, ci, sz, ctypes.POINTER(_Plan)]
    for f in ("qmm_gemv", "qmm_gemm", "qmm_moe_gemm", "qmm_unpack", "qmm_get_plan",
              "qmm_gemv_batch_prepare", "qmm_gemv_batched", "qmm_gemv_swiglu", "qmm_gemm_f16out", "qmm_moe_swiglu",
              "qmm_gemv_residual", "qmm_moe_combine", "qmm_gemm_grouped", "qmm_gemm_noalloc",
              "qmm_set_override"):
        getattr(lib, f).restype = ci
    lib.qmm_status_string.argtypes = [ci]
    lib.qmm_status_string.restype = ctypes.c_char_p
    lib.qmm_last_error.restype = ctypes.c_char_p
    lib.qmm_abi_version.restype = ci
    _lib = lib
    return lib


def _addr(v):
    if v is None:
        return None
    if isinstance(v, int):
        return v
    return v.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str) -> None:
    if status != QMM_OK:
        detail = load().qmm_last_error().decode()
        raise QmmError(status, func, detail)


def qmm_status_string(status: int) -> str:
    return load().qmm_status_string(int(status)).decode()


def qmm_last_error() -> str:
    return load().qmm_last_error().decode()


def qmm_abi_version() -> int:
    return load().qmm_abi_version()


def qmm_gemv(w_packed, scales, mins, x, y, n, k, bits, group_size, stream=None) -> None:
    """y[n] = sum_k (s*q + m)[n][k] x[k] (fp16 x, fp32 y); asynchronous."""
    _check(load().qmm_gemv(_addr(w_packed), _addr(scales), _addr(mins), _addr(x), _addr(y),
                           int(n), int(k), int(bits), int(group_size), _stream(stream)),
           "qmm_gemv")


def qmm_gemv_residual(w_packed, scales, mins, x, residual, y, n, k, bits, group_size,
                      stream=None) -> None:
    """y[n] = residual[n] + sum_k (s*q + m)[n][k] x[k] (residual may be y); asynchronous."""
    _check(load().qmm_gemv_residual(_addr(w_packed), _addr(scales), _addr(mins), _addr(x),
                                    _addr(residual), _addr(y), int(n), int(k), int(bits),
                                    int(group_size), _stream(stream)),
           "qmm_gemv_residual")


def qmm_gemv_swiglu(gate_w, gate_scales, gate_mins, up_w, up_scales, up_mins, x, h, n, k, bits,
                    group_size, stream=None) -> None:
    """h[n] = silu(g[n]) * u[n] with g = Wg x, u = Wu x (fp16 x, fp32 h); asynchronous."""
    _check(load().qmm_gemv_swiglu(_addr(gate_w), _addr(gate_scales), _addr(gate_mins), _addr(up_w),
                                  _addr(up_scales), _addr(up_mins), _addr(x), _addr(h), int(n),
                                  int(k), int(bits), int(group_size), _stream(stream)),
           "qmm_gemv_swiglu")


def qmm_gemm_f16out(w_packed, scales, mins, x, y, m, n, k, bits, group_size, workspace=None,
                    workspace_bytes=0, stream=None) -> None:
    """As qmm_gemm with y fp16 [m][n] (each sum rounded once); asynchronous."""
    _check(load().qmm_gemm_f16out(_addr(w_packed), _addr(scales), _addr(mins), _addr(x), _addr(y),
                                  int(m), int(n), int(k), int(bits), int(group_size), _addr(workspace),
                                  int(workspace_bytes), _stream(stream)),
           "qmm_gemm_f16out")


def qmm_gemm(w_packed, scales, mins, x, y, m, n, k, bits, group_size, workspace=None,
             workspace_bytes=0, stream=None) -> None:
    """y[m][n] = sum_k (s*q + m)[n][k] x[m][k]; asynchronous."""
    _check(load().qmm_gemm(_addr(w_packed), _addr(scales), _addr(mins), _addr(x), _addr(y),
                           int(m), int(n), int(k), int(bits), int(group_size), _addr(workspace),
                           int(workspace_bytes), _stream(stream)),
           "qmm_gemm")


def qmm_gemm_noalloc(w_packed, scales, mins, x, y, m, n, k, bits, group_size, stream=None) -> None:
    """As qmm_gemm with no workspace: the library's own fixed scratch array
    holds any K-split partial sums; asynchronous."""
    _check(load().qmm_gemm_noalloc(_addr(w_packed), _addr(scales), _addr(mins), _addr(x), _addr(y),
                                   int(m), int(n), int(k), int(bits), int(group_size), _stream(stream)),
           "qmm_gemm_noalloc")


def qmm_set_override(name: str, value: int) -> None:
    """Process-wide launch-plan override (value < 0 removes it)."""
    _check(load().qmm_set_override(name.encode(), int(value)), "qmm_set_override")


class overrides:
    """Context manager: ``with overrides(QMM_GEMM_TILE_M=64): ...`` sets the
    named launch-plan overrides and removes them on exit."""

    def __init__(self, **values):
        self.values = values

    def __enter__(self):
        for name, value in self.values.items():
            qmm_set_override(name, value)
        return self

    def __exit__(self, *exc):
        for name in self.values:
            qmm_set_override(name, -1)
        return False


def _members(members):
    arr = (GemmMember * len(members))()
    for d, (w, s, mn, y, n) in zip(arr, members):
        d.w_packed, d.scales, d.mins, d.y, d.n = _addr(w), _addr(s), _addr(mn), _addr(y), int(n)
    return arr


def qmm_gemm_grouped(members, x, m, k, bits, group_size, workspace=None, workspace_bytes=0,
                     stream=None) -> None:
    """members: [(w_packed, scales, mins, y, n)]; y_i = X W_i^T for all in one launch."""
    arr = _members(members)
    _check(load().qmm_gemm_grouped(ctypes.addressof(arr), len(members), _addr(x), int(m), int(k),
                                   int(bits), int(group_size), _addr(workspace), int(workspace_bytes),
                                   _stream(stream)),
           "qmm_gemm_grouped")


def qmm_gemm_grouped_workspace_bytes(members, m, k, bits, group_size) -> int:
    arr = _members(members)
    return int(load().qmm_gemm_grouped_workspace_bytes(ctypes.addressof(arr), len(members), int(m), int(k),
                                                       int(bits), int(group_size)))


def qmm_gemm_workspace_bytes(m, n, k, bits, group_size) -> int:
    return int(load().qmm_gemm_workspace_bytes(int(m), int(n), int(k), int(bits), int(group_size)))


def qmm_moe_gemm(w_packed, scales, mins, x, x_rows, x_rows_count, expert_offsets, y, p_rows,
                 n_experts, n, k, bits, group_size, stream=None) -> None:
    """Expert-grouped rows: y[p] = W_{e(p)} x[x_rows[p]]; asynchronous."""
    _check(load().qmm_moe_gemm(_addr(w_packed), _addr(scales), _addr(mins), _addr(x),
                               _addr(x_rows), int(x_rows_count), _addr(expert_offsets), _addr(y),
                               int(p_rows), int(n_experts), int(n), int(k), int(bits),
                               int(group_size), _stream(stream)),
           "qmm_moe_gemm")


def qmm_moe_combine(w_packed, scales, mins, x, x_rows, x_rows_count, expert_offsets, pair_token,
                    pair_weight, y, n_tokens, p_rows, n_experts, n, k, bits, group_size,
                    stream=None) -> None:
    """y[token[p]] += weight[p] * W_{e(p)} x[row(p)] (accumulates into y); asynchronous."""
    _check(load().qmm_moe_combine(_addr(w_packed), _addr(scales), _addr(mins), _addr(x),
                                  _addr(x_rows), int(x_rows_count), _addr(expert_offsets),
                                  _addr(pair_token), _addr(pair_weight), _addr(y), int(n_tokens),
                                  int(p_rows), int(n_experts), int(n), int(k), int(bits),
                                  int(group_size), _stream(stream)),
           "qmm_moe_combine")


def qmm_moe_swiglu(gate_w, gate_scales, gate_mins, up_w, up_scales, up_mins, x, x_rows,
                   x_rows_count, expert_offsets, h, p_rows, n_experts, n, k, bits, group_size,
                   stream=None) -> None:
    """h[p] = silu(Wg_{e(p)} x[row(p)]) * (Wu_{e(p)} x[row(p)]); asynchronous."""
    _check(load().qmm_moe_swiglu(_addr(gate_w), _addr(gate_scales), _addr(gate_mins), _addr(up_w),
                                 _addr(up_scales), _addr(up_mins), _addr(x), _addr(x_rows),
                                 int(x_rows_count), _addr(expert_offsets), _addr(h), int(p_rows),
                                 int(n_experts), int(n), int(k), int(bits), int(group_size),
                                 _stream(stream)),
           "qmm_moe_swiglu")


def qmm_unpack(w_packed, codes, n, k, bits, stream=None) -> None:
    """codes[n][k] (uint8) = the packed codes; asynchronous."""
    _check(load().qmm_unpack(_addr(w_packed), _addr(codes), int(n), int(k), int(bits),
                             _stream(stream)),
           "qmm_unpack")


def qmm_gemv_batch_prepare(descs, bits, group_size) -> None:
    """Fill the library-owned fields of a ``GemvDesc`` array (host memory)."""
    _check(load().qmm_gemv_batch_prepare(ctypes.addressof(descs), len(descs), int(bits),
                                         int(group_size)),
           "qmm_gemv_batch_prepare")


def qmm_gemv_batched(descs_device, descs_host, bits, group_size, stream=None) -> None:
    """One launch over every GEMV of a prepared descriptor array.
    ``descs_device``: device copy (tensor or address); ``descs_host``: the
    ``GemvDesc`` array it was copied from."""
    _check(load().qmm_gemv_batched(_addr(descs_device), ctypes.addressof(descs_host),
                                   len(descs_host), int(bits), int(group_size), _stream(stream)),
           "qmm_gemv_batched")


def qmm_get_plan(op, m, n, k, bits, group_size, cu_count=0, workspace_bytes=0) -> dict:
    """The launch plan the library would use (op 0 gemv, 1 gemm, 2 moe,
    3 batched gemv with n = total rows and k = largest k)."""
    plan = _Plan()
    _check(load().qmm_get_plan(int(op), int(m), int(n), int(k), int(bits), int(group_size),
                               int(cu_count), int(workspace_bytes), ctypes.byref(plan)),
           "qmm_get_plan")
    return {f: getattr(plan, f) for f, _ in _Plan._fields_ if f != "reserved"} | {
        "multipass": bool(plan.reserved[0]), "staged": bool(plan.reserved[1]),
        "late": bool(plan.reserved[2])}
