"""CPU oracle for the quantized matmul -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never does: it shares no code, header,
table or helper with the HIP kernels.  The arithmetic lives in
``qmm_oracle.c`` (plain C, double precision, k-ordered loops); this module
builds it with gcc and marshals numpy arrays into it.

What it computes is the plain definition of the method: unpack each b-bit
code from the row bitstream, form w = scale * q + min per group along K, and
take the dot product with the fp16 activations in double precision.  Pages:
"Apple Silicon 로컬 LLM 추론의 새 기준 BaseRT" (thakicloud.com), section
"BaseRT는 무엇인가" (affine quantization, Q2 to Q8), and "BaseRT claims
fastest Apple Silicon inference" (thetesserapress.com), section "What BaseRT
does differently" (GEMV for M = 1, GEMM for M > 1, dequantization inside the
compute loop).

Pinning (what each function is checked against, in ``tests/test_oracle_pins.py``):
  * fp16 decoder      -- numpy's float16 -> float64 on all 65,536 patterns.
  * unpack / pack     -- hand-worked bit-order vectors, numpy ``unpackbits``
                         (a library bit reader), round trips both ways.
  * qmm (GEMV / GEMM) -- numpy float64 matmul of weights dequantized by
                         library routines; closed form for constant codes;
                         one-hot activations; exact integer cases;
                         exact power-of-two scaling and sign symmetry.
  * qmm_sample        -- the same rows of full qmm.
  * moe               -- per-expert numpy matmuls over the expert's rows.
  * silu               -- printed values of the logistic function at +-1,
                         the odd-part identity silu(v) - silu(-v) = v, limits.
  * fp16 weights (bits 16: the unquantized "Q16/FP16" format, no scales or
    mins) -- decoded by the pinned fp16 decoder and multiplied in float64
    with numpy; pinned against the Q8 path (integer codes with scale 1 and
    min 0 are exact fp16 weights), one-hot activations and exact integers.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqmm_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def compile_source(src: str, out: str) -> str:
    """Compile an oracle source file to a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.qmo_fp16_to_double.argtypes = [ctypes.c_uint16]
    lib.qmo_fp16_to_double.restype = ctypes.c_double
    lib.qmo_fp16_array_to_double.argtypes = [p, i64, p]
    lib.qmo_unpack.argtypes = [p, i64, i64, ci, p]
    lib.qmo_pack.argtypes = [p, i64, i64, ci, p]
    lib.qmo_dequant.argtypes = [p, p, p, i64, i64, ci, ci, p]
    lib.qmo_qmm.argtypes = [p, p, p, p, i64, i64, i64, ci, ci, p, p]
    lib.qmo_qmm_sample.argtypes = [p, p, p, p, i64, ci, ci, p, p, i64, p, p]
    lib.qmo_moe.argtypes = [p, p, p, p, p, p, i64, i64, i64, ci, ci, p, p]
    lib.qmo_threads.restype = ci
    lib.qmo_set_threads.argtypes = [ci]
    for f in ("qmo_fp16_array_to_double", "qmo_unpack", "qmo_pack", "qmo_dequant",
              "qmo_qmm", "qmo_qmm_sample", "qmo_moe", "qmo_set_threads"):
        getattr(lib, f).restype = None
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def use_library(path: str | None) -> None:
    """Route every function of this module to another build of the oracle
    (``None`` restores the default build).  Tests use it to check that the
    pins catch mistakes planted in a copy of the source."""
    global _lib
    _lib = None if path is None else _bind(ctypes.CDLL(path))


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _as_u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a.astype(np.uint16, copy=False)


def _check_format(k: int, bits: int, group: int):
    if bits not in (2, 3, 4, 5, 6, 7, 8, 16):
        raise ValueError("bits must be in 2..8 or 16 (fp16 weights)")
    if (k * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32")
    if group <= 0 or k % group:
        raise ValueError("K must be a multiple of the group size")


def threads() -> int:
    return _load().qmo_threads()


def set_threads(t: int) -> None:
    _load().qmo_set_threads(int(t))


def fp16_to_double(h) -> np.ndarray:
    """Decode fp16 bit patterns (uint16 or float16 array) to float64."""
    h = _as_u16(h)
    out = np.empty(h.shape, dtype=np.float64)
    _load().qmo_fp16_array_to_double(_ptr(h), h.size, _ptr(out))
    return out


def unpack(w_packed, n: int, k: int, bits: int) -> np.ndarray:
    """Codes [N][K] uint8 from the packed [N][K*bits/32] uint32 rows."""
    _check_format(k, bits, k)
    w = _c(w_packed, np.uint32)
    assert w.size == n * k * bits // 32
    out = np.empty((n, k), dtype=np.uint8)
    _load().qmo_unpack(_ptr(w), n, k, bits, _ptr(out))
    return out


def pack(codes, bits: int) -> np.ndarray:
    """Packed [N][K*bits/32] uint32 rows from codes [N][K] (values < 2^bits)."""
    codes = _c(codes, np.uint8)
    n, k = codes.shape
    _check_format(k, bits, k)
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range for %d bits" % bits)
    out = np.empty((n, k * bits // 32), dtype=np.uint32)
    _load().qmo_pack(_ptr(codes), n, k, bits, _ptr(out))
    return out


def dequant(w_packed, scales, mins, n: int, k: int, bits: int, group: int) -> np.ndarray:
    """Dequantized weights [N][K] float64: scale * q + min."""
    _check_format(k, bits, group)
    w = _c(w_packed, np.uint32)
    s, m = _as_u16(scales), _as_u16(mins)
    assert s.size == n * (k // group) and m.size == s.size
    out = np.empty((n, k), dtype=np.float64)
    _load().qmo_dequant(_ptr(w), _ptr(s), _ptr(m), n, k, bits, group, _ptr(out))
    return out


def f16_weights(w_words, n: int, k: int) -> np.ndarray:
    """fp16 weights [n][k] as float64 from their words: word j of a row holds
    k = 2j in its low 16 bits and k = 2j + 1 in its high 16 bits."""
    w = _c(w_words, np.uint32).reshape(n, k // 2)
    h = np.empty((n, k), dtype=np.uint16)
    h[:, 0::2] = (w & 0xFFFF).astype(np.uint16)
    h[:, 1::2] = (w >> 16).astype(np.uint16)
    return fp16_to_double(h)


def _qmm_f16(w_words, x2, n: int, k: int):
    wd = f16_weights(w_words, n, k)
    xd = fp16_to_double(x2)
    return xd @ wd.T, np.abs(xd) @ np.abs(wd).T


def qmm(w_packed, scales, mins, x, n: int, k: int, bits: int, group: int):
    """(y, a) with y[M][N] = X W^T and a[M][N] = sum_k |w x|, both float64.

    x is fp16 [M][K] (or [K] for the GEMV; y and a are then [N]).  bits 16:
    w_packed holds fp16 weights (see f16_weights); scales and mins unused."""
    _check_format(k, bits, group)
    x = _as_u16(x)
    vec = x.ndim == 1
    x2 = x.reshape(-1, k)
    m = x2.shape[0]
    if bits == 16:
        y, a = _qmm_f16(w_packed, x2, n, k)
        return (y[0], a[0]) if vec else (y, a)
    w = _c(w_packed, np.uint32)
    s, mn = _as_u16(scales), _as_u16(mins)
    assert w.size == n * k * bits // 32
    assert s.size == n * (k // group) and mn.size == s.size
    y = np.empty((m, n), dtype=np.float64)
    a = np.empty((m, n), dtype=np.float64)
    _load().qmo_qmm(_ptr(w), _ptr(s), _ptr(mn), _ptr(x2), m, n, k, bits, group,
                    _ptr(y), _ptr(a))
    if vec:
        return y[0], a[0]
    return y, a


def qmm_sample(w_packed, scales, mins, x, k: int, bits: int, group: int,
               rows_m, rows_n):
    """(y, a) at the listed (m, n) positions only, float64 [count]."""
    _check_format(k, bits, group)
    x = _as_u16(x).reshape(-1, k)
    w = _c(w_packed, np.uint32)
    rm = _c(rows_m, np.int64)
    rn = _c(rows_n, np.int64)
    assert rm.shape == rn.shape
    if bits == 16:
        n = w.size // (k // 2)
        if rm.size and (rm.min() < 0 or rm.max() >= x.shape[0] or rn.min() < 0 or rn.max() >= n):
            raise IndexError("sample position out of range")
        wd = f16_weights(w.reshape(n, k // 2)[rn], rn.size, k)
        xd = fp16_to_double(x[rm])
        return np.sum(wd * xd, axis=1), np.sum(np.abs(wd) * np.abs(xd), axis=1)
    s, mn = _as_u16(scales), _as_u16(mins)
    n = s.size // (k // group)
    if rm.size and (rm.min() < 0 or rm.max() >= x.shape[0]
                    or rn.min() < 0 or rn.max() >= n):
        raise IndexError("sample position out of range")
    y = np.empty(rm.size, dtype=np.float64)
    a = np.empty(rm.size, dtype=np.float64)
    _load().qmo_qmm_sample(_ptr(w), _ptr(s), _ptr(mn), _ptr(x), k, bits, group,
                           _ptr(rm), _ptr(rn), rm.size, _ptr(y), _ptr(a))
    return y, a


def moe(w_packed, scales, mins, x, x_rows, offsets, n_experts: int, n: int, k: int,
        bits: int, group: int):
    """(y, a) [P][N] float64 for expert-sorted rows (see qmo_moe in the C file).

    w_packed [E][N][K*bits/32], scales/mins [E][N][K/group], x fp16 [rows][K],
    x_rows int32 [P] or None, offsets int32 [E+1]."""
    _check_format(k, bits, group)
    w = _c(w_packed, np.uint32)
    x = _as_u16(x).reshape(-1, k)
    off = _c(offsets, np.int32)
    if bits == 16:
        return _moe_f16(w, x, x_rows, off, n_experts, n, k)
    s, mn = _as_u16(scales), _as_u16(mins)
    assert off.size == n_experts + 1
    p = int(off[-1])
    if x_rows is not None:
        xr = _c(x_rows, np.int32)
        assert xr.size == p
        if p and (xr.min() < 0 or xr.max() >= x.shape[0]):
            raise IndexError("x_rows out of range")
        xr_ptr = _ptr(xr)
    else:
        assert x.shape[0] >= p
        xr = None
        xr_ptr = None
    assert w.size == n_experts * n * k * bits // 32
    y = np.zeros((p, n), dtype=np.float64)
    a = np.zeros((p, n), dtype=np.float64)
    _load().qmo_moe(_ptr(w), _ptr(s), _ptr(mn), _ptr(x), xr_ptr, _ptr(off),
                    n_experts, n, k, bits, group, _ptr(y), _ptr(a))
    return y, a


def _moe_f16(w, x, x_rows, off, n_experts: int, n: int, k: int):
    """Row p of expert e (off[e] <= p < off[e+1]) times activation row
    x_rows[p] (or p), with expert e's fp16 weights."""
    assert off.size == n_experts + 1 and w.size == n_experts * n * k // 2
    p = int(off[-1])
    xr = np.arange(p) if x_rows is None else _c(x_rows, np.int32)
    assert xr.size == p
    if p and (xr.min() < 0 or xr.max() >= x.shape[0]):
        raise IndexError("x_rows out of range")
    we = w.reshape(n_experts, n, k // 2)
    y = np.zeros((p, n), dtype=np.float64)
    a = np.zeros((p, n), dtype=np.float64)
    for e in range(n_experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        yy, aa = _qmm_f16(we[e], x[xr[lo:hi]], n, k)
        y[lo:hi], a[lo:hi] = yy, aa
    return y, a


def moe_combine(y_pair, a_pair, pair_token, pair_weight, n_tokens: int, y0=None):
    """(y, a) [T][N] float64: the routing-weighted sum of each token's expert
    outputs (the combine step of a mixture-of-experts layer, BaseRT pages,
    MoE sections): y[t] = y0[t] + sum of pair_weight[p] * y_pair[p] over the
    pairs p routed from token t; a[t] = sum of |pair_weight[p]| * a_pair[p]
    (the error scale of the weighted sum).  y0 defaults to zeros.  Weights are
    taken as given (float32 inputs widened exactly to float64)."""
    y_pair = np.asarray(y_pair, dtype=np.float64)
    a_pair = np.asarray(a_pair, dtype=np.float64)
    tok = np.asarray(pair_token, dtype=np.int64)
    wgt = np.asarray(pair_weight, dtype=np.float64)
    n = y_pair.shape[1]
    y = np.zeros((n_tokens, n)) if y0 is None else np.array(y0, dtype=np.float64).reshape(n_tokens, n)
    a = np.zeros((n_tokens, n))
    for p in range(tok.size):
        t = int(tok[p])
        if 0 <= t < n_tokens:
            y[t] += wgt[p] * y_pair[p]
            a[t] += abs(wgt[p]) * a_pair[p]
    return y, a


def silu(v) -> np.ndarray:
    """silu(v) = v / (1 + e^-v) = v * sigmoid(v), float64 (the gate of a
    SwiGLU feed-forward block: h = silu(Wg x) * (Wu x))."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):  # e^-v -> inf gives the limit -0
        return v / (1.0 + np.exp(-v))


def within_tolerance(y, y_ref, a_ref, rel: float = 2e-3, abs_: float = 1e-5):
    """Elementwise |y - y_ref| <= rel * a_ref + abs_ (the acceptance bound)."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= rel * a_ref + abs_
