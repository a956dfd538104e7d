"""Torch-side plumbing around the C ABI: move numpy inputs to device memory
and allocate outputs.  No arithmetic of the method happens here; every
product is computed by the library's kernels.
"""
from __future__ import annotations

import ctypes
import functools

import numpy as np
import torch

from . import (QMM_OK, GemvDesc, _check, _stream, load, qmm_gemm, qmm_gemm_f16out, qmm_gemm_workspace_bytes, qmm_gemv, qmm_gemv_batch_prepare,
               qmm_gemv_swiglu, qmm_moe_swiglu, qmm_gemv_residual, qmm_moe_combine, qmm_gemm_grouped,
               qmm_gemm_grouped_workspace_bytes,
               qmm_gemv_batched, qmm_moe_gemm, qmm_unpack)


def device_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a numpy array to the device, keeping its bits (uint32 -> int32,
    float16 stays float16, uint16 -> int16 views)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload_matrix(q: dict, device="cuda") -> dict:
    """dict(w, scales, mins, n, k, bits, group) with device tensors."""
    out = dict(q)
    for key in ("w", "scales", "mins"):
        out[key] = None if q[key] is None else device_tensor(q[key], device)
    return out


def gemv(dq: dict, x: torch.Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if y is None:
        y = torch.empty(dq["n"], dtype=torch.float32, device=x.device)
    qmm_gemv(dq["w"], dq["scales"], dq["mins"], x, y, dq["n"], dq["k"], dq["bits"], dq["group"],
             stream=stream)
    return y


def gemv_residual(dq: dict, x: torch.Tensor, residual: torch.Tensor, y: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """y = residual + W x in one launch (residual may be y)."""
    if y is None:
        y = torch.empty(dq["n"], dtype=torch.float32, device=x.device)
    qmm_gemv_residual(dq["w"], dq["scales"], dq["mins"], x, residual, y, dq["n"], dq["k"], dq["bits"],
                      dq["group"], stream=stream)
    return y


def gemv_swiglu(dg: dict, du: dict, x: torch.Tensor, h: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """h = silu(Wg x) * (Wu x) in one launch (both matrices in one format)."""
    assert dg["n"] == du["n"] and dg["k"] == du["k"]
    assert dg["bits"] == du["bits"] and dg["group"] == du["group"]
    if h is None:
        h = torch.empty(dg["n"], dtype=torch.float32, device=x.device)
    qmm_gemv_swiglu(dg["w"], dg["scales"], dg["mins"], du["w"], du["scales"], du["mins"], x, h,
                    dg["n"], dg["k"], dg["bits"], dg["group"], stream=stream)
    return h


def gemm(dq: dict, x: torch.Tensor, y: torch.Tensor | None = None, workspace=None,
         stream=None, out_fp16: bool = False) -> torch.Tensor:
    """Y = X W^T: fp32 output, or fp16 (qmm_gemm_f16out) with out_fp16."""
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, dq["n"]), dtype=torch.float16 if out_fp16 else torch.float32,
                        device=x.device)
    if workspace is None:
        need = qmm_gemm_workspace_bytes(m, dq["n"], dq["k"], dq["bits"], dq["group"])
        # Zeroed: the split-K arrival counters at its start must read zero
        # before the first call (every call leaves them zero).
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=x.device) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = qmm_gemm_f16out if out_fp16 else qmm_gemm
    fn(dq["w"], dq["scales"], dq["mins"], x, y, m, dq["n"], dq["k"], dq["bits"],
       dq["group"], workspace=workspace, workspace_bytes=ws_bytes, stream=stream)
    return y


def gemm_grouped(dqs: list, x: torch.Tensor, ys: list | None = None, workspace=None,
                 stream=None) -> list:
    """Y_i = X W_i^T for every matrix in dqs (same bits, group and K) in one launch."""
    m = x.shape[0]
    if ys is None:
        ys = [torch.empty((m, dq["n"]), dtype=torch.float32, device=x.device) for dq in dqs]
    members = [(dq["w"], dq["scales"], dq["mins"], y, dq["n"]) for dq, y in zip(dqs, ys)]
    bits, group, k = dqs[0]["bits"], dqs[0]["group"], dqs[0]["k"]
    if workspace is None:
        need = qmm_gemm_grouped_workspace_bytes(members, m, k, bits, group)
        # Zeroed: the arrival counters at its start must read zero at first use.
        workspace = torch.zeros(max(need, 16), dtype=torch.uint8, device=x.device) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    qmm_gemm_grouped(members, x, m, k, bits, group, workspace=workspace, workspace_bytes=ws_bytes,
                     stream=stream)
    return ys


def moe(dst: dict, x: torch.Tensor, x_rows: torch.Tensor | None, offsets: torch.Tensor,
        p_rows: int, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if y is None:
        y = torch.empty((p_rows, dst["n"]), dtype=torch.float32, device=x.device)
    qmm_moe_gemm(dst["w"], dst["scales"], dst["mins"], x, x_rows, x.shape[0], offsets, y, p_rows,
                 dst["n_experts"], dst["n"], dst["k"], dst["bits"], dst["group"], stream=stream)
    return y


def moe_combine(dst: dict, x: torch.Tensor, x_rows: torch.Tensor | None, offsets: torch.Tensor,
                pair_token: torch.Tensor, pair_weight: torch.Tensor, p_rows: int, y: torch.Tensor,
                stream=None) -> torch.Tensor:
    """Expert rows with the routing-weighted combine: y[token[p]] += weight[p] * row p
    (y [tokens][n] fp32, accumulated in place)."""
    qmm_moe_combine(dst["w"], dst["scales"], dst["mins"], x, x_rows, x.shape[0], offsets, pair_token,
                    pair_weight, y, y.shape[0], p_rows, dst["n_experts"], dst["n"], dst["k"], dst["bits"],
                    dst["group"], stream=stream)
    return y


def moe_swiglu(dg: dict, du: dict, x: torch.Tensor, x_rows: torch.Tensor | None,
               offsets: torch.Tensor, p_rows: int, h: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Fused gate/up rows of the selected experts: h = silu(g) * u."""
    if h is None:
        h = torch.empty((p_rows, dg["n"]), dtype=torch.float32, device=x.device)
    qmm_moe_swiglu(dg["w"], dg["scales"], dg["mins"], du["w"], du["scales"], du["mins"], x, x_rows,
                   x.shape[0], offsets, h, p_rows, dg["n_experts"], dg["n"], dg["k"], dg["bits"],
                   dg["group"], stream=stream)
    return h


def unpack(dq: dict, stream=None) -> torch.Tensor:
    codes = torch.empty((dq["n"], dq["k"]), dtype=torch.uint8, device=dq["w"].device)
    qmm_unpack(dq["w"], codes, dq["n"], dq["k"], dq["bits"], stream=stream)
    return codes


class GemvBatch:
    """A prepared batched launch: host descriptors plus their device copy.

    items: list of (device matrix dict, x tensor [k], y tensor [n]); every
    matrix must share bits and group size."""

    def __init__(self, items, bits: int, group: int, device="cuda"):
        self.bits, self.group = bits, group
        self.host = (GemvDesc * len(items))()
        for d, (dq, x, y) in zip(self.host, items):
            assert dq["bits"] == bits and dq["group"] == group
            ptr = lambda t: 0 if t is None else t.data_ptr()
            d.w_packed, d.scales, d.mins = ptr(dq["w"]), ptr(dq["scales"]), ptr(dq["mins"])
            d.x, d.y = x.data_ptr(), y.data_ptr()
            d.n, d.k = dq["n"], dq["k"]
        qmm_gemv_batch_prepare(self.host, bits, group)
        raw = np.frombuffer(bytes(self.host), dtype=np.uint8).copy()
        self.device = torch.from_numpy(raw).to(device)
        self.keep = items  # the buffers must outlive the batch
        # The call's fixed arguments, converted once: a launch then costs one
        # foreign call (the host time before the first launch of a timed
        # region counts in it).
        self._launch = functools.partial(load().qmm_gemv_batched, self.device.data_ptr(),
                                         ctypes.addressof(self.host), len(self.host), bits, group)

    def __call__(self, stream=None) -> None:
        status = self._launch(_stream(stream))
        if status != QMM_OK:
            _check(status, "qmm_gemv_batched")
