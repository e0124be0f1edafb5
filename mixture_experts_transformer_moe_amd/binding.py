"""ctypes binding of libmoe.so (argument marshalling only).

Every function here passes ``tensor.data_ptr()`` and the current HIP stream to
the C entry point of the same name declared in ``include/moe.h``; all
arithmetic runs in the library's kernels.  PyTorch provides device memory and
streams.  There is no fallback: a missing library, a CPU tensor or a non-zero
status raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from .configs import MoEShape

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

# the entry points include/moe.h declares
EXPORTS = ("moe_version", "moe_status_string", "moe_last_error", "moe_workspace_bytes",
           "moe_route", "moe_permute", "moe_pack_weights", "moe_packed_bytes", "moe_grouped_gate_up",
           "moe_grouped_down", "moe_grouped_ffn", "moe_fp8_packed_bytes", "moe_quantize_weights_fp8",
           "moe_grouped_gate_up_fp8", "moe_grouped_down_fp8", "moe_combine",
           "moe_route_masked", "moe_train_workspace_bytes", "moe_packed_transposed_bytes",
           "moe_pack_weights_transposed", "moe_load_stats", "moe_grouped_gate_up_train",
           "moe_combine_backward", "moe_grouped_backward_h", "moe_grouped_backward_x",
           "moe_weight_grads", "moe_bias_grad", "moe_shared_ffn", "moe_permute_static")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("Fs", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("dtype", ctypes.c_int32)]


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(moe_shape)


def lib() -> ctypes.CDLL:
    """Loads libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_transformer_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_version.restype = ctypes.c_int
        L.moe_version.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [_SP]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P]
        L.moe_permute.restype = ctypes.c_int
        L.moe_permute.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.moe_permute_static.restype = ctypes.c_int
        L.moe_permute_static.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_pack_weights.restype = ctypes.c_int
        L.moe_pack_weights.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, _P]
        L.moe_packed_bytes.restype = ctypes.c_size_t
        L.moe_packed_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.moe_grouped_gate_up.restype = ctypes.c_int
        L.moe_grouped_gate_up.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_grouped_down.restype = ctypes.c_int
        L.moe_grouped_down.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P]
        L.moe_shared_ffn.restype = ctypes.c_int
        L.moe_shared_ffn.argtypes = [_SP, _P, _P, _P, _P, _P, _P]
        L.moe_grouped_ffn.restype = ctypes.c_int
        L.moe_grouped_ffn.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_fp8_packed_bytes.restype = ctypes.c_size_t
        L.moe_fp8_packed_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        L.moe_quantize_weights_fp8.restype = ctypes.c_int
        L.moe_quantize_weights_fp8.argtypes = [_P, _P, _P, ctypes.c_int64, ctypes.c_int32,
                                               ctypes.c_int32, _P]
        L.moe_grouped_gate_up_fp8.restype = ctypes.c_int
        L.moe_grouped_gate_up_fp8.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_grouped_down_fp8.restype = ctypes.c_int
        L.moe_grouped_down_fp8.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [_SP, _P, _P, _P, _P, _P, _P]
        # training pass
        L.moe_route_masked.restype = ctypes.c_int
        L.moe_route_masked.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_train_workspace_bytes.restype = ctypes.c_size_t
        L.moe_train_workspace_bytes.argtypes = [_SP]
        L.moe_packed_transposed_bytes.restype = ctypes.c_size_t
        L.moe_packed_transposed_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32]
        L.moe_pack_weights_transposed.restype = ctypes.c_int
        L.moe_pack_weights_transposed.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, _P]
        L.moe_load_stats.restype = ctypes.c_int
        L.moe_load_stats.argtypes = [_SP, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]
        L.moe_grouped_gate_up_train.restype = ctypes.c_int
        L.moe_grouped_gate_up_train.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        L.moe_combine_backward.restype = ctypes.c_int
        L.moe_combine_backward.argtypes = [_SP] + [_P] * 11
        L.moe_grouped_backward_h.restype = ctypes.c_int
        L.moe_grouped_backward_h.argtypes = [_SP] + [_P] * 9
        L.moe_grouped_backward_x.restype = ctypes.c_int
        L.moe_grouped_backward_x.argtypes = [_SP] + [_P] * 12
        L.moe_weight_grads.restype = ctypes.c_int
        L.moe_weight_grads.argtypes = [_SP] + [_P] * 15
        L.moe_bias_grad.restype = ctypes.c_int
        L.moe_bias_grad.argtypes = [_SP, _P, _P, _P, ctypes.c_size_t, _P]
        _lib = L
    return _lib


def make_shape(s: MoEShape) -> moe_shape:
    return moe_shape(s.T, s.D, s.E, s.k, s.F, s.Fs, float(s.alpha),
                     MOE_BF16 if s.dtype == "bf16" else MOE_F32)


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        detail = lib().moe_last_error().decode()
        raise MoEError(status, f"{what} failed ({lib().moe_status_string(status).decode()}): {detail}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def workspace_bytes(shape: moe_shape) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(shape)))


def moe_route(shape, x, w_router, bias, logits, topk_idx, topk_w, stream=None):
    _check(lib().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits),
                           _ptr(topk_idx), _ptr(topk_w), _stream(stream)), "moe_route")


def moe_permute(shape, topk_idx, x, counts, offsets, sorted_token, slot_of, x_perm, workspace,
                stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(x), _ptr(counts),
                             _ptr(offsets), _ptr(sorted_token), _ptr(slot_of), _ptr(x_perm),
                             _ptr(workspace), nbytes, _stream(stream)), "moe_permute")


def moe_permute_static(shape, topk_idx, x, counts, offsets, sorted_token, slot_of, x_perm, stream=None):
    _check(lib().moe_permute_static(ctypes.byref(shape), _ptr(topk_idx), _ptr(x), _ptr(counts),
                                    _ptr(offsets), _ptr(sorted_token), _ptr(slot_of), _ptr(x_perm),
                                    _stream(stream)), "moe_permute_static")


def moe_pack_weights(w, w_packed, count, rows, cols, dtype, stream=None):
    _check(lib().moe_pack_weights(_ptr(w), _ptr(w_packed), int(count), int(rows), int(cols), int(dtype),
                                  _stream(stream)), "moe_pack_weights")


def moe_packed_bytes(count, rows, cols, dtype) -> int:
    return int(lib().moe_packed_bytes(int(count), int(rows), int(cols), int(dtype)))


def pack(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Packed copy of a [rows, cols] or [count, rows, cols] weight tensor (a flat
    tensor of w's dtype holding moe_packed_bytes bytes)."""
    if w.dim() == 2:
        count, rows, cols = 1, w.shape[0], w.shape[1]
    else:
        count, rows, cols = w.shape
    dtype = MOE_BF16 if w.dtype == torch.bfloat16 else MOE_F32
    nbytes = moe_packed_bytes(count, rows, cols, dtype)
    if nbytes == 0 and count * rows * cols > 0:
        raise MoEError(MOE_ERR_INVALID_ARG, f"moe_packed_bytes: cannot pack [{count}, {rows}, {cols}]")
    out = torch.empty(nbytes // w.element_size(), dtype=w.dtype, device=w.device)
    moe_pack_weights(w.contiguous(), out, count, rows, cols, dtype, stream)
    return out


def moe_grouped_gate_up(shape, x_perm, sorted_token, x, offsets, w_gate_up, ws_gate_up, h,
                        stream=None):
    _check(lib().moe_grouped_gate_up(ctypes.byref(shape), _ptr(x_perm), _ptr(sorted_token), _ptr(x),
                                     _ptr(offsets), _ptr(w_gate_up), _ptr(ws_gate_up), _ptr(h),
                                     _stream(stream)), "moe_grouped_gate_up")


def moe_grouped_down(shape, h, offsets, w_down, ws_down, y_perm, y_shared, stream=None):
    _check(lib().moe_grouped_down(ctypes.byref(shape), _ptr(h), _ptr(offsets), _ptr(w_down),
                                  _ptr(ws_down), _ptr(y_perm), _ptr(y_shared), _stream(stream)),
           "moe_grouped_down")


def moe_shared_ffn(shape, x, ws_gate_up, ws_down, h_shared, y_shared, stream=None):
    _check(lib().moe_shared_ffn(ctypes.byref(shape), _ptr(x), _ptr(ws_gate_up), _ptr(ws_down),
                                _ptr(h_shared), _ptr(y_shared), _stream(stream)), "moe_shared_ffn")


def moe_grouped_ffn(shape, x_perm, sorted_token, x, offsets, w_gate_up, w_down, ws_gate_up, ws_down,
                    h, y_perm, y_shared, stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(shape), _ptr(x_perm), _ptr(sorted_token), _ptr(x),
                                 _ptr(offsets), _ptr(w_gate_up), _ptr(w_down), _ptr(ws_gate_up),
                                 _ptr(ws_down), _ptr(h), _ptr(y_perm), _ptr(y_shared),
                                 _stream(stream)), "moe_grouped_ffn")


def moe_fp8_packed_bytes(count, rows, cols) -> int:
    return int(lib().moe_fp8_packed_bytes(int(count), int(rows), int(cols)))


def moe_quantize_weights_fp8(w, w_fp8, scales, count, rows, cols, stream=None):
    _check(lib().moe_quantize_weights_fp8(_ptr(w), _ptr(w_fp8), _ptr(scales), int(count), int(rows),
                                          int(cols), _stream(stream)), "moe_quantize_weights_fp8")


def quantize_fp8(w: torch.Tensor, stream=None):
    """FP8 codes (flat uint8, packed) and row scales (float32 [count, rows]) of a
    bf16 [rows, cols] or [count, rows, cols] weight tensor."""
    if w.dim() == 2:
        count, rows, cols = 1, w.shape[0], w.shape[1]
    else:
        count, rows, cols = w.shape
    nbytes = moe_fp8_packed_bytes(count, rows, cols)
    if nbytes == 0 and count * rows * cols > 0:
        raise MoEError(MOE_ERR_INVALID_ARG, f"moe_fp8_packed_bytes: cannot pack [{count}, {rows}, {cols}]")
    codes = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    scales = torch.empty((count, rows), dtype=torch.float32, device=w.device)
    moe_quantize_weights_fp8(w.contiguous(), codes, scales, count, rows, cols, stream)
    return codes, scales


def moe_grouped_gate_up_fp8(shape, x_perm, sorted_token, x, offsets, w_gate_up, w_gate_up_scale,
                            ws_gate_up, ws_gate_up_scale, h, stream=None):
    _check(lib().moe_grouped_gate_up_fp8(ctypes.byref(shape), _ptr(x_perm), _ptr(sorted_token),
                                         _ptr(x), _ptr(offsets), _ptr(w_gate_up),
                                         _ptr(w_gate_up_scale), _ptr(ws_gate_up),
                                         _ptr(ws_gate_up_scale), _ptr(h), _stream(stream)),
           "moe_grouped_gate_up_fp8")


def moe_grouped_down_fp8(shape, h, offsets, w_down, w_down_scale, ws_down, ws_down_scale, y_perm,
                         y_shared, stream=None):
    _check(lib().moe_grouped_down_fp8(ctypes.byref(shape), _ptr(h), _ptr(offsets), _ptr(w_down),
                                      _ptr(w_down_scale), _ptr(ws_down), _ptr(ws_down_scale),
                                      _ptr(y_perm), _ptr(y_shared), _stream(stream)),
           "moe_grouped_down_fp8")


def moe_combine(shape, y_perm, y_shared, slot_of, topk_w, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(y_shared), _ptr(slot_of),
                             _ptr(topk_w), _ptr(out), _stream(stream)), "moe_combine")


# ---------------------------------------------------------------------------
# buffers and the whole layer
# ---------------------------------------------------------------------------

def storage_dtype(s: MoEShape) -> torch.dtype:
    return torch.bfloat16 if s.dtype == "bf16" else torch.float32


def to_device(a, s: MoEShape, device) -> torch.Tensor:
    """Storage-encoded numpy array (fp32, or bf16 bits as uint16) -> device tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


@dataclass
class LayerBuffers:
    logits: torch.Tensor
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_token: torch.Tensor
    slot_of: torch.Tensor
    x_perm: Optional[torch.Tensor]
    workspace: torch.Tensor
    h: torch.Tensor
    y_perm: torch.Tensor
    y_shared: Optional[torch.Tensor]
    out: torch.Tensor


def alloc_buffers(s: MoEShape, device="cuda", with_x_perm: bool = True) -> LayerBuffers:
    dt = storage_dtype(s)
    S = s.S
    i32 = dict(dtype=torch.int32, device=device)
    shape_c = make_shape(s)
    ws = max(workspace_bytes(shape_c), 256)
    return LayerBuffers(
        logits=torch.empty((s.T, s.E), dtype=torch.float32, device=device),
        topk_idx=torch.empty((s.T, s.k), **i32),
        topk_w=torch.empty((s.T, s.k), dtype=torch.float32, device=device),
        counts=torch.empty((s.E,), **i32),
        offsets=torch.empty((s.E + 1,), **i32),
        sorted_token=torch.empty((S,), **i32),
        slot_of=torch.empty((s.T, s.k), **i32),
        x_perm=torch.empty((S, s.D), dtype=dt, device=device) if with_x_perm else None,
        workspace=torch.empty((ws,), dtype=torch.uint8, device=device),
        h=torch.empty((S * s.F + s.T * s.Fs,), dtype=dt, device=device),
        y_perm=torch.empty((S, s.D), dtype=dt, device=device),
        y_shared=torch.empty((s.T, s.D), dtype=dt, device=device) if s.Fs else None,
        out=torch.empty((s.T, s.D), dtype=dt, device=device),
    )


@dataclass
class LayerWeights:
    """Layer weights on the device; expert weights in the packed layout (bf16),
    or FP8 codes with their row scales (``fp8``)."""
    w_router: torch.Tensor
    bias: Optional[torch.Tensor]
    w_gate_up: torch.Tensor       # E packed [2F, D] matrices (flat)
    w_down: torch.Tensor          # E packed [D, F] matrices (flat)
    ws_gate_up: Optional[torch.Tensor]
    ws_down: Optional[torch.Tensor]
    fp8: bool = False
    w_gate_up_scale: Optional[torch.Tensor] = None    # FP8: [E, 2F]
    w_down_scale: Optional[torch.Tensor] = None       # FP8: [E, D]
    ws_gate_up_scale: Optional[torch.Tensor] = None   # FP8: [1, 2Fs]
    ws_down_scale: Optional[torch.Tensor] = None      # FP8: [1, D]


def upload_weights(s: MoEShape, w_router, bias, wgu, wd, shared, device="cuda",
                   fp8: bool = False) -> LayerWeights:
    """Host arrays in storage encoding -> LayerWeights (expert weights packed on
    the device, or quantised to FP8 there)."""
    td = lambda a: to_device(a, s, device)
    router = td(w_router)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(device)
    if not fp8:
        return LayerWeights(
            w_router=router, bias=b,
            w_gate_up=pack(td(wgu)),
            w_down=pack(td(wd)),
            ws_gate_up=None if shared is None else pack(td(shared[0])),
            ws_down=None if shared is None else pack(td(shared[1])),
        )
    gu, gus = quantize_fp8(td(wgu))
    dn, dns = quantize_fp8(td(wd))
    sgu = sgus = sdn = sdns = None
    if shared is not None:
        sgu, sgus = quantize_fp8(td(shared[0]))
        sdn, sdns = quantize_fp8(td(shared[1]))
    return LayerWeights(w_router=router, bias=b, w_gate_up=gu, w_down=dn, ws_gate_up=sgu,
                        ws_down=sdn, fp8=True, w_gate_up_scale=gus, w_down_scale=dns,
                        ws_gate_up_scale=sgus, ws_down_scale=sdns)


def upload(inputs, device="cuda", fp8: bool = False):
    """Seeded inputs (``inputs.LayerInputs``) -> (x, LayerWeights) on the device."""
    s = inputs.shape
    wgu, wd = inputs.all_experts()
    w = upload_weights(s, inputs.w_router, inputs.bias, wgu, wd, inputs.shared(), device, fp8)
    return to_device(inputs.x, s, device), w


def layer_forward(s: MoEShape, x: torch.Tensor, w: LayerWeights, b: LayerBuffers,
                  stream=None) -> torch.Tensor:
    """route -> permute -> grouped gate/up + SwiGLU -> grouped down -> combine."""
    c = make_shape(s)
    moe_route(c, x, w.w_router, w.bias, b.logits, b.topk_idx, b.topk_w, stream)
    moe_permute(c, b.topk_idx, x, b.counts, b.offsets, b.sorted_token, b.slot_of, b.x_perm,
                b.workspace, stream)
    grouped_ffn(c, x, w, b, stream)
    moe_combine(c, b.y_perm, b.y_shared, b.slot_of, b.topk_w, b.out, stream)
    return b.out


def grouped_ffn(c: moe_shape, x: torch.Tensor, w: LayerWeights, b: LayerBuffers, stream=None):
    """Both grouped GEMMs, with bf16 or FP8 expert weights."""
    if w.fp8:
        moe_grouped_gate_up_fp8(c, b.x_perm, b.sorted_token, x, b.offsets, w.w_gate_up,
                                w.w_gate_up_scale, w.ws_gate_up, w.ws_gate_up_scale, b.h, stream)
        moe_grouped_down_fp8(c, b.h, b.offsets, w.w_down, w.w_down_scale, w.ws_down, w.ws_down_scale,
                             b.y_perm, b.y_shared, stream)
    else:
        moe_grouped_gate_up(c, b.x_perm, b.sorted_token, x, b.offsets, w.w_gate_up, w.ws_gate_up,
                            b.h, stream)
        moe_grouped_down(c, b.h, b.offsets, w.w_down, w.ws_down, b.y_perm, b.y_shared, stream)


# ---------------------------------------------------------------------------
# training pass
# ---------------------------------------------------------------------------

def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_route_masked(shape, x, w_router, bias, mask, logits, topk_idx, topk_w, stream=None):
    _check(lib().moe_route_masked(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(mask),
                                  _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_route_masked")


def train_workspace_bytes(shape: moe_shape) -> int:
    return int(lib().moe_train_workspace_bytes(ctypes.byref(shape)))


def moe_packed_transposed_bytes(count, rows, cols, k_padded) -> int:
    return int(lib().moe_packed_transposed_bytes(int(count), int(rows), int(cols), int(k_padded)))


def moe_pack_weights_transposed(w, w_packed, count, rows, cols, k_padded, stream=None):
    _check(lib().moe_pack_weights_transposed(_ptr(w), _ptr(w_packed), int(count), int(rows), int(cols),
                                             int(k_padded), _stream(stream)), "moe_pack_weights_transposed")


def pack_transposed(w: torch.Tensor, k_padded: Optional[int] = None, stream=None) -> torch.Tensor:
    """Packed transposes of a bf16 [rows, cols] or [count, rows, cols] tensor
    (flat bf16 tensor of moe_packed_transposed_bytes bytes)."""
    if w.dim() == 2:
        count, rows, cols = 1, w.shape[0], w.shape[1]
    else:
        count, rows, cols = w.shape
    kp = rows if k_padded is None else k_padded
    nbytes = moe_packed_transposed_bytes(count, rows, cols, kp)
    if nbytes == 0 and count * cols * kp > 0:
        raise MoEError(MOE_ERR_INVALID_ARG, f"cannot pack the transpose of [{count}, {rows}, {cols}]")
    out = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w.device)
    moe_pack_weights_transposed(w.contiguous(), out, count, rows, cols, kp, stream)
    return out


def moe_load_stats(shape, logits, topk_idx, counts, counts_global, beta, f, p, aux_loss, aux_coef,
                   workspace, stream=None):
    _check(lib().moe_load_stats(ctypes.byref(shape), _ptr(logits), _ptr(topk_idx), _ptr(counts),
                                _ptr(counts_global), float(beta), _ptr(f), _ptr(p), _ptr(aux_loss),
                                _ptr(aux_coef), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_load_stats")


def moe_grouped_gate_up_train(shape, x_perm, sorted_token, x, offsets, w_gate_up, ws_gate_up, gu, h,
                              stream=None):
    _check(lib().moe_grouped_gate_up_train(ctypes.byref(shape), _ptr(x_perm), _ptr(sorted_token), _ptr(x),
                                           _ptr(offsets), _ptr(w_gate_up), _ptr(ws_gate_up), _ptr(gu),
                                           _ptr(h), _stream(stream)), "moe_grouped_gate_up_train")


def moe_combine_backward(shape, dout, y_perm, slot_of, topk_idx, topk_w, logits, aux_coef, dy_perm, dz,
                         dz_bf16, stream=None):
    _check(lib().moe_combine_backward(ctypes.byref(shape), _ptr(dout), _ptr(y_perm), _ptr(slot_of),
                                      _ptr(topk_idx), _ptr(topk_w), _ptr(logits), _ptr(aux_coef),
                                      _ptr(dy_perm), _ptr(dz), _ptr(dz_bf16), _stream(stream)),
           "moe_combine_backward")


def moe_grouped_backward_h(shape, dy_perm, dout, offsets, w_down_t, ws_down_t, gu, dh, dgu, stream=None):
    _check(lib().moe_grouped_backward_h(ctypes.byref(shape), _ptr(dy_perm), _ptr(dout), _ptr(offsets),
                                        _ptr(w_down_t), _ptr(ws_down_t), _ptr(gu), _ptr(dh), _ptr(dgu),
                                        _stream(stream)), "moe_grouped_backward_h")


def moe_grouped_backward_x(shape, dgu, offsets, w_gate_up_t, ws_gate_up_t, dz_bf16, w_router_t, slot_of,
                           dx_perm, dx_shared, dx_router, dx, stream=None):
    _check(lib().moe_grouped_backward_x(ctypes.byref(shape), _ptr(dgu), _ptr(offsets), _ptr(w_gate_up_t),
                                        _ptr(ws_gate_up_t), _ptr(dz_bf16), _ptr(w_router_t), _ptr(slot_of),
                                        _ptr(dx_perm), _ptr(dx_shared), _ptr(dx_router), _ptr(dx),
                                        _stream(stream)), "moe_grouped_backward_x")


def moe_weight_grads(shape, x, sorted_token, x_perm, offsets, dgu, dy_perm, dout, h, dz_bf16,
                     dw_gate_up, dw_down, dws_gate_up, dws_down, dw_router, stream=None):
    _check(lib().moe_weight_grads(ctypes.byref(shape), _ptr(x), _ptr(sorted_token), _ptr(x_perm),
                                  _ptr(offsets), _ptr(dgu), _ptr(dy_perm), _ptr(dout), _ptr(h),
                                  _ptr(dz_bf16), _ptr(dw_gate_up), _ptr(dw_down), _ptr(dws_gate_up),
                                  _ptr(dws_down), _ptr(dw_router), _stream(stream)), "moe_weight_grads")


def moe_bias_grad(shape, dz, dbias, workspace, stream=None):
    _check(lib().moe_bias_grad(ctypes.byref(shape), _ptr(dz), _ptr(dbias), _ptr(workspace),
                               _nbytes(workspace), _stream(stream)), "moe_bias_grad")


@dataclass
class TrainWeights:
    """The forward weights plus the packed transposes the backward products use."""
    fwd: LayerWeights
    w_down_t: torch.Tensor        # E packed [F, D]
    w_gate_up_t: torch.Tensor     # E packed [D, 2F]
    ws_down_t: Optional[torch.Tensor]
    ws_gate_up_t: Optional[torch.Tensor]
    w_router_t: torch.Tensor      # packed [D, 256]


def upload_train_weights(s: MoEShape, w_router, bias, wgu, wd, shared, device="cuda") -> TrainWeights:
    if s.dtype != "bf16":
        raise MoEError(MOE_ERR_UNSUPPORTED, "the training pass is bf16 only")
    fwd = upload_weights(s, w_router, bias, wgu, wd, shared, device)
    td = lambda a: to_device(a, s, device)
    return TrainWeights(
        fwd=fwd,
        w_down_t=pack_transposed(td(wd)),
        w_gate_up_t=pack_transposed(td(wgu)),
        ws_down_t=None if shared is None else pack_transposed(td(shared[1])),
        ws_gate_up_t=None if shared is None else pack_transposed(td(shared[0])),
        w_router_t=pack_transposed(fwd.w_router, k_padded=256),
    )


@dataclass
class TrainBuffers:
    fwd: LayerBuffers
    mask: Optional[torch.Tensor]
    gu: torch.Tensor              # [S, 2F] + [T, 2Fs]
    f: torch.Tensor
    p: torch.Tensor
    aux_loss: torch.Tensor
    aux_coef: torch.Tensor
    train_ws: torch.Tensor
    dy_perm: torch.Tensor
    dz: torch.Tensor
    dz16: torch.Tensor
    dh: torch.Tensor
    dgu: torch.Tensor
    dx_perm: torch.Tensor
    dx_shared: Optional[torch.Tensor]
    dx_router: torch.Tensor
    dx: torch.Tensor
    dw_gate_up: torch.Tensor
    dw_down: torch.Tensor
    dws_gate_up: Optional[torch.Tensor]
    dws_down: Optional[torch.Tensor]
    dw_router: torch.Tensor
    dbias: torch.Tensor


def alloc_train_buffers(s: MoEShape, mask: Optional[torch.Tensor] = None, device="cuda",
                        with_x_perm: bool = False) -> TrainBuffers:
    bf, f32 = dict(dtype=torch.bfloat16, device=device), dict(dtype=torch.float32, device=device)
    S, T = s.S, s.T
    c = make_shape(s)
    return TrainBuffers(
        fwd=alloc_buffers(s, device, with_x_perm=with_x_perm), mask=mask,
        gu=torch.empty((S * 2 * s.F + T * 2 * s.Fs,), **bf),
        f=torch.empty((s.E,), **f32), p=torch.empty((s.E,), **f32),
        aux_loss=torch.empty((1,), **f32), aux_coef=torch.empty((s.E,), **f32),
        train_ws=torch.empty((max(train_workspace_bytes(c), 256),), dtype=torch.uint8, device=device),
        dy_perm=torch.empty((S, s.D), **bf), dz=torch.empty((T, s.E), **f32),
        dz16=torch.empty((T, 256), **bf),
        dh=torch.empty((S * s.F + T * s.Fs,), **bf), dgu=torch.empty((S * 2 * s.F + T * 2 * s.Fs,), **bf),
        dx_perm=torch.empty((S, s.D), **bf),
        dx_shared=torch.empty((T, s.D), **bf) if s.Fs else None,
        dx_router=torch.empty((T, s.D), **bf), dx=torch.empty((T, s.D), **bf),
        dw_gate_up=torch.empty((s.E, 2 * s.F, s.D), **bf), dw_down=torch.empty((s.E, s.D, s.F), **bf),
        dws_gate_up=torch.empty((2 * s.Fs, s.D), **bf) if s.Fs else None,
        dws_down=torch.empty((s.D, s.Fs), **bf) if s.Fs else None,
        dw_router=torch.empty((s.E, s.D), **f32), dbias=torch.empty((s.E,), **f32),
    )


def train_forward(s: MoEShape, x: torch.Tensor, w: TrainWeights, b: TrainBuffers, beta: float,
                  counts_global: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Masked route -> permute -> load statistics -> gate/up keeping [g | u] ->
    down -> combine."""
    c = make_shape(s)
    fb, fw = b.fwd, w.fwd
    moe_route_masked(c, x, fw.w_router, fw.bias, b.mask, fb.logits, fb.topk_idx, fb.topk_w, stream)
    moe_permute(c, fb.topk_idx, x, fb.counts, fb.offsets, fb.sorted_token, fb.slot_of, fb.x_perm,
                fb.workspace, stream)
    moe_load_stats(c, fb.logits, fb.topk_idx, fb.counts, counts_global, beta, b.f, b.p, b.aux_loss,
                   b.aux_coef, b.train_ws, stream)
    moe_grouped_gate_up_train(c, fb.x_perm, fb.sorted_token, x, fb.offsets, fw.w_gate_up, fw.ws_gate_up,
                              b.gu, fb.h, stream)
    moe_grouped_down(c, fb.h, fb.offsets, fw.w_down, fw.ws_down, fb.y_perm, fb.y_shared, stream)
    moe_combine(c, fb.y_perm, fb.y_shared, fb.slot_of, fb.topk_w, fb.out, stream)
    return fb.out


def train_backward(s: MoEShape, x: torch.Tensor, dout: torch.Tensor, w: TrainWeights, b: TrainBuffers,
                   with_aux: bool = True, stream=None) -> torch.Tensor:
    """Combine backward -> dh and SwiGLU backward -> dx -> weight gradients."""
    c = make_shape(s)
    fb = b.fwd
    moe_combine_backward(c, dout, fb.y_perm, fb.slot_of, fb.topk_idx, fb.topk_w, fb.logits,
                         b.aux_coef if with_aux else None, b.dy_perm, b.dz, b.dz16, stream)
    moe_grouped_backward_h(c, b.dy_perm, dout, fb.offsets, w.w_down_t, w.ws_down_t, b.gu, b.dh, b.dgu,
                           stream)
    moe_grouped_backward_x(c, b.dgu, fb.offsets, w.w_gate_up_t, w.ws_gate_up_t, b.dz16, w.w_router_t,
                           fb.slot_of, b.dx_perm, b.dx_shared, b.dx_router, b.dx, stream)
    moe_weight_grads(c, x, fb.sorted_token, fb.x_perm, fb.offsets, b.dgu, b.dy_perm, dout, fb.h, b.dz16,
                     b.dw_gate_up, b.dw_down, b.dws_gate_up, b.dws_down, b.dw_router, stream)
    moe_bias_grad(c, b.dz, b.dbias, b.train_ws, stream)
    return b.dx
