"""Producer-fused NVFP4 activation quantization for MI355X (gfx950).

Thin ctypes binding over ``libnvfp4act.so`` (C ABI in ``include/nvfp4act.h``).
This module only turns torch tensors into pointers and sizes, calls the entry
point of the same name on the current torch stream, and raises on a nonzero
status: every step of the computation runs in the library's HIP kernels.
If the library is missing the import fails loudly; there is no fallback.

Entry points (see ``include/nvfp4act.h`` for the exact contract):
  nvfp4_quantize(x, global_amax)                          standalone quantize
  rms_adaln_nvfp4(x, weight, table, frame_idx, eps, global_amax)
  swiglu_nvfp4(projection, global_amax)                   value-first [m, 2f]
  swiglu_packed_nvfp4(projection, global_amax, bias, interleaved)
                                                          bias before SiLU; value-first
                                                          or paired columns
each returning ``(codes, scales)``; and the per-call (dynamic) amax forms
  nvfp4_quantize_dynamic(x), rms_adaln_nvfp4_dynamic(x, weight, table, frame_idx, eps),
  residual_rms_nvfp4(h, gamma, eps, global_amax, residual=(o, bias, scale))
                                                          fp32 residual stream (in place) +
                                                          RMSNorm with an fp32 weight
  residual_rms_adaln_nvfp4(h, weight, table, frame_idx, eps, global_amax,
                           residual=(o, bias, gate_table))
                                                          gated residual (own table) + RMSNorm
                                                          + adaLN (next block's table)
  rms_silu_nvfp4(x, gamma, eps, global_amax)              fp16 channels-last [rows, c]:
                                                          RMSNorm + SiLU, plain scale layout
  ln_adaln_fp8(x, scale, shift, eps, act_scale)            fp16 [m, k]: LayerNorm (fp32 statistics)
                                                          + adaLN -> per-tensor FP8 E4M3 codes
                                                          [m, k]; ln_adaln_fp8_dynamic(x, scale,
                                                          shift, eps) returns (codes, act_scale)
  swiglu_nvfp4_dynamic(projection), swiglu_packed_nvfp4_dynamic(projection, bias, interleaved),
  residual_rms_nvfp4_dynamic(h, gamma, eps, residual),
  residual_rms_adaln_nvfp4_dynamic(h, weight, table, frame_idx, eps, residual),
  rms_silu_nvfp4_dynamic(x, gamma, eps)
returning ``(codes, scales, amax)`` with ``amax`` a one-element float32 device tensor, codes ``[m, k/2]`` uint8, scales
``[pad(m), k/16]`` uint8 in the 128x4 swizzle (buffer shapes as the FastVideo
API page's ``new_quantized``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4act.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libnvfp4act.so is not built (run python nvfp4_activation_quantization_amd/build.py "
                      "or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

_P, _I64, _F, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
_SIGS = {
    "nvfp4act_padded_rows": (_I64, [_I64]),
    "nvfp4act_codes_bytes": (_I64, [_I64, _I64]),
    "nvfp4act_scales_bytes": (_I64, [_I64, _I64]),
    "nvfp4act_global_scale": (_F, [_F]),
    "nvfp4act_status_string": (ctypes.c_char_p, [_I]),
    "nvfp4act_last_hip_error": (_I, []),
    "nvfp4act_init": (_I, []),
    "nvfp4_quantize": (_I, [_P, _I64, _I64, _F, _P, _P, _P]),
    "rms_adaln_nvfp4": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _F, _P, _P, _P, _P, _P, _P]),
    "swiglu_nvfp4": (_I, [_P, _P, _I64, _I64, _I64, _F, _P, _P, _P, _P]),
    "nvfp4_quantize_dynamic": (_I, [_P, _I64, _I64, _P, _P, _P, _P]),
    "rms_adaln_nvfp4_dynamic": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "swiglu_nvfp4_dynamic": (_I, [_P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "swiglu_packed_nvfp4": (_I, [_P, _P, _I, _I64, _I64, _I64, _F, _P, _P, _P, _P]),
    "swiglu_packed_nvfp4_dynamic": (_I, [_P, _P, _I, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "residual_rms_nvfp4": (_I, [_P, _P, _P, _P, _P, _F, _I64, _I64, _F, _P, _P, _P, _P, _P]),
    "residual_rms_nvfp4_dynamic": (_I, [_P, _P, _P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "residual_rms_adaln_nvfp4": (_I, [_P, _P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _F,
                                      _P, _P, _P, _P, _P, _P]),
    "residual_rms_adaln_nvfp4_dynamic": (_I, [_P, _P, _P, _P, _I64, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64,
                                              _P, _P, _P, _P, _P, _P, _P]),
    "rms_silu_nvfp4": (_I, [_P, _P, _F, _I64, _I64, _F, _P, _P, _P, _P, _P]),
    "rms_silu_nvfp4_dynamic": (_I, [_P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "ln_adaln_fp8": (_I, [_P, _P, _P, _F, _I64, _I64, _F, _P, _P, _P, _P, _P]),
    "ln_adaln_fp8_dynamic": (_I, [_P, _P, _P, _F, _I64, _I64, _P, _P, _P, _P, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)
STATUS = {0: "ok", 1: "null", 2: "shape", 3: "align", 4: "value", 5: "device", 6: "launch", 7: "table"}


class NVFP4Error(RuntimeError):
    def __init__(self, status: int):
        msg = _lib.nvfp4act_status_string(status).decode()
        if status == 6:
            msg += " (hip error %d)" % _lib.nvfp4act_last_hip_error()
        super().__init__("nvfp4act status %d: %s" % (status, msg))
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise NVFP4Error(status)


def library():
    """The loaded ctypes library (raw C ABI)."""
    return _lib


def padded_rows(m: int) -> int:
    return _lib.nvfp4act_padded_rows(m)


def global_scale(global_amax: float) -> float:
    return _lib.nvfp4act_global_scale(global_amax)


def init() -> None:
    """Build the per-device tables on the current device (optional; waits)."""
    _check(_lib.nvfp4act_init())


def new_quantized(m: int, k: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Output buffers for an [m, k] activation: codes [m, k/2], scales [pad(m), k/16]."""
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((padded_rows(m), k // 16), dtype=torch.uint8, device=device)
    return codes, scales


def _bf16_ptr(t: torch.Tensor, name: str) -> int:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("%s must hold bf16 values (bfloat16 or a 16-bit integer view)" % name)
    if not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    return t.data_ptr()


def _out_ptr(t, dtype, shape, name):
    if t is None:
        return 0
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("%s must be a contiguous %s device tensor of shape %s" % (name, dtype, tuple(shape)))
    return t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def nvfp4_quantize(x: torch.Tensor, global_amax: float, codes=None, scales=None, stream=None):
    """Standalone NVFP4 quantize of a contiguous bf16 [m, k] tensor."""
    m, k = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, x.device)
    _check(_lib.nvfp4_quantize(_bf16_ptr(x, "x"), m, k, float(global_amax),
                               _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                               _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                               _stream(stream, x.device)))
    return codes, scales


def _amax_ptr(amax_out, device):
    if amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=device)
    if amax_out.dtype != torch.float32 or amax_out.numel() < 1 or not amax_out.is_cuda:
        raise ValueError("amax_out must be a float32 device tensor with at least one element")
    return amax_out, amax_out.data_ptr()


def nvfp4_quantize_dynamic(x: torch.Tensor, amax_out=None, codes=None, scales=None, stream=None):
    """Standalone NVFP4 quantize under the tensor's own amax (computed on the device)."""
    m, k = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, x.device)
    amax_out, ap = _amax_ptr(amax_out, x.device)
    _check(_lib.nvfp4_quantize_dynamic(_bf16_ptr(x, "x"), m, k, ap,
                                       _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                                       _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                                       _stream(stream, x.device)))
    return codes, scales, amax_out


def rms_adaln_nvfp4(x: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                    eps: float, global_amax: float, codes=None, scales=None, rstd_out=None, y_out=None,
                    status_word=None, stream=None):
    """Fused RMSNorm + adaLN -> NVFP4.

    x [m, k] bf16; weight [k] bf16; table [T, 2, k] bf16 holding (shift, scale) per
    frame; frame_idx [m] int32.  Optional outputs: rstd_out [m] fp32, y_out [m, k]
    bf16, status_word [1] int32/uint32 (bit 0: a frame index was out of range).
    """
    m, k = x.shape
    if not x.is_contiguous() or not table.is_contiguous() or not weight.is_contiguous():
        raise ValueError("x, weight and table must be contiguous")
    if table.dim() != 3 or table.shape[1] != 2 or table.shape[2] != k:
        raise ValueError("table must be [T, 2, k]")
    if frame_idx.dtype != torch.int32 or not frame_idx.is_contiguous() or frame_idx.numel() != m:
        raise ValueError("frame_idx must be a contiguous int32 tensor of m elements")
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, x.device)
    tab = _bf16_ptr(table, "table")
    sw = 0
    if status_word is not None:
        if status_word.dtype not in (torch.int32, torch.uint32) or not status_word.is_cuda:
            raise ValueError("status_word must be a 32-bit device tensor")
        sw = status_word.data_ptr()
    _check(_lib.rms_adaln_nvfp4(
        _bf16_ptr(x, "x"), _bf16_ptr(weight, "weight"), tab, tab + 2 * k, 2 * k, table.shape[0],
        frame_idx.data_ptr(), float(eps), m, k, float(global_amax),
        _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
        _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
        _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
        _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k), "y_out") if y_out is not None else 0,
        sw, _stream(stream, x.device)))
    return codes, scales


def rms_adaln_nvfp4_dynamic(x: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                            eps: float, amax_out=None, codes=None, scales=None, rstd_out=None, y_out=None,
                            status_word=None, stream=None):
    """Fused RMSNorm + adaLN -> NVFP4 under the amax of this call's own y (computed on the
    device by an amax pass).  Arguments as rms_adaln_nvfp4 without global_amax."""
    m, k = x.shape
    if not x.is_contiguous() or not table.is_contiguous() or not weight.is_contiguous():
        raise ValueError("x, weight and table must be contiguous")
    if table.dim() != 3 or table.shape[1] != 2 or table.shape[2] != k:
        raise ValueError("table must be [T, 2, k]")
    if frame_idx.dtype != torch.int32 or not frame_idx.is_contiguous() or frame_idx.numel() != m:
        raise ValueError("frame_idx must be a contiguous int32 tensor of m elements")
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, x.device)
    amax_out, ap = _amax_ptr(amax_out, x.device)
    tab = _bf16_ptr(table, "table")
    sw = 0
    if status_word is not None:
        if status_word.dtype not in (torch.int32, torch.uint32) or not status_word.is_cuda:
            raise ValueError("status_word must be a 32-bit device tensor")
        sw = status_word.data_ptr()
    _check(_lib.rms_adaln_nvfp4_dynamic(
        _bf16_ptr(x, "x"), _bf16_ptr(weight, "weight"), tab, tab + 2 * k, 2 * k, table.shape[0],
        frame_idx.data_ptr(), float(eps), m, k, ap,
        _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
        _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
        _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
        _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k), "y_out") if y_out is not None else 0,
        sw, _stream(stream, x.device)))
    return codes, scales, amax_out


def swiglu_nvfp4(projection: torch.Tensor, global_amax: float, codes=None, scales=None, y_out=None,
                 gate: torch.Tensor | None = None, stream=None):
    """SwiGLU -> NVFP4.

    With gate=None, projection is a value-first [m, 2f] tensor (up = first f columns,
    gate = last f).  Otherwise projection is up [m, f] and gate [m, f], two views with
    the same row stride (unit column stride).
    """
    if gate is None:
        m, two_f = projection.shape
        f = two_f // 2
        if not projection.is_contiguous():
            raise ValueError("projection must be contiguous")
        up_ptr = _bf16_ptr(projection, "projection")
        gate_ptr = up_ptr + 2 * f
        ld = two_f
    else:
        m, f = projection.shape
        if gate.shape != projection.shape or projection.stride(1) != 1 or gate.stride(1) != 1 \
                or projection.stride(0) != gate.stride(0):
            raise ValueError("up and gate must be [m, f] views with unit column stride and equal row stride")
        up_ptr = _bf16_ptr(projection, "up")
        gate_ptr = _bf16_ptr(gate, "gate")
        ld = projection.stride(0)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, f, projection.device)
    _check(_lib.swiglu_nvfp4(up_ptr, gate_ptr, ld, m, f, float(global_amax),
                             _out_ptr(codes, torch.uint8, (m, f // 2), "codes"),
                             _out_ptr(scales, torch.uint8, (padded_rows(m), f // 16), "scales"),
                             _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, f), "y_out")
                             if y_out is not None else 0,
                             _stream(stream, projection.device)))
    return codes, scales


def swiglu_nvfp4_dynamic(projection: torch.Tensor, amax_out=None, codes=None, scales=None, y_out=None,
                         gate: torch.Tensor | None = None, stream=None):
    """SwiGLU -> NVFP4 under the amax of this call's own y (computed on the device).
    Arguments as swiglu_nvfp4 without global_amax."""
    if gate is None:
        m, two_f = projection.shape
        f = two_f // 2
        if not projection.is_contiguous():
            raise ValueError("projection must be contiguous")
        up_ptr = _bf16_ptr(projection, "projection")
        gate_ptr = up_ptr + 2 * f
        ld = two_f
    else:
        m, f = projection.shape
        if gate.shape != projection.shape or projection.stride(1) != 1 or gate.stride(1) != 1 \
                or projection.stride(0) != gate.stride(0):
            raise ValueError("up and gate must be [m, f] views with unit column stride and equal row stride")
        up_ptr = _bf16_ptr(projection, "up")
        gate_ptr = _bf16_ptr(gate, "gate")
        ld = projection.stride(0)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, f, projection.device)
    amax_out, ap = _amax_ptr(amax_out, projection.device)
    _check(_lib.swiglu_nvfp4_dynamic(up_ptr, gate_ptr, ld, m, f, ap,
                                     _out_ptr(codes, torch.uint8, (m, f // 2), "codes"),
                                     _out_ptr(scales, torch.uint8, (padded_rows(m), f // 16), "scales"),
                                     _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, f), "y_out")
                                     if y_out is not None else 0,
                                     _stream(stream, projection.device)))
    return codes, scales, amax_out


def _packed_args(projection, bias):
    if projection.dim() != 2 or projection.stride(1) != 1:
        raise ValueError("projection must be a [m, 2f] view with unit column stride")
    m, two_f = projection.shape
    f = two_f // 2
    if bias is not None and (bias.numel() != two_f or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous tensor of 2f = %d values" % two_f)
    pp = _bf16_ptr(projection, "projection")
    bp = _bf16_ptr(bias, "bias") if bias is not None else 0
    return m, f, pp, bp, projection.stride(0)


def swiglu_packed_nvfp4(projection: torch.Tensor, global_amax: float, bias: torch.Tensor | None = None,
                        interleaved: bool = False, codes=None, scales=None, y_out=None, stream=None):
    """SwiGLU -> NVFP4 of a packed [m, 2f] projection, with an optional bias of 2f values
    (in the projection's column order) added as bf16 before SiLU.  interleaved=False:
    value columns first, then gate columns; True: value of column j at 2j, gate at 2j+1.
    The projection may be a row-strided view (unit column stride)."""
    m, f, pp, bp, ld = _packed_args(projection, bias)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, f, projection.device)
    _check(_lib.swiglu_packed_nvfp4(pp, bp, int(bool(interleaved)), ld, m, f, float(global_amax),
                                    _out_ptr(codes, torch.uint8, (m, f // 2), "codes"),
                                    _out_ptr(scales, torch.uint8, (padded_rows(m), f // 16), "scales"),
                                    _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, f), "y_out")
                                    if y_out is not None else 0,
                                    _stream(stream, projection.device)))
    return codes, scales


def swiglu_packed_nvfp4_dynamic(projection: torch.Tensor, bias: torch.Tensor | None = None,
                                interleaved: bool = False, amax_out=None, codes=None, scales=None, y_out=None,
                                stream=None):
    """swiglu_packed_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    m, f, pp, bp, ld = _packed_args(projection, bias)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, f, projection.device)
    amax_out, ap = _amax_ptr(amax_out, projection.device)
    _check(_lib.swiglu_packed_nvfp4_dynamic(pp, bp, int(bool(interleaved)), ld, m, f, ap,
                                            _out_ptr(codes, torch.uint8, (m, f // 2), "codes"),
                                            _out_ptr(scales, torch.uint8, (padded_rows(m), f // 16), "scales"),
                                            _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, f),
                                                     "y_out") if y_out is not None else 0,
                                            _stream(stream, projection.device)))
    return codes, scales, amax_out


def _f32_ptr(t, n, name):
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or t.numel() != n:
        raise ValueError("%s must be a contiguous float32 device tensor of %d values" % (name, n))
    return t.data_ptr()


def _residual_args(h, gamma, residual):
    if h.dim() != 2 or h.dtype != torch.float32 or not h.is_cuda or not h.is_contiguous():
        raise ValueError("h must be a contiguous float32 [m, k] device tensor")
    m, k = h.shape
    gp = _f32_ptr(gamma, k, "gamma")
    op = bp = sp = 0
    if residual is not None:
        o, bias, scale = residual
        if tuple(o.shape) != (m, k) or not o.is_contiguous():
            raise ValueError("o must be a contiguous [m, k] tensor")
        op = _bf16_ptr(o, "o")
        if bias is not None:
            if bias.numel() != k or not bias.is_contiguous():
                raise ValueError("bias must be a contiguous tensor of k values")
            bp = _bf16_ptr(bias, "bias")
        sp = _f32_ptr(scale, k, "scale")
    return m, k, gp, op, bp, sp


def residual_rms_nvfp4(h: torch.Tensor, gamma: torch.Tensor, eps: float, global_amax: float, residual=None,
                       codes=None, scales=None, rstd_out=None, y_out=None, stream=None):
    """In place h += bf16(o + bias) * scale (residual = (o, bias or None, scale), or None for
    no residual add), then NVFP4 of bf16(rms_norm(h, gamma, eps)) with the fp32 weight gamma.
    h: contiguous float32 [m, k]."""
    m, k, gp, op, bp, sp = _residual_args(h, gamma, residual)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, h.device)
    _check(_lib.residual_rms_nvfp4(h.data_ptr(), op, bp, sp, gp, float(eps), m, k, float(global_amax),
                                   _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                                   _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                                   _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
                                   _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k), "y_out")
                                   if y_out is not None else 0,
                                   _stream(stream, h.device)))
    return codes, scales


def residual_rms_nvfp4_dynamic(h: torch.Tensor, gamma: torch.Tensor, eps: float, residual=None, amax_out=None,
                               codes=None, scales=None, rstd_out=None, y_out=None, stream=None):
    """residual_rms_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    m, k, gp, op, bp, sp = _residual_args(h, gamma, residual)
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, h.device)
    amax_out, ap = _amax_ptr(amax_out, h.device)
    _check(_lib.residual_rms_nvfp4_dynamic(h.data_ptr(), op, bp, sp, gp, float(eps), m, k, ap,
                                           _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                                           _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                                           _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
                                           _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k),
                                                    "y_out") if y_out is not None else 0,
                                           _stream(stream, h.device)))
    return codes, scales, amax_out


def _fold_args(h, weight, table, frame_idx, residual):
    if h.dim() != 2 or h.dtype != torch.float32 or not h.is_cuda or not h.is_contiguous():
        raise ValueError("h must be a contiguous float32 [m, k] device tensor")
    m, k = h.shape
    if table.dim() != 3 or table.shape[1] != 2 or table.shape[2] != k or not table.is_contiguous():
        raise ValueError("table must be a contiguous [T, 2, k] tensor of (shift, scale) rows")
    if weight.numel() != k or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous tensor of k values")
    if frame_idx.dtype != torch.int32 or frame_idx.numel() != m or not frame_idx.is_cuda:
        raise ValueError("frame_idx must be an int32 device tensor of m values")
    tp = _bf16_ptr(table, "table")
    args = dict(m=m, k=k, w=_bf16_ptr(weight, "weight"), shift=tp, scale=tp + 2 * k, frame_stride=2 * k,
                frames=table.shape[0], idx=frame_idx.data_ptr(), o=0, bias=0, gate=0, gate_stride=k)
    if residual is not None:
        o, bias, gate = residual
        if tuple(o.shape) != (m, k) or not o.is_contiguous():
            raise ValueError("o must be a contiguous [m, k] tensor")
        if gate.dim() != 2 or gate.shape[1] != k or gate.stride(1) != 1:
            raise ValueError("gate must be a [T, k] table with unit column stride")
        args["o"] = _bf16_ptr(o, "o")
        if bias is not None:
            if bias.numel() != k or not bias.is_contiguous():
                raise ValueError("bias must be a contiguous tensor of k values")
            args["bias"] = _bf16_ptr(bias, "bias")
        args["gate"] = _bf16_ptr(gate, "gate")
        args["gate_stride"] = gate.stride(0)
    return args


def residual_rms_adaln_nvfp4(h: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                             eps: float, global_amax: float, residual=None, codes=None, scales=None, rstd_out=None,
                             y_out=None, status_word=None, stream=None):
    """In place h += bf16(o + bias) * gate[frame_idx[r]] (residual = (o, bias or None, gate table [T, k]), the
    folding block's gates), then RMSNorm + adaLN with the next block's (shift, scale) table [T, 2, k] -> NVFP4.
    h: contiguous float32 [m, k]."""
    a = _fold_args(h, weight, table, frame_idx, residual)
    m, k = a["m"], a["k"]
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, h.device)
    _check(_lib.residual_rms_adaln_nvfp4(h.data_ptr(), a["o"], a["bias"], a["gate"], a["gate_stride"], a["w"],
                                         a["shift"], a["scale"], a["frame_stride"], a["frames"], a["idx"],
                                         float(eps), m, k, float(global_amax),
                                         _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                                         _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                                         _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
                                         _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k), "y_out")
                                         if y_out is not None else 0,
                                         status_word.data_ptr() if status_word is not None else 0,
                                         _stream(stream, h.device)))
    return codes, scales


def residual_rms_adaln_nvfp4_dynamic(h: torch.Tensor, weight: torch.Tensor, table: torch.Tensor,
                                     frame_idx: torch.Tensor, eps: float, residual=None, amax_out=None, codes=None,
                                     scales=None, rstd_out=None, y_out=None, status_word=None, stream=None):
    """residual_rms_adaln_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    a = _fold_args(h, weight, table, frame_idx, residual)
    m, k = a["m"], a["k"]
    if codes is None or scales is None:
        codes, scales = new_quantized(m, k, h.device)
    amax_out, ap = _amax_ptr(amax_out, h.device)
    _check(_lib.residual_rms_adaln_nvfp4_dynamic(h.data_ptr(), a["o"], a["bias"], a["gate"], a["gate_stride"],
                                                 a["w"], a["shift"], a["scale"], a["frame_stride"], a["frames"],
                                                 a["idx"], float(eps), m, k, ap,
                                                 _out_ptr(codes, torch.uint8, (m, k // 2), "codes"),
                                                 _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales"),
                                                 _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
                                                 _out_ptr(y_out, y_out.dtype if y_out is not None else None, (m, k),
                                                          "y_out") if y_out is not None else 0,
                                                 status_word.data_ptr() if status_word is not None else 0,
                                                 _stream(stream, h.device)))
    return codes, scales, amax_out


def _f16_ptr(t, name):
    if t.dtype not in (torch.float16, torch.int16, torch.uint16):
        raise TypeError("%s must hold fp16 values (float16 or a 16-bit integer view)" % name)
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    return t.data_ptr()


def _rms_silu_args(x, gamma):
    if x.dim() < 2:
        raise ValueError("x must be channels-last with at least two dimensions")
    c = x.shape[-1]
    rows = x.numel() // c if c else 0
    if gamma.numel() != c:
        raise ValueError("gamma must hold c values")
    return rows, c, _f16_ptr(x, "x"), _f16_ptr(gamma, "gamma")


def rms_silu_nvfp4(x: torch.Tensor, gamma: torch.Tensor, eps: float, global_amax: float, codes=None, scales=None,
                   rstd_out=None, y_out=None, stream=None):
    """Channels-last fp16 x [..., c] (rows = every leading index): RMSNorm over c (fp32
    statistic, fp16 affine gamma [c]) + SiLU -> NVFP4.  Returns (codes [rows, c/2], scales
    [rows, c/16]) with the scale bytes in plain row order."""
    rows, c, xp, gp = _rms_silu_args(x, gamma)
    if codes is None:
        codes = torch.empty((rows, c // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, c // 16), dtype=torch.uint8, device=x.device)
    _check(_lib.rms_silu_nvfp4(xp, gp, float(eps), rows, c, float(global_amax),
                               _out_ptr(codes, torch.uint8, (rows, c // 2), "codes"),
                               _out_ptr(scales, torch.uint8, (rows, c // 16), "scales"),
                               _out_ptr(rstd_out, torch.float32, (rows,), "rstd_out"),
                               _out_ptr(y_out, y_out.dtype if y_out is not None else None, (rows, c), "y_out")
                               if y_out is not None else 0,
                               _stream(stream, x.device)))
    return codes, scales


def rms_silu_nvfp4_dynamic(x: torch.Tensor, gamma: torch.Tensor, eps: float, amax_out=None, codes=None,
                           scales=None, rstd_out=None, y_out=None, stream=None):
    """rms_silu_nvfp4 under the amax of this call's own y.  Returns (codes, scales, amax_out)."""
    rows, c, xp, gp = _rms_silu_args(x, gamma)
    if codes is None:
        codes = torch.empty((rows, c // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, c // 16), dtype=torch.uint8, device=x.device)
    amax_out, ap = _amax_ptr(amax_out, x.device)
    _check(_lib.rms_silu_nvfp4_dynamic(xp, gp, float(eps), rows, c, ap,
                                       _out_ptr(codes, torch.uint8, (rows, c // 2), "codes"),
                                       _out_ptr(scales, torch.uint8, (rows, c // 16), "scales"),
                                       _out_ptr(rstd_out, torch.float32, (rows,), "rstd_out"),
                                       _out_ptr(y_out, y_out.dtype if y_out is not None else None, (rows, c),
                                                "y_out") if y_out is not None else 0,
                                       _stream(stream, x.device)))
    return codes, scales, amax_out


def _ln_args(x, scale, shift):
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    for t, name in ((scale, "scale"), (shift, "shift")):
        if t.dtype != torch.float32 or t.numel() != k or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous float32 device tensor of k values" % name)
    return m, k, _f16_ptr(x, "x")


def _ln_outs(m, k, device, codes, mean_out, rstd_out, y_out):
    if codes is None:
        codes = torch.empty((m, k), dtype=torch.uint8, device=device)
    return codes, (_out_ptr(codes, torch.uint8, (m, k), "codes"), _out_ptr(mean_out, torch.float32, (m,), "mean_out"),
                   _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"),
                   _out_ptr(y_out, torch.float32, (m, k), "y_out"))


def ln_adaln_fp8(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float, act_scale: float,
                 codes=None, mean_out=None, rstd_out=None, y_out=None, stream=None):
    """fp16 x [m, k]: LayerNorm with fp32 statistics, adaLN (fp32 scale and shift [k]), then
    per-tensor FP8 E4M3 codes of y / act_scale.  Returns codes [m, k] uint8."""
    m, k, xp = _ln_args(x, scale, shift)
    codes, outs = _ln_outs(m, k, x.device, codes, mean_out, rstd_out, y_out)
    _check(_lib.ln_adaln_fp8(xp, scale.data_ptr(), shift.data_ptr(), float(eps), m, k, float(act_scale), *outs,
                             _stream(stream, x.device)))
    return codes


def ln_adaln_fp8_dynamic(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float,
                         act_scale_out=None, codes=None, mean_out=None, rstd_out=None, y_out=None, stream=None):
    """ln_adaln_fp8 under this call's own scale max|y| / 448, computed on the device.
    Returns (codes, act_scale_out) with act_scale_out a one-element float32 device tensor."""
    m, k, xp = _ln_args(x, scale, shift)
    codes, outs = _ln_outs(m, k, x.device, codes, mean_out, rstd_out, y_out)
    act_scale_out, ap = _amax_ptr(act_scale_out, x.device)
    _check(_lib.ln_adaln_fp8_dynamic(xp, scale.data_ptr(), shift.data_ptr(), float(eps), m, k, ap, *outs,
                                     _stream(stream, x.device)))
    return codes, act_scale_out
