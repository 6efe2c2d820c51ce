"""Producer-fused NVFP4 activation quantization for MI355X (gfx950).

Thin ctypes binding over ``libnvfp4act.so`` (C ABI in ``include/nvfp4act.h``).
This module only turns torch tensors into pointers and sizes, calls the entry
point of the same name on the current torch stream, and raises on a nonzero
status: every step of the computation runs in the library's HIP kernels.
If the library is missing, or was built from other sources than the ones next
to it, the import fails loudly; there is no fallback.

Entry points (see ``include/nvfp4act.h`` for the exact contract):
  nvfp4_quantize(x, global_amax)                          standalone quantize
  rms_adaln_nvfp4(x, weight, table, frame_idx, eps, global_amax)
  swiglu_nvfp4(projection, global_amax)                   value-first [m, 2f]
  swiglu_packed_nvfp4(projection, global_amax, bias, interleaved)
                                                          bias before SiLU; value-first
                                                          or paired columns
  residual_rms_nvfp4(h, gamma, eps, global_amax, residual=(o, bias, scale))
                                                          fp32 residual stream (in place) +
                                                          RMSNorm with an fp32 weight
  residual_rms_adaln_nvfp4(h, weight, table, frame_idx, eps, global_amax,
                           residual=(o, bias, gate_table))
                                                          gated residual (own table) + RMSNorm
                                                          + adaLN (next block's table)
  rms_silu_nvfp4(x, gamma, eps, global_amax)              fp16 channels-last [rows, c]:
                                                          RMSNorm + SiLU, plain scale layout
  ln_adaln_fp8(x, scale, shift, eps, act_scale)           fp16 [m, k]: LayerNorm (fp32 statistics)
                                                          + adaLN -> per-tensor FP8 E4M3 codes [m, k]
each returning ``(codes, scales)`` (ln_adaln_fp8: codes); the per-call (dynamic) amax
forms ``<name>_dynamic(...)`` take ``amax_out`` instead of the static amax and return
``(codes, scales, amax)`` with ``amax`` a one-element float32 device tensor
(ln_adaln_fp8_dynamic: ``(codes, act_scale)``); and
  rms_adaln_nvfp4_dynamic_noalloc(x, weight, table, frame_idx, eps)
                                                          the per-call form whose amax word lives
                                                          in the library's device scratch
codes are ``[m, k/2]`` uint8 and scales ``[pad(m), k/16]`` uint8 in the 128x4 swizzle
(buffer shapes as the FastVideo API page's ``new_quantized``).
"""
from __future__ import annotations

import ctypes
import glob
import hashlib
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4act.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libnvfp4act.so is not built (run python nvfp4_activation_quantization_amd/build.py "
                      "or __graft_entry__.build())")


def source_digest() -> str:
    """sha256 over the library's sources (csrc/* and include/nvfp4act.h, in name order): the
    value the build compiles into the library."""
    h = hashlib.sha256()
    root = os.path.dirname(_PKG)
    paths = sorted(glob.glob(os.path.join(_PKG, "csrc", "*"))) + [os.path.join(root, "include", "nvfp4act.h")]
    for path in paths:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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
    "nvfp4act_source_digest": (ctypes.c_char_p, []),
    "nvfp4_quantize": (_I, [_P, _I64, _I64, _F, _P, _P, _P]),
    "rms_adaln_nvfp4": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _F, _P, _P, _P, _P, _P, _P]),
    "swiglu_nvfp4": (_I, [_P, _P, _I64, _I64, _I64, _F, _P, _P, _P, _P]),
    "nvfp4_quantize_dynamic": (_I, [_P, _I64, _I64, _P, _P, _P, _P]),
    "rms_adaln_nvfp4_dynamic": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "rms_adaln_nvfp4_dynamic_noalloc": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _F, _I64, _I64, _P, _P, _P, _P, _P,
                                            _P]),
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

if os.path.isdir(os.path.join(_PKG, "csrc")) and _lib.nvfp4act_source_digest().decode() != source_digest():
    raise ImportError("libnvfp4act.so was built from other sources than those in %s/csrc: rebuild it "
                      "(python nvfp4_activation_quantization_amd/build.py)" % _PKG)

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
    """Probe the current device (optional: every entry point does it on first use)."""
    _check(_lib.nvfp4act_init())


def new_quantized(m: int, k: int, device) -> tuple[torch.Tensor, torch.Tensor]:
    """Output buffers for an [m, k] activation: codes [m, k/2], scales [pad(m), k/16]."""
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((padded_rows(m), k // 16), dtype=torch.uint8, device=device)
    return codes, scales


# ---- argument marshalling ------------------------------------------------------------------

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)    # bf16 values or their 16-bit patterns
_F16 = (torch.float16, torch.int16, torch.uint16)      # fp16 values or their 16-bit patterns


def _in_ptr(t: torch.Tensor, dtypes, name: str, numel=None, contiguous=True) -> int:
    if t.dtype not in dtypes:
        raise TypeError("%s must have one of the dtypes %s" % (name, ", ".join(str(d) for d in dtypes)))
    if not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d values" % (name, numel))
    return t.data_ptr()


def _bf16_ptr(t: torch.Tensor, name: str, numel=None) -> int:
    return _in_ptr(t, _BF16, name, numel)


def _f16_ptr(t: torch.Tensor, name: str, numel=None) -> int:
    return _in_ptr(t, _F16, name, numel)


def _f32_ptr(t: torch.Tensor, name: str, numel=None) -> int:
    return _in_ptr(t, (torch.float32,), name, numel)


def _out_ptr(t, dtypes, shape, name) -> int:
    """Pointer of an optional output (0 when None); its dtype must be one the kernel writes."""
    if t is None:
        return 0
    if isinstance(dtypes, torch.dtype):
        dtypes = (dtypes,)
    if t.dtype not in dtypes or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("%s must be a contiguous device tensor of shape %s and dtype %s"
                         % (name, tuple(shape), " or ".join(str(d) for d in dtypes)))
    return t.data_ptr()


def _status_ptr(status_word) -> int:
    if status_word is None:
        return 0
    if status_word.dtype not in (torch.int32, torch.uint32) or not status_word.is_cuda or status_word.numel() < 1:
        raise ValueError("status_word must be a 32-bit device tensor with at least one element")
    return status_word.data_ptr()


def _idx_ptr(frame_idx: torch.Tensor, m: int) -> int:
    if frame_idx.dtype != torch.int32 or frame_idx.numel() != m:
        raise ValueError("frame_idx must be an int32 tensor of m = %d values" % m)
    return _in_ptr(frame_idx, (torch.int32,), "frame_idx")


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _quant_outs(m, k, device, codes, scales):
    """(codes, scales, their pointers) for an [m, k] activation, allocated when not given."""
    if codes is None or scales is None:
        c, s = new_quantized(m, k, device)
        codes = c if codes is None else codes
        scales = s if scales is None else scales
    return codes, scales, _out_ptr(codes, torch.uint8, (m, k // 2), "codes"), \
        _out_ptr(scales, torch.uint8, (padded_rows(m), k // 16), "scales")


def _amax_ptr(amax_out, device):
    if amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=device)
    if amax_out.dtype != torch.float32 or amax_out.numel() < 1 or not amax_out.is_cuda:
        raise ValueError("amax_out must be a float32 device tensor with at least one element")
    return amax_out, amax_out.data_ptr()


def _call(static_fn, dynamic_fn, args_before, args_after, global_amax, amax_out, device, dynamic):
    """Call the static form with the float global_amax, or the per-call form with a device
    amax pointer; returns the amax tensor of the per-call form (None otherwise)."""
    if dynamic:
        amax_out, ap = _amax_ptr(amax_out, device)
        _check(dynamic_fn(*args_before, ap, *args_after))
        return amax_out
    _check(static_fn(*args_before, float(global_amax), *args_after))
    return None


# ---- standalone quantize ---------------------------------------------------------------------

def _quantize(x, global_amax, amax_out, dynamic, codes, scales, stream):
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    xp = _bf16_ptr(x, "x")
    codes, scales, cp, sp = _quant_outs(m, k, x.device, codes, scales)
    amax = _call(_lib.nvfp4_quantize, _lib.nvfp4_quantize_dynamic, (xp, m, k), (cp, sp, _stream(stream, x.device)),
                 global_amax, amax_out, x.device, dynamic)
    return (codes, scales, amax) if dynamic else (codes, scales)


def nvfp4_quantize(x: torch.Tensor, global_amax: float, codes=None, scales=None, stream=None):
    """Standalone NVFP4 quantize of a contiguous bf16 [m, k] tensor."""
    return _quantize(x, global_amax, None, False, codes, scales, stream)


def nvfp4_quantize_dynamic(x: torch.Tensor, amax_out=None, codes=None, scales=None, stream=None):
    """Standalone NVFP4 quantize under the tensor's own amax (computed on the device)."""
    return _quantize(x, 0.0, amax_out, True, codes, scales, stream)


# ---- RMSNorm + adaLN -------------------------------------------------------------------------

def _rms_adaln_args(x, weight, table, frame_idx, eps, codes, scales, rstd_out, y_out, status_word, stream):
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    if table.dim() != 3 or table.shape[1] != 2 or table.shape[2] != k:
        raise ValueError("table must be [T, 2, k] (shift, scale) rows")
    xp = _bf16_ptr(x, "x")
    wp = _bf16_ptr(weight, "weight", k)
    tp = _bf16_ptr(table, "table")
    ip = _idx_ptr(frame_idx, m)
    codes, scales, cp, sp = _quant_outs(m, k, x.device, codes, scales)
    before = (xp, wp, tp, tp + 2 * k, 2 * k, table.shape[0], ip, float(eps), m, k)
    after = (cp, sp, _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"), _out_ptr(y_out, _BF16, (m, k), "y_out"),
             _status_ptr(status_word), _stream(stream, x.device))
    return codes, scales, before, after


def rms_adaln_nvfp4(x: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                    eps: float, global_amax: float, codes=None, scales=None, rstd_out=None, y_out=None,
                    status_word=None, stream=None):
    """Fused RMSNorm + adaLN -> NVFP4.

    x [m, k] bf16; weight [k] bf16; table [T, 2, k] bf16 holding (shift, scale) per
    frame; frame_idx [m] int32 (device).  Optional outputs: rstd_out [m] fp32, y_out
    [m, k] bf16 (or a 16-bit integer view), status_word (bit 0: a frame index was out of
    range).
    """
    codes, scales, before, after = _rms_adaln_args(x, weight, table, frame_idx, eps, codes, scales, rstd_out, y_out,
                                                   status_word, stream)
    _call(_lib.rms_adaln_nvfp4, None, before, after, global_amax, None, x.device, False)
    return codes, scales


def rms_adaln_nvfp4_dynamic(x: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                            eps: float, amax_out=None, codes=None, scales=None, rstd_out=None, y_out=None,
                            status_word=None, stream=None):
    """Fused RMSNorm + adaLN -> NVFP4 under the amax of this call's own y (computed on the
    device by an amax pass).  Arguments as rms_adaln_nvfp4 without global_amax."""
    codes, scales, before, after = _rms_adaln_args(x, weight, table, frame_idx, eps, codes, scales, rstd_out, y_out,
                                                   status_word, stream)
    amax = _call(None, _lib.rms_adaln_nvfp4_dynamic, before, after, 0.0, amax_out, x.device, True)
    return codes, scales, amax


def rms_adaln_nvfp4_dynamic_noalloc(x: torch.Tensor, weight: torch.Tensor, table: torch.Tensor,
                                    frame_idx: torch.Tensor, eps: float, codes=None, scales=None, rstd_out=None,
                                    y_out=None, status_word=None, stream=None):
    """rms_adaln_nvfp4_dynamic whose amax word is the library's device scratch (the entry
    point allocates nothing; pass codes and scales to allocate nothing here either).
    Calls that overlap on one device race on that word."""
    codes, scales, before, after = _rms_adaln_args(x, weight, table, frame_idx, eps, codes, scales, rstd_out, y_out,
                                                   status_word, stream)
    _check(_lib.rms_adaln_nvfp4_dynamic_noalloc(*before, *after))
    return codes, scales


# ---- SwiGLU ----------------------------------------------------------------------------------

def _swiglu_args(projection, gate, codes, scales, y_out, stream):
    if gate is None:
        if projection.dim() != 2:
            raise ValueError("projection must be [m, 2f]")
        m, two_f = projection.shape
        f = two_f // 2
        up_ptr = _bf16_ptr(projection, "projection")
        gate_ptr = up_ptr + 2 * f
        ld = two_f
    else:
        m, f = projection.shape
        if gate.shape != projection.shape or projection.stride(1) != 1 or gate.stride(1) != 1 \
                or projection.stride(0) != gate.stride(0):
            raise ValueError("up and gate must be [m, f] views with unit column stride and equal row stride")
        up_ptr = _in_ptr(projection, _BF16, "up", contiguous=False)
        gate_ptr = _in_ptr(gate, _BF16, "gate", contiguous=False)
        ld = projection.stride(0)
    codes, scales, cp, sp = _quant_outs(m, f, projection.device, codes, scales)
    before = (up_ptr, gate_ptr, ld, m, f)
    after = (cp, sp, _out_ptr(y_out, _BF16, (m, f), "y_out"), _stream(stream, projection.device))
    return codes, scales, before, after


def swiglu_nvfp4(projection: torch.Tensor, global_amax: float, codes=None, scales=None, y_out=None,
                 gate: torch.Tensor | None = None, stream=None):
    """SwiGLU -> NVFP4.

    With gate=None, projection is a value-first [m, 2f] tensor (up = first f columns,
    gate = last f).  Otherwise projection is up [m, f] and gate [m, f], two views with
    the same row stride (unit column stride).
    """
    codes, scales, before, after = _swiglu_args(projection, gate, codes, scales, y_out, stream)
    _call(_lib.swiglu_nvfp4, None, before, after, global_amax, None, projection.device, False)
    return codes, scales


def swiglu_nvfp4_dynamic(projection: torch.Tensor, amax_out=None, codes=None, scales=None, y_out=None,
                         gate: torch.Tensor | None = None, stream=None):
    """SwiGLU -> NVFP4 under the amax of this call's own y (computed on the device).
    Arguments as swiglu_nvfp4 without global_amax."""
    codes, scales, before, after = _swiglu_args(projection, gate, codes, scales, y_out, stream)
    amax = _call(None, _lib.swiglu_nvfp4_dynamic, before, after, 0.0, amax_out, projection.device, True)
    return codes, scales, amax


def _packed_args(projection, bias, interleaved, codes, scales, y_out, stream):
    if projection.dim() != 2 or projection.stride(1) != 1:
        raise ValueError("projection must be a [m, 2f] view with unit column stride")
    m, two_f = projection.shape
    f = two_f // 2
    pp = _in_ptr(projection, _BF16, "projection", contiguous=False)
    bp = _bf16_ptr(bias, "bias", two_f) if bias is not None else 0
    codes, scales, cp, sp = _quant_outs(m, f, projection.device, codes, scales)
    before = (pp, bp, int(bool(interleaved)), projection.stride(0), m, f)
    after = (cp, sp, _out_ptr(y_out, _BF16, (m, f), "y_out"), _stream(stream, projection.device))
    return codes, scales, before, after


def swiglu_packed_nvfp4(projection: torch.Tensor, global_amax: float, bias: torch.Tensor | None = None,
                        interleaved: bool = False, codes=None, scales=None, y_out=None, stream=None):
    """SwiGLU -> NVFP4 of a packed [m, 2f] projection, with an optional bias of 2f values
    (in the projection's column order) added as bf16 before SiLU.  interleaved=False:
    value columns first, then gate columns; True: value of column j at 2j, gate at 2j+1.
    The projection may be a row-strided view (unit column stride)."""
    codes, scales, before, after = _packed_args(projection, bias, interleaved, codes, scales, y_out, stream)
    _call(_lib.swiglu_packed_nvfp4, None, before, after, global_amax, None, projection.device, False)
    return codes, scales


def swiglu_packed_nvfp4_dynamic(projection: torch.Tensor, bias: torch.Tensor | None = None,
                                interleaved: bool = False, amax_out=None, codes=None, scales=None, y_out=None,
                                stream=None):
    """swiglu_packed_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    codes, scales, before, after = _packed_args(projection, bias, interleaved, codes, scales, y_out, stream)
    amax = _call(None, _lib.swiglu_packed_nvfp4_dynamic, before, after, 0.0, amax_out, projection.device, True)
    return codes, scales, amax


# ---- residual stream + RMSNorm -----------------------------------------------------------------

def _h_shape(h):
    if h.dim() != 2 or h.dtype != torch.float32 or not h.is_cuda or not h.is_contiguous():
        raise ValueError("h must be a contiguous float32 [m, k] device tensor")
    return h.shape


def _branch(o, bias, m, k):
    if tuple(o.shape) != (m, k):
        raise ValueError("o must be a contiguous [m, k] tensor")
    op = _bf16_ptr(o, "o")
    bp = _bf16_ptr(bias, "bias", k) if bias is not None else 0
    return op, bp


def _residual_args(h, gamma, eps, residual, codes, scales, rstd_out, y_out, stream):
    m, k = _h_shape(h)
    gp = _f32_ptr(gamma, "gamma", k)
    op = bp = sp = 0
    if residual is not None:
        o, bias, scale = residual
        op, bp = _branch(o, bias, m, k)
        sp = _f32_ptr(scale, "scale", k)
    codes, scales, cp, sc = _quant_outs(m, k, h.device, codes, scales)
    before = (h.data_ptr(), op, bp, sp, gp, float(eps), m, k)
    after = (cp, sc, _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"), _out_ptr(y_out, _BF16, (m, k), "y_out"),
             _stream(stream, h.device))
    return codes, scales, before, after


def residual_rms_nvfp4(h: torch.Tensor, gamma: torch.Tensor, eps: float, global_amax: float, residual=None,
                       codes=None, scales=None, rstd_out=None, y_out=None, stream=None):
    """In place h += bf16(o + bias) * scale (residual = (o, bias or None, scale), or None for
    no residual add), then NVFP4 of bf16(rms_norm(h, gamma, eps)) with the fp32 weight gamma.
    h: contiguous float32 [m, k]."""
    codes, scales, before, after = _residual_args(h, gamma, eps, residual, codes, scales, rstd_out, y_out, stream)
    _call(_lib.residual_rms_nvfp4, None, before, after, global_amax, None, h.device, False)
    return codes, scales


def residual_rms_nvfp4_dynamic(h: torch.Tensor, gamma: torch.Tensor, eps: float, residual=None, amax_out=None,
                               codes=None, scales=None, rstd_out=None, y_out=None, stream=None):
    """residual_rms_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    codes, scales, before, after = _residual_args(h, gamma, eps, residual, codes, scales, rstd_out, y_out, stream)
    amax = _call(None, _lib.residual_rms_nvfp4_dynamic, before, after, 0.0, amax_out, h.device, True)
    return codes, scales, amax


def _fold_args(h, weight, table, frame_idx, eps, residual, codes, scales, rstd_out, y_out, status_word, stream):
    m, k = _h_shape(h)
    if table.dim() != 3 or table.shape[1] != 2 or table.shape[2] != k:
        raise ValueError("table must be a contiguous [T, 2, k] tensor of (shift, scale) rows")
    tp = _bf16_ptr(table, "table")
    wp = _bf16_ptr(weight, "weight", k)
    ip = _idx_ptr(frame_idx, m)
    op = bp = gp = 0
    gate_stride = k
    if residual is not None:
        o, bias, gate = residual
        op, bp = _branch(o, bias, m, k)
        if gate.dim() != 2 or gate.shape[1] != k or gate.stride(1) != 1:
            raise ValueError("gate must be a [T, k] table with unit column stride")
        gp = _in_ptr(gate, _BF16, "gate", contiguous=False)
        gate_stride = gate.stride(0)
    codes, scales, cp, sc = _quant_outs(m, k, h.device, codes, scales)
    before = (h.data_ptr(), op, bp, gp, gate_stride, wp, tp, tp + 2 * k, 2 * k, table.shape[0], ip, float(eps), m, k)
    after = (cp, sc, _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"), _out_ptr(y_out, _BF16, (m, k), "y_out"),
             _status_ptr(status_word), _stream(stream, h.device))
    return codes, scales, before, after


def residual_rms_adaln_nvfp4(h: torch.Tensor, weight: torch.Tensor, table: torch.Tensor, frame_idx: torch.Tensor,
                             eps: float, global_amax: float, residual=None, codes=None, scales=None, rstd_out=None,
                             y_out=None, status_word=None, stream=None):
    """In place h += bf16(o + bias) * gate[frame_idx[r]] (residual = (o, bias or None, gate table [T, k]), the
    folding block's gates), then RMSNorm + adaLN with the next block's (shift, scale) table [T, 2, k] -> NVFP4.
    h: contiguous float32 [m, k]."""
    codes, scales, before, after = _fold_args(h, weight, table, frame_idx, eps, residual, codes, scales, rstd_out,
                                              y_out, status_word, stream)
    _call(_lib.residual_rms_adaln_nvfp4, None, before, after, global_amax, None, h.device, False)
    return codes, scales


def residual_rms_adaln_nvfp4_dynamic(h: torch.Tensor, weight: torch.Tensor, table: torch.Tensor,
                                     frame_idx: torch.Tensor, eps: float, residual=None, amax_out=None, codes=None,
                                     scales=None, rstd_out=None, y_out=None, status_word=None, stream=None):
    """residual_rms_adaln_nvfp4 under the amax of this call's own y (computed on the device).
    Returns (codes, scales, amax_out)."""
    codes, scales, before, after = _fold_args(h, weight, table, frame_idx, eps, residual, codes, scales, rstd_out,
                                              y_out, status_word, stream)
    amax = _call(None, _lib.residual_rms_adaln_nvfp4_dynamic, before, after, 0.0, amax_out, h.device, True)
    return codes, scales, amax


# ---- channels-last RMSNorm + SiLU (fp16) --------------------------------------------------------

def _rms_silu_args(x, gamma, eps, codes, scales, rstd_out, y_out, stream):
    if x.dim() < 2:
        raise ValueError("x must be channels-last with at least two dimensions")
    c = x.shape[-1]
    rows = x.numel() // c if c else 0
    xp = _f16_ptr(x, "x")
    gp = _f16_ptr(gamma, "gamma", c)
    if codes is None:
        codes = torch.empty((rows, c // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, c // 16), dtype=torch.uint8, device=x.device)
    before = (xp, gp, float(eps), rows, c)
    after = (_out_ptr(codes, torch.uint8, (rows, c // 2), "codes"), _out_ptr(scales, torch.uint8, (rows, c // 16),
                                                                              "scales"),
             _out_ptr(rstd_out, torch.float32, (rows,), "rstd_out"), _out_ptr(y_out, _F16, (rows, c), "y_out"),
             _stream(stream, x.device))
    return codes, scales, before, after


def rms_silu_nvfp4(x: torch.Tensor, gamma: torch.Tensor, eps: float, global_amax: float, codes=None, scales=None,
                   rstd_out=None, y_out=None, stream=None):
    """Channels-last fp16 x [..., c] (rows = every leading index): RMSNorm over c (fp32
    statistic, fp16 affine gamma [c]) + SiLU -> NVFP4.  Returns (codes [rows, c/2], scales
    [rows, c/16]) with the scale bytes in plain row order."""
    codes, scales, before, after = _rms_silu_args(x, gamma, eps, codes, scales, rstd_out, y_out, stream)
    _call(_lib.rms_silu_nvfp4, None, before, after, global_amax, None, x.device, False)
    return codes, scales


def rms_silu_nvfp4_dynamic(x: torch.Tensor, gamma: torch.Tensor, eps: float, amax_out=None, codes=None,
                           scales=None, rstd_out=None, y_out=None, stream=None):
    """rms_silu_nvfp4 under the amax of this call's own y.  Returns (codes, scales, amax_out)."""
    codes, scales, before, after = _rms_silu_args(x, gamma, eps, codes, scales, rstd_out, y_out, stream)
    amax = _call(None, _lib.rms_silu_nvfp4_dynamic, before, after, 0.0, amax_out, x.device, True)
    return codes, scales, amax


# ---- LayerNorm + adaLN -> FP8 -------------------------------------------------------------------

def _ln_args(x, scale, shift, eps, codes, mean_out, rstd_out, y_out, stream):
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    xp = _f16_ptr(x, "x")
    scp = _f32_ptr(scale, "scale", k)
    shp = _f32_ptr(shift, "shift", k)
    if codes is None:
        codes = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    before = (xp, scp, shp, float(eps), m, k)
    after = (_out_ptr(codes, torch.uint8, (m, k), "codes"), _out_ptr(mean_out, torch.float32, (m,), "mean_out"),
             _out_ptr(rstd_out, torch.float32, (m,), "rstd_out"), _out_ptr(y_out, torch.float32, (m, k), "y_out"),
             _stream(stream, x.device))
    return codes, before, after


def ln_adaln_fp8(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float, act_scale: float,
                 codes=None, mean_out=None, rstd_out=None, y_out=None, stream=None):
    """fp16 x [m, k]: LayerNorm with fp32 statistics, adaLN (fp32 scale and shift [k]), then
    per-tensor FP8 E4M3 codes of y / act_scale.  Returns codes [m, k] uint8."""
    codes, before, after = _ln_args(x, scale, shift, eps, codes, mean_out, rstd_out, y_out, stream)
    _call(_lib.ln_adaln_fp8, None, before, after, act_scale, None, x.device, False)
    return codes


def ln_adaln_fp8_dynamic(x: torch.Tensor, scale: torch.Tensor, shift: torch.Tensor, eps: float,
                         act_scale_out=None, codes=None, mean_out=None, rstd_out=None, y_out=None, stream=None):
    """ln_adaln_fp8 under this call's own scale max|y| / 448, computed on the device.
    Returns (codes, act_scale_out) with act_scale_out a one-element float32 device tensor."""
    codes, before, after = _ln_args(x, scale, shift, eps, codes, mean_out, rstd_out, y_out, stream)
    act_scale = _call(None, _lib.ln_adaln_fp8_dynamic, before, after, 0.0, act_scale_out, x.device, True)
    return codes, act_scale
