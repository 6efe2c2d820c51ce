"""CPU oracle for producer-fused NVFP4 activation quantization.

TEST INFRASTRUCTURE ONLY.  The oracle defines, bit for bit, what the GPU
library computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does.
It shares no code, header, table or constant generator with the HIP path.

The arithmetic lives in plain C (``nvfp4_oracle.c``, single-threaded,
IEEE fp32 with FTZ/DAZ cleared).  This module compiles it with gcc, loads it
with ctypes and converts numpy arrays.  ``silu_exact`` is an independent
pure-Python derivation of the SiLU table used to pin the C one.

Every function here follows the passages cited in ``nvfp4_oracle.c``:
the FastVideo API page ``minimax_h3_nvfp4_fused`` (quantize, swiglu_quantize,
new_quantized), TensorRT-LLM PR #21483 (Summary: producer-fused quantize), the
FastVideo branch compare's ``minimax_h3_swiglu_quant.cuh`` (scale_fp8,
scale_float, fp4_pair, quant_probe) and the FastVideo commit log (int64
indexing, frame-index bounds contract).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
# NVFP4_ORACLE_LIB names another build of the same source to load instead (the test suite's
# AddressSanitizer / UndefinedBehaviorSanitizer build, see build_sanitized)
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-msse2", "-mfpmath=sse", "-fvisibility=hidden"]


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` (always, when force)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


# the sanitizers replace -O2 (they need frame pointers and keep every access)
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build_sanitized(path: str) -> str:
    """Compile the same source with AddressSanitizer and UndefinedBehaviorSanitizer into
    ``path`` (host code only: the oracle has no GPU code).  A process that loads it needs the
    ASan runtime preloaded and NVFP4_ORACLE_LIB=path."""
    flags = [f for f in GCC_FLAGS if f != "-O2"] + SANITIZE_FLAGS
    subprocess.run(["gcc", *flags, _SRC, "-o", path, "-lm"], check=True)
    return path


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        F = ctypes.c_float
        sig = {
            "orc_bf16_round": (None, [P, P, I64]),
            "orc_e4m3_encode": (None, [P, P, I64]),
            "orc_e4m3_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_e2m1_encode": (None, [P, P, I64]),
            "orc_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
            "orc_scale_offset": (I64, [I64, I64, I64]),
            "orc_padded_rows": (I64, [I64]),
            "orc_global_scale": (F, [F]),
            "orc_dynamic_global_scale": (F, [F]),
            "orc_max_abs_bf16": (F, [P, I64]),
            "orc_nvfp4_quantize_gsf": (None, [P, I64, I64, F, P, P]),
            "orc_rms_adaln_rows_gsf": (None, [P, I64, I64, P, P, P, P, I64, I64, P, F, F,
                                              P, P, P, P, P, P]),
            "orc_swiglu_rows_gsf": (None, [P, P, I64, I64, I64, P, P, F, P, P, P, P]),
            "orc_swiglu_packed_rows_gsf": (None, [P, P, ctypes.c_int, I64, I64, I64, P, P, F,
                                                  P, P, P, P]),
            "orc_rms_rstd": (F, [P, I64, F]),
            "orc_rms_sum_f32": (F, [P, I64]),
            "orc_rms_rstd_f32": (F, [P, I64, F]),
            "orc_residual_rms_rows_gsf": (None, [P, P, P, P, P, F, I64, I64, P, F, P, P, P, P, P]),
            "orc_residual_rms_adaln_rows_gsf": (None, [P, P, P, P, I64, P, P, P, I64, I64, P, F, I64, I64, P, F,
                                                       P, P, P, P, P, P]),
            "orc_quantize_rows": (None, [P, I64, I64, F, P, P]),
            "orc_nvfp4_quantize": (None, [P, I64, I64, F, P, P]),
            "orc_rms_adaln_rows": (None, [P, I64, I64, P, P, P, P, I64, I64, P, F, F,
                                          P, P, P, P, P, P]),
            "orc_silu_table": (ctypes.c_int, [P]),
            "orc_silu_table_f16": (ctypes.c_int, [P]),
            "orc_tree_sum_f32": (F, [P, I64, ctypes.c_int]),
            "orc_e4m3_encode_signed": (None, [P, P, I64]),
            "orc_ln_adaln_fp8_rows": (None, [P, P, P, F, I64, I64, F, P, P, P, P]),
            "orc_fp8_inverse_scale": (F, [F]),
            "orc_fp8_dynamic_scale": (F, [F]),
            "orc_fp8_dynamic_inverse": (F, [F]),
            "orc_f16_round": (None, [P, P, I64]),
            "orc_rms_rstd_f16row": (F, [P, I64, F]),
            "orc_rms_sum_f16row": (F, [P, I64]),
            "orc_rms_silu_rows_gsf": (None, [P, P, F, I64, I64, P, F, P, P, P, P]),
            "orc_swiglu_rows": (None, [P, P, I64, I64, I64, P, P, F, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# codecs
# --------------------------------------------------------------------------

def bf16_round(f32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN -> 0x7FC0)."""
    a = _c(f32, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_bf16_round(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f32(u16) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(f32) -> np.ndarray:
    """Non-negative fp32 -> E4M3 code, nearest, ties to even, saturating at 448."""
    a = _c(f32, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().orc_e4m3_encode(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_value(code: int) -> float:
    return _load().orc_e4m3_value(int(code))


def e2m1_encode(f32) -> np.ndarray:
    """fp32 -> E2M1 4-bit code (sign bit 3), nearest, ties to even, saturating at 6."""
    a = _c(f32, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().orc_e2m1_encode(_ptr(a), _ptr(out), a.size)
    return out


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def scale_offset(r: int, b: int, k: int) -> int:
    return _load().orc_scale_offset(int(r), int(b), int(k))


def scale_offsets(rows, k: int) -> np.ndarray:
    """Swizzled byte offsets [len(rows), k/16] of every block of the given rows
    (same layout as orc_scale_offset, vectorised)."""
    r = np.asarray(rows, np.int64)[:, None]
    b = np.arange(k // 16, dtype=np.int64)[None, :]
    return (((r // 128) * (k // 64) + b // 4) * 512 + (r % 32) * 16 + ((r // 32) % 4) * 4 + b % 4)


def padded_rows(m: int) -> int:
    return _load().orc_padded_rows(int(m))


def global_scale(global_amax: float) -> float:
    return _load().orc_global_scale(float(global_amax))


def dynamic_global_scale(amax: float) -> float:
    """Global scale of a per-call amax: 2688 / amax when positive and finite, else 0."""
    return _load().orc_dynamic_global_scale(float(amax))


def max_abs(u16) -> float:
    """max |x| over bf16 patterns, as fp32 (exact)."""
    a = _c(u16, np.uint16)
    return _load().orc_max_abs_bf16(_ptr(a), a.size)


def rms_rstd(x_row_u16, eps: float) -> float:
    a = _c(x_row_u16, np.uint16)
    return _load().orc_rms_rstd(_ptr(a), a.size, float(eps))


# --------------------------------------------------------------------------
# producers
# --------------------------------------------------------------------------

def quantize_rows(y_u16, global_amax: float):
    """Block-quantize bf16 rows: returns codes [n, k/2], plain-order scale bytes [n, k/16]."""
    y = _c(y_u16, np.uint16)
    n, k = y.shape
    codes = np.empty((n, k // 2), np.uint8)
    sb = np.empty((n, k // 16), np.uint8)
    _load().orc_quantize_rows(_ptr(y), n, k, float(global_amax), _ptr(codes), _ptr(sb))
    return codes, sb


def nvfp4_quantize(x_u16, global_amax: float, gsf: float | None = None):
    """Standalone quantize: codes [m, k/2] and swizzled scales [pad(m), k/16].

    With gsf given, that global scale is used as is (global_amax is ignored)."""
    x = _c(x_u16, np.uint16)
    m, k = x.shape
    codes = np.empty((m, k // 2), np.uint8)
    scales = np.empty((padded_rows(m), k // 16), np.uint8)
    if gsf is None:
        _load().orc_nvfp4_quantize(_ptr(x), m, k, float(global_amax), _ptr(codes), _ptr(scales))
    else:
        _load().orc_nvfp4_quantize_gsf(_ptr(x), m, k, float(gsf), _ptr(codes), _ptr(scales))
    return codes, scales


def nvfp4_quantize_dynamic(x_u16):
    """Standalone quantize under the tensor's own amax (per-call scale, the FlashRT
    dynamic activation scale): returns (codes, scales, amax)."""
    amax = max_abs(x_u16)
    codes, scales = nvfp4_quantize(x_u16, 0.0, gsf=dynamic_global_scale(amax))
    return codes, scales, amax


def rms_adaln_rows(x_u16, w_u16, table_u16, frame_idx, eps: float, global_amax: float,
                   row_ids=None, want_y: bool = False, scales_rows: int | None = None,
                   gsf: float | None = None):
    """RMSNorm + adaLN -> NVFP4 for rows of x.

    table_u16: [T, 2, k] bf16 (shift, scale).  frame_idx: per-row frame.
    row_ids: the rows' indices in the full tensor (default 0..n-1).
    gsf: use this global scale as is (global_amax is then ignored).
    Returns dict(codes [n,k/2], scale_bytes [n,k/16], rstd [n], y [n,k] or None,
    status, scales: swizzled [scales_rows, k/16] when scales_rows is given).
    """
    x = _c(x_u16, np.uint16)
    n, k = x.shape
    w = _c(w_u16, np.uint16)
    tab = _c(table_u16, np.uint16)
    t_frames = tab.shape[0]
    idx = _c(frame_idx, np.int32)
    rid = None if row_ids is None else _c(row_ids, np.int64)
    codes = np.empty((n, k // 2), np.uint8)
    sb = np.empty((n, k // 16), np.uint8)
    rstd = np.empty(n, np.float32)
    y = np.empty((n, k), np.uint16) if want_y else None
    scales = None
    if scales_rows is not None:
        scales = np.zeros((scales_rows, k // 16), np.uint8)
    status = np.zeros(1, np.uint32)
    shift_ptr = tab.ctypes.data                    # table row t: shift at t*2k elements
    scale_ptr = tab.ctypes.data + k * tab.itemsize  # ... and scale k elements further
    fn = _load().orc_rms_adaln_rows if gsf is None else _load().orc_rms_adaln_rows_gsf
    fn(_ptr(x), n, k, _ptr(rid), _ptr(w), shift_ptr, scale_ptr, 2 * k, t_frames, _ptr(idx), float(eps),
       float(global_amax if gsf is None else gsf), _ptr(codes), _ptr(sb), _ptr(scales), _ptr(rstd),
       _ptr(y), _ptr(status))
    return dict(codes=codes, scale_bytes=sb, rstd=rstd, y=y, status=int(status[0]), scales=scales)


def rms_adaln_dynamic(x_u16, w_u16, table_u16, frame_idx, eps: float, want_y: bool = False,
                      scales_rows: int | None = None):
    """RMSNorm + adaLN -> NVFP4 under the amax of the tensor's own y (two passes: y, then
    the quantizer with dynamic_global_scale(max|y|)).  The result dict gains 'amax'."""
    first = rms_adaln_rows(x_u16, w_u16, table_u16, frame_idx, eps, 1.0, want_y=True)
    amax = max_abs(first["y"])
    out = rms_adaln_rows(x_u16, w_u16, table_u16, frame_idx, eps, 0.0, want_y=want_y,
                         scales_rows=scales_rows, gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


def rms_sum_f32(h_row) -> float:
    """The fixed-tree sum of h^2 over one fp32 row (k % 256 == 0)."""
    h = _c(h_row, np.float32).reshape(-1)
    return _load().orc_rms_sum_f32(_ptr(h), h.size)


def rms_rstd_f32(h_row, eps: float) -> float:
    h = _c(h_row, np.float32).reshape(-1)
    return _load().orc_rms_rstd_f32(_ptr(h), h.size, float(eps))


def residual_rms_rows(h_f32, o_u16, bias_u16, scale_f32, gamma_f32, eps: float, global_amax: float,
                      row_ids=None, want_y: bool = False, scales_rows: int | None = None,
                      gsf: float | None = None):
    """fp32 residual stream + RMSNorm (fp32 gamma) -> NVFP4 over rows.

    h_f32 [n, k] is not modified: the updated stream is returned as 'h'.  o_u16 [n, k]
    bf16 or None (no residual add); bias_u16 [k] bf16 or None; scale_f32, gamma_f32 [k].
    gsf: use this global scale as is (global_amax is then ignored).
    Returns dict(codes, scale_bytes, y, scales, rstd, h).
    """
    h = np.array(h_f32, dtype=np.float32, copy=True, order="C")
    n, k = h.shape
    o = None if o_u16 is None else _c(o_u16, np.uint16)
    bias = None if bias_u16 is None else _c(bias_u16, np.uint16).reshape(-1)
    scale = None if scale_f32 is None else _c(scale_f32, np.float32).reshape(-1)
    gamma = _c(gamma_f32, np.float32).reshape(-1)
    if o is not None and (o.shape != (n, k) or scale is None or scale.size != k):
        raise ValueError("o must be [n, k] and scale [k] when a residual is given")
    if gamma.size != k or (bias is not None and bias.size != k):
        raise ValueError("gamma and bias hold k values")
    rid = None if row_ids is None else _c(row_ids, np.int64)
    codes = np.empty((n, k // 2), np.uint8)
    sb = np.empty((n, k // 16), np.uint8)
    rstd = np.empty(n, np.float32)
    y = np.empty((n, k), np.uint16) if want_y else None
    scales = None if scales_rows is None else np.zeros((scales_rows, k // 16), np.uint8)
    g = float(global_scale(global_amax) if gsf is None else gsf)
    _load().orc_residual_rms_rows_gsf(_ptr(h), _ptr(o), _ptr(bias), _ptr(scale), _ptr(gamma), float(eps), n, k,
                                      _ptr(rid), g, _ptr(codes), _ptr(sb), _ptr(scales), _ptr(rstd), _ptr(y))
    return dict(codes=codes, scale_bytes=sb, y=y, scales=scales, rstd=rstd, h=h)


def residual_rms_dynamic(h_f32, o_u16, bias_u16, scale_f32, gamma_f32, eps: float, want_y: bool = False,
                         scales_rows: int | None = None):
    """residual_rms_rows under the amax of the call's own y (two passes over the same
    input h).  The result dict gains 'amax'."""
    first = residual_rms_rows(h_f32, o_u16, bias_u16, scale_f32, gamma_f32, eps, 1.0, want_y=True)
    amax = max_abs(first["y"])
    out = residual_rms_rows(h_f32, o_u16, bias_u16, scale_f32, gamma_f32, eps, 0.0, want_y=want_y,
                            scales_rows=scales_rows, gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


def residual_rms_adaln_rows(h_f32, o_u16, bias_u16, gate_table_u16, w_u16, table_u16, frame_idx, eps: float,
                            global_amax: float, row_ids=None, want_y: bool = False,
                            scales_rows: int | None = None, gsf: float | None = None):
    """Gated residual add into an fp32 stream, then RMSNorm + adaLN -> NVFP4 over rows.

    h_f32 [n, k] is not modified (the updated stream is returned as 'h').  o_u16 [n, k] bf16
    or None; bias_u16 [k] or None; gate_table_u16 [T, k] (the folding block's gates);
    w_u16 [k]; table_u16 [T, 2, k] (the next block's shift, scale); frame_idx [n].
    Returns dict(codes, scale_bytes, y, scales, rstd, h, status).
    """
    h = np.array(h_f32, dtype=np.float32, copy=True, order="C")
    n, k = h.shape
    o = None if o_u16 is None else _c(o_u16, np.uint16)
    bias = None if bias_u16 is None else _c(bias_u16, np.uint16).reshape(-1)
    gate = _c(gate_table_u16, np.uint16)
    w = _c(w_u16, np.uint16).reshape(-1)
    tab = _c(table_u16, np.uint16)
    T = tab.shape[0]
    if gate.shape != (T, k) or tab.shape != (T, 2, k) or w.size != k:
        raise ValueError("gate table [T, k], table [T, 2, k] and w [k] expected")
    if o is not None and o.shape != (n, k):
        raise ValueError("o must be [n, k]")
    idx = _c(frame_idx, np.int32).reshape(-1)
    rid = None if row_ids is None else _c(row_ids, np.int64)
    codes = np.empty((n, k // 2), np.uint8)
    sb = np.empty((n, k // 16), np.uint8)
    rstd = np.empty(n, np.float32)
    y = np.empty((n, k), np.uint16) if want_y else None
    scales = None if scales_rows is None else np.zeros((scales_rows, k // 16), np.uint8)
    status = np.zeros(1, np.uint32)
    g = float(global_scale(global_amax) if gsf is None else gsf)
    shift_ptr = tab.ctypes.data
    scale_ptr = tab.ctypes.data + k * tab.itemsize
    _load().orc_residual_rms_adaln_rows_gsf(_ptr(h), _ptr(o), _ptr(bias), _ptr(gate), k, _ptr(w), shift_ptr,
                                            scale_ptr, 2 * k, T, _ptr(idx), float(eps), n, k, _ptr(rid), g,
                                            _ptr(codes), _ptr(sb), _ptr(scales), _ptr(rstd), _ptr(y), _ptr(status))
    return dict(codes=codes, scale_bytes=sb, y=y, scales=scales, rstd=rstd, h=h, status=int(status[0]))


def residual_rms_adaln_dynamic(h_f32, o_u16, bias_u16, gate_table_u16, w_u16, table_u16, frame_idx, eps: float,
                               want_y: bool = False, scales_rows: int | None = None):
    """residual_rms_adaln_rows under the amax of the call's own y.  Adds 'amax'."""
    first = residual_rms_adaln_rows(h_f32, o_u16, bias_u16, gate_table_u16, w_u16, table_u16, frame_idx, eps, 1.0,
                                    want_y=True)
    amax = max_abs(first["y"])
    out = residual_rms_adaln_rows(h_f32, o_u16, bias_u16, gate_table_u16, w_u16, table_u16, frame_idx, eps, 0.0,
                                  want_y=want_y, scales_rows=scales_rows, gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


_silu_cache = None


def silu_table() -> np.ndarray:
    """The 65536-entry bf16 SiLU table (C, long double, single rounding)."""
    global _silu_cache
    if _silu_cache is None:
        t = np.empty(65536, np.uint16)
        amb = _load().orc_silu_table(_ptr(t))
        if amb:
            raise RuntimeError("oracle SiLU table: %d entries undecidable in long double" % amb)
        _silu_cache = t
    return _silu_cache


def swiglu_rows(up_u16, gate_u16, global_amax: float, row_ids=None, want_y: bool = False,
                scales_rows: int | None = None, gsf: float | None = None):
    """SwiGLU -> NVFP4: y = bf16(S[gate] * up), then the block quantizer.

    up_u16 / gate_u16: [n, f] bf16 (views into a packed [n, 2f] are fine).
    gsf: use this global scale as is (global_amax is then ignored).
    """
    up = _c(up_u16, np.uint16)
    gate = _c(gate_u16, np.uint16)
    n, f = up.shape
    table = silu_table()
    rid = None if row_ids is None else _c(row_ids, np.int64)
    codes = np.empty((n, f // 2), np.uint8)
    sb = np.empty((n, f // 16), np.uint8)
    y = np.empty((n, f), np.uint16) if want_y else None
    scales = None
    if scales_rows is not None:
        scales = np.zeros((scales_rows, f // 16), np.uint8)
    fn = _load().orc_swiglu_rows if gsf is None else _load().orc_swiglu_rows_gsf
    fn(_ptr(up), _ptr(gate), f, n, f, _ptr(rid), _ptr(table), float(global_amax if gsf is None else gsf),
       _ptr(codes), _ptr(sb), _ptr(scales), _ptr(y))
    return dict(codes=codes, scale_bytes=sb, y=y, scales=scales)


def swiglu_dynamic(up_u16, gate_u16, want_y: bool = False, scales_rows: int | None = None):
    """SwiGLU -> NVFP4 under the amax of the tensor's own y (two passes).  The result dict
    gains 'amax'."""
    first = swiglu_rows(up_u16, gate_u16, 1.0, want_y=True)
    amax = max_abs(first["y"])
    out = swiglu_rows(up_u16, gate_u16, 0.0, want_y=want_y, scales_rows=scales_rows,
                      gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


def swiglu_packed_rows(proj_u16, bias_u16, interleaved: bool, global_amax: float, row_ids=None,
                       want_y: bool = False, scales_rows: int | None = None, gsf: float | None = None):
    """SwiGLU -> NVFP4 of a packed projection [n, 2f] with an optional bf16 bias [2f].

    interleaved False: value columns [0, f), gate columns [f, 2f); True: value at column
    2j and gate at 2j + 1.  bias (None: no bias) follows the projection's column order and
    is added as a bf16 tensor add before SiLU and the product.
    gsf: use this global scale as is (global_amax is then ignored).
    """
    proj = _c(proj_u16, np.uint16)
    n, two_f = proj.shape
    f = two_f // 2
    bias = None if bias_u16 is None else _c(bias_u16, np.uint16).reshape(-1)
    if bias is not None and bias.size != two_f:
        raise ValueError("bias must hold 2f entries")
    rid = None if row_ids is None else _c(row_ids, np.int64)
    codes = np.empty((n, f // 2), np.uint8)
    sb = np.empty((n, f // 16), np.uint8)
    y = np.empty((n, f), np.uint16) if want_y else None
    scales = None if scales_rows is None else np.zeros((scales_rows, f // 16), np.uint8)
    g = float(global_scale(global_amax) if gsf is None else gsf)
    _load().orc_swiglu_packed_rows_gsf(_ptr(proj), _ptr(bias), int(bool(interleaved)), two_f, n, f, _ptr(rid),
                                       _ptr(silu_table()), g, _ptr(codes), _ptr(sb), _ptr(scales), _ptr(y))
    return dict(codes=codes, scale_bytes=sb, y=y, scales=scales)


def swiglu_packed_dynamic(proj_u16, bias_u16, interleaved: bool, want_y: bool = False,
                          scales_rows: int | None = None):
    """swiglu_packed_rows under the amax of the tensor's own y (two passes).  The result
    dict gains 'amax'."""
    first = swiglu_packed_rows(proj_u16, bias_u16, interleaved, 1.0, want_y=True)
    amax = max_abs(first["y"])
    out = swiglu_packed_rows(proj_u16, bias_u16, interleaved, 0.0, want_y=want_y, scales_rows=scales_rows,
                             gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


# --------------------------------------------------------------------------
# fp16: codec, SiLU table, channels-last RMSNorm + SiLU -> NVFP4
# --------------------------------------------------------------------------

def f16_round(f32) -> np.ndarray:
    """fp32 -> fp16 bit patterns, round to nearest even (NaN -> 0x7E00)."""
    a = _c(f32, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_f16_round(_ptr(a), _ptr(out), a.size)
    return out


def f16_to_f32(u16) -> np.ndarray:
    return np.asarray(u16, np.uint16).view(np.float16).astype(np.float32)


_silu16_cache = None


def silu_table_f16() -> np.ndarray:
    """The 65536-entry fp16 SiLU table (C, long double, single rounding)."""
    global _silu16_cache
    if _silu16_cache is None:
        t = np.empty(65536, np.uint16)
        amb = _load().orc_silu_table_f16(_ptr(t))
        if amb:
            raise RuntimeError("oracle fp16 SiLU table: %d entries undecidable in long double" % amb)
        _silu16_cache = t
    return _silu16_cache


def rms_sum_f16row(x_row_u16) -> float:
    """The fixed-tree sum of x^2 over one fp16 row (c % 16 == 0, c <= 512)."""
    x = _c(x_row_u16, np.uint16).reshape(-1)
    return _load().orc_rms_sum_f16row(_ptr(x), x.size)


def rms_rstd_f16row(x_row_u16, eps: float) -> float:
    x = _c(x_row_u16, np.uint16).reshape(-1)
    return _load().orc_rms_rstd_f16row(_ptr(x), x.size, float(eps))


def rms_silu_rows(x_u16, gamma_u16, eps: float, global_amax: float, want_y: bool = False,
                  gsf: float | None = None):
    """Channels-last RMSNorm (fp32 statistic, fp16 affine) + SiLU -> NVFP4 over rows.

    x_u16 [n, c] fp16 patterns (c % 16 == 0, c <= 512); gamma_u16 [c] fp16.
    Returns dict(codes [n, c/2], scale_bytes [n, c/16] (the plain scale layout of this
    producer), rstd [n], y [n, c] fp16 or None).
    """
    x = _c(x_u16, np.uint16)
    n, c = x.shape
    if c % 16 or c > 512:
        raise ValueError("c must be a multiple of 16, at most 512")
    gamma = _c(gamma_u16, np.uint16).reshape(-1)
    codes = np.empty((n, c // 2), np.uint8)
    sb = np.empty((n, c // 16), np.uint8)
    rstd = np.empty(n, np.float32)
    y = np.empty((n, c), np.uint16) if want_y else None
    g = float(global_scale(global_amax) if gsf is None else gsf)
    _load().orc_rms_silu_rows_gsf(_ptr(x), _ptr(gamma), float(eps), n, c, _ptr(silu_table_f16()), g, _ptr(codes),
                                  _ptr(sb), _ptr(rstd), _ptr(y))
    return dict(codes=codes, scale_bytes=sb, rstd=rstd, y=y)


def max_abs_f16(u16) -> float:
    """max |x| over fp16 patterns (no NaN), as fp32 (exact)."""
    return float(np.abs(f16_to_f32(u16)).max()) if np.asarray(u16).size else 0.0


def rms_silu_dynamic(x_u16, gamma_u16, eps: float, want_y: bool = False):
    """rms_silu_rows under the amax of the call's own y.  Adds 'amax'."""
    first = rms_silu_rows(x_u16, gamma_u16, eps, 1.0, want_y=True)
    amax = max_abs_f16(first["y"])
    out = rms_silu_rows(x_u16, gamma_u16, eps, 0.0, want_y=want_y, gsf=dynamic_global_scale(amax))
    out["amax"] = amax
    return out


def tree_sum_f32(v_f32, squares: bool = False) -> float:
    """The fixed-tree sum (or sum of squares, fma) of one fp32 row, k % 512 == 0."""
    v = _c(v_f32, np.float32).reshape(-1)
    return _load().orc_tree_sum_f32(_ptr(v), v.size, int(bool(squares)))


def e4m3_encode_signed(f32) -> np.ndarray:
    a = _c(f32, np.float32)
    out = np.empty(a.shape, np.uint8)
    _load().orc_e4m3_encode_signed(_ptr(a), _ptr(out), a.size)
    return out


def fp8_inverse_scale(act_scale: float) -> float:
    return _load().orc_fp8_inverse_scale(float(act_scale))


def fp8_dynamic_scale(amax: float) -> float:
    """The per-call FP8 scale amax / 448 (fp32)."""
    return _load().orc_fp8_dynamic_scale(float(amax))


def fp8_dynamic_inverse(act_scale: float) -> float:
    """1 / act_scale, or 0 when act_scale is 0 or the reciprocal overflows."""
    return _load().orc_fp8_dynamic_inverse(float(act_scale))


def ln_adaln_fp8_rows(x_u16, scale_f32, shift_f32, eps: float, act_scale: float | None = None,
                      inv_scale: float | None = None, want_y: bool = True):
    """LayerNorm (fp32 statistics) + adaLN -> per-tensor FP8 E4M3 over fp16 rows [n, k].

    act_scale: the static per-tensor scale (codes = E4M3(y * (1 / act_scale))); or pass
    inv_scale directly.  Returns dict(codes [n, k] u8, mean [n], rstd [n], y [n, k] fp32,
    or None without want_y).
    """
    x = _c(x_u16, np.uint16)
    n, k = x.shape
    sc = _c(scale_f32, np.float32).reshape(-1)
    sh = _c(shift_f32, np.float32).reshape(-1)
    if sc.size != k or sh.size != k or k % 512:
        raise ValueError("scale and shift hold k values; k % 512 == 0")
    inv = fp8_inverse_scale(act_scale) if inv_scale is None else float(inv_scale)
    codes = np.empty((n, k), np.uint8)
    mean = np.empty(n, np.float32)
    rstd = np.empty(n, np.float32)
    y = np.empty((n, k), np.float32) if want_y else None
    _load().orc_ln_adaln_fp8_rows(_ptr(x), _ptr(sc), _ptr(sh), float(eps), n, k, inv, _ptr(codes), _ptr(mean),
                                  _ptr(rstd), _ptr(y) if want_y else None)
    return dict(codes=codes, mean=mean, rstd=rstd, y=y)


def ln_adaln_fp8_dynamic(x_u16, scale_f32, shift_f32, eps: float):
    """The per-call form: act_scale = max|y| / 448 from the call's own y, then the
    quantizer with 1 / act_scale (0 when the scale is 0).  Adds 'amax' and 'act_scale'."""
    first = ln_adaln_fp8_rows(x_u16, scale_f32, shift_f32, eps, inv_scale=1.0)
    amax = float(np.abs(first["y"]).max()) if first["y"].size else 0.0
    act = fp8_dynamic_scale(amax)
    inv = fp8_dynamic_inverse(act)
    out = ln_adaln_fp8_rows(x_u16, scale_f32, shift_f32, eps, inv_scale=inv)
    out["amax"], out["act_scale"] = amax, act
    return out


def _round_fraction_to_f16(q: Fraction) -> int:
    """Exact rational -> nearest fp16 bit pattern, ties to even."""
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a == 0:
        return sign
    if a >= 65520:
        return sign | 0x7C00
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    elif Fraction(2) ** (E + 1) <= a:
        E += 1
    qexp = -24 if E < -14 else E - 10
    n = a / (Fraction(2) ** qexp)
    fl = n.numerator // n.denominator
    frac = n - fl
    if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 45):
        raise ArithmeticError("SiLU value too close to an fp16 midpoint for 60-digit evaluation")
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    value = float(Fraction(fl) * Fraction(2) ** qexp)   # exact: <= 11 significant bits
    return sign | int(np.array([value], np.float16).view(np.uint16)[0])


def silu_exact_f16() -> np.ndarray:
    """fp16 SiLU table from Python's decimal module (60 digits), independent of the C
    table.  g <= -25 gives |g| e^g < 2^-25 (half the smallest fp16 subnormal): -0;
    g >= 20 differs from g by a relative e^-20, below half an fp16 ulp: g."""
    import decimal
    ctx = decimal.Context(prec=60)
    out = np.empty(65536, np.uint16)
    vals = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    for g in range(65536):
        e = (g >> 10) & 0x1F
        if e == 0x1F:
            out[g] = 0x7E00 if (g & 0x3FF) else (0x8000 if g & 0x8000 else 0x7C00)
            continue
        x = float(vals[g])
        if x <= -25.0:
            out[g] = 0x8000
            continue
        if x >= 20.0:
            out[g] = g
            continue
        if x == 0.0:
            out[g] = g
            continue
        dx = decimal.Decimal(x)
        s = ctx.divide(dx, ctx.add(decimal.Decimal(1), ctx.exp(ctx.minus(dx))))
        out[g] = _round_fraction_to_f16(Fraction(s))
    return out


# --------------------------------------------------------------------------
# independent derivation of the SiLU table (exact decimal arithmetic)
# --------------------------------------------------------------------------

def _round_fraction_to_bf16(q: Fraction) -> int:
    """Exact rational -> nearest bf16 bit pattern, ties to even."""
    sign = 0x8000 if q < 0 else 0
    a = -q if q < 0 else q
    if a == 0:
        return sign
    # exponent E with 2^E <= a < 2^(E+1)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    elif Fraction(2) ** (E + 1) <= a:
        E += 1
    qexp = -133 if E < -126 else E - 7
    n = a / (Fraction(2) ** qexp)
    fl = n.numerator // n.denominator
    frac = n - fl
    if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 45):
        raise ArithmeticError("SiLU value too close to a bf16 midpoint for 60-digit evaluation")
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    value = Fraction(fl) * Fraction(2) ** qexp
    if value >= Fraction(2) ** 128:
        return sign | 0x7F80
    # encode: value = fl * 2^qexp, fl <= 256
    f = np.float32(float(value))  # exact: <= 9 significant bits, in fp32 range
    return sign | int(np.array([f], np.float32).view(np.uint32)[0] >> 16)


def silu_exact() -> np.ndarray:
    """SiLU table from Python's decimal module (60 significant digits).

    For |g| >= 100 the rounding is decided by a bound instead of evaluating:
    g <= -100 gives |g| e^g < 2^-134 (half the smallest bf16 subnormal), so -0;
    g >= 100 differs from g by a relative e^-100, far below half a bf16 ulp, so g.
    """
    import decimal
    ctx = decimal.Context(prec=60)
    out = np.empty(65536, np.uint16)
    for g in range(65536):
        e = (g >> 7) & 0xFF
        if e == 0xFF:
            out[g] = 0x7FC0 if (g & 0x7F) else (0x8000 if g & 0x8000 else 0x7F80)
            continue
        x = float(np.array([g << 16], np.uint32).view(np.float32)[0])
        if x <= -100.0:
            out[g] = 0x8000
            continue
        if x >= 100.0:
            out[g] = g
            continue
        if x == 0.0:
            out[g] = g  # silu(+-0) = +-0
            continue
        dx = decimal.Decimal(x)  # exact binary value
        s = ctx.divide(dx, ctx.add(decimal.Decimal(1), ctx.exp(ctx.minus(dx))))
        out[g] = _round_fraction_to_bf16(Fraction(s))
    return out
