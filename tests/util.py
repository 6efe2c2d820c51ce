"""Helpers shared by the GPU parity tests: host<->device moves of bf16 patterns and
row-parallel oracle calls (ctypes releases the GIL, rows are independent)."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_device(a_u16: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(device)


def to_host(t) -> np.ndarray:
    a = t.cpu().numpy()
    if a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def split_rows(n: int, parts: int):
    step = max(1, (n + parts - 1) // parts)
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def oracle_rms_adaln(x, w, table, idx, eps, amax, row_ids=None, want_y=True, gsf=None):
    """oracle.rms_adaln_rows over row blocks in parallel threads; concatenated results
    (gsf: a global scale used as is instead of the one of amax)."""
    n = x.shape[0]
    rid = np.arange(n, dtype=np.int64) if row_ids is None else np.asarray(row_ids, np.int64)

    def part(se):
        s, e = se
        return oracle.rms_adaln_rows(x[s:e], w, table, idx[s:e], eps, amax, row_ids=rid[s:e], want_y=want_y,
                                     gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes", "rstd")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    out["status"] = int(np.bitwise_or.reduce([r["status"] for r in res]))
    return out


def oracle_quantize_rows(y, amax):
    n = y.shape[0]

    def part(se):
        s, e = se
        return oracle.quantize_rows(y[s:e], amax)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def oracle_swiglu(up, gate, amax, want_y=True, gsf=None):
    n = up.shape[0]
    oracle.silu_table()  # build once before the threads start

    def part(se):
        s, e = se
        return oracle.swiglu_rows(up[s:e], gate[s:e], amax, want_y=want_y, gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    return out


def oracle_swiglu_packed(proj, bias, interleaved, amax, want_y=True, gsf=None):
    """oracle.swiglu_packed_rows over row blocks in parallel threads."""
    n = proj.shape[0]
    oracle.silu_table()

    def part(se):
        s, e = se
        return oracle.swiglu_packed_rows(proj[s:e], bias, interleaved, amax, want_y=want_y, gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    return out


def oracle_residual_rms(h, o, bias, scale, gamma, eps, amax, want_y=True, gsf=None):
    """oracle.residual_rms_rows over row blocks in parallel threads; concatenated results
    (the updated stream as 'h')."""
    n = h.shape[0]

    def part(se):
        s, e = se
        return oracle.residual_rms_rows(h[s:e], None if o is None else o[s:e], bias, scale, gamma, eps, amax,
                                        want_y=want_y, gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes", "rstd", "h")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    return out


def oracle_residual_adaln(h, o, bias, gate, w, table, idx, eps, amax, want_y=True, gsf=None):
    """oracle.residual_rms_adaln_rows over row blocks in parallel threads."""
    n = h.shape[0]

    def part(se):
        s, e = se
        return oracle.residual_rms_adaln_rows(h[s:e], None if o is None else o[s:e], bias, gate, w, table,
                                              idx[s:e], eps, amax, want_y=want_y, gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes", "rstd", "h")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    out["status"] = int(np.bitwise_or.reduce([r["status"] for r in res]))
    return out


def oracle_rms_silu(x, gamma, eps, amax, want_y=True, gsf=None):
    """oracle.rms_silu_rows over row blocks in parallel threads."""
    n = x.shape[0]
    oracle.silu_table_f16()

    def part(se):
        s, e = se
        return oracle.rms_silu_rows(x[s:e], gamma, eps, amax, want_y=want_y, gsf=gsf)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "scale_bytes", "rstd")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    return out


def scales_from_rows(scale_bytes: np.ndarray, m: int, k: int, rows=None) -> np.ndarray:
    """Place plain-order scale bytes of rows into a zeroed swizzled [pad(m), k/16] buffer."""
    buf = np.zeros(oracle.padded_rows(m) * (k // 16), np.uint8)
    r = np.arange(scale_bytes.shape[0]) if rows is None else np.asarray(rows)
    buf[oracle.scale_offsets(r, k)] = scale_bytes
    return buf.reshape(oracle.padded_rows(m), k // 16)


def gather_scales(scales_buf: np.ndarray, rows, k: int) -> np.ndarray:
    """Plain-order scale bytes [len(rows), k/16] read out of a swizzled buffer."""
    return scales_buf.reshape(-1)[oracle.scale_offsets(np.asarray(rows), k)]


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    d = np.argwhere(a != b)
    if len(d) == 0:
        return "equal"
    i = tuple(d[0])
    return "%d mismatches; first at %s: got %r want %r" % (len(d), i, a[i], b[i])


def oracle_ln_fp8(x, scale, shift, eps, inv_scale, want_y=True):
    """oracle.ln_adaln_fp8_rows (codes under inv_scale) over row blocks in parallel threads."""
    n = x.shape[0]

    def part(se):
        s, e = se
        return oracle.ln_adaln_fp8_rows(x[s:e], scale, shift, eps, inv_scale=inv_scale, want_y=want_y)

    with ThreadPoolExecutor(threads()) as ex:
        res = list(ex.map(part, split_rows(n, 4 * threads())))
    out = {key: np.concatenate([r[key] for r in res]) for key in ("codes", "mean", "rstd")}
    out["y"] = np.concatenate([r["y"] for r in res]) if want_y else None
    return out


def oracle_ln_fp8_amax(x, scale, shift, eps) -> float:
    """max |y| of the LayerNorm + adaLN output over all rows (the per-call amax), by blocks."""
    n = x.shape[0]

    def part(se):
        s, e = se
        y = oracle.ln_adaln_fp8_rows(x[s:e], scale, shift, eps, inv_scale=1.0)["y"]
        return float(np.abs(y).max()) if y.size else 0.0

    with ThreadPoolExecutor(threads()) as ex:
        return max(ex.map(part, split_rows(n, 16 * threads())), default=0.0)
