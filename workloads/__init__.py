"""Seeded synthetic inputs for the NVFP4 activation-quantization producers.

This module holds input construction only: random draws, shapes, frame
indices and the bf16 conversion of the drawn fp32 samples (done by torch's
own ``Tensor.to(torch.bfloat16)``).  It contains none of the method's
arithmetic, and both the CPU oracle and the GPU library consume what it
produces.

Workloads (shapes from the pages' H3 block: 56 heads x 128 = 7168 hidden,
a 34x60 latent grid per frame over 31 frames = 63,240 tokens from
544x960x124 video; SwiGLU hidden 19,456; and a 300,000-token shape past the
2^31-element boundary reported in the FastVideo commit log):

  rms_adaln_256x2048       tiny RMSNorm+adaLN (8 frames, frame = token // 32)
  quantize_63240x7168      attention-output quantize (per-head std)
  rms_adaln_63240x7168     RMSNorm+adaLN at the H3 block shape (31 frames)
  swiglu_16384x19456       SwiGLU producer over a value-first [M, 2F] projection
  rms_adaln_300000x7168    RMSNorm+adaLN over 2.15e9 elements (147 frames)
  swiglu_bias_16384x19456  the same projection shape, value-first, with a bf16 bias
                           of 2F values (std 0.25) added before SiLU
  swiglu_paired_16384x19456  the same with value/gate columns paired (2j, 2j + 1)
  residual_rms_63240x7168  fp32 residual stream h (the H3 block shape, N(0,1) with the
                           36 outlier columns x30 of rms_adaln_63240x7168), a bf16 branch
                           output o ~ N(0,1), bf16 bias (std 0.25), fp32 per-channel
                           scale (std 0.2) and fp32 RMSNorm weight 1 + 0.1 N(0,1)
  residual_adaln_63240x7168  the same stream and branch, gated by a per-frame bf16 gate
                           table (31 x 7168, std 0.2) of the folding block, then RMSNorm
                           (bf16 weight) + adaLN with the next block's (shift, scale) table
                           (31 frames, frame = token // 2040, as rms_adaln_63240x7168)
  rms_silu_16x120x216x192  fp16 channels-last VAE activations: 16 frames of 120 x 216
                           voxels (half the 432 x 240 clip in each direction), 192
                           channels; x ~ N(0,1), gamma = 1 + 0.1 N(0,1), eps = 1e-6
  ln_fp8_63240x7168        LayerNorm + adaLN -> per-tensor FP8 over fp16 hidden states of
                           the H3 block shape (the recipe of rms_adaln_63240x7168 in
                           fp16); fp32 modulation vectors scale, shift ~ 0.1 N(0,1)

Seeds: numpy ``PCG64``; the seed of role ``role`` in workload number ``i``
(1..11 in the order above) is ``1000*i + role`` with roles 1 x (or h), 2 weight
(or bias), 3 modulation table (or residual scale), 4 calibration rows, 5
outlier pick, 6 per-head std, 8 the residual branch o, 9 its calibration rows,
10 the fp32 RMSNorm weight, 11 the gate table, 12 the bias where a weight is
drawn too.
Large tensors are drawn in 4096-row chunks, chunk ``c`` from
``SeedSequence(1000*i + role).spawn(n_chunks)[c]``, so any chunk can be
regenerated alone and chunks can be drawn in parallel threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 4096
ROLE_X, ROLE_W, ROLE_TABLE, ROLE_CAL, ROLE_OUTLIER, ROLE_HEADSTD = 1, 2, 3, 4, 5, 6
ROLE_O, ROLE_CAL_O, ROLE_GAMMA, ROLE_GATE, ROLE_BIAS = 8, 9, 10, 11, 12


def to_f16(a: np.ndarray) -> np.ndarray:
    """fp32 samples -> fp16 bit patterns (uint16), via torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 samples -> bf16 bit patterns (uint16), via torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rng(i: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * i + role))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class Workload:
    name: str
    number: int               # 1..5, selects the seeds
    kind: str                 # "rms_adaln" | "quantize" | "swiglu" | "residual_rms" | "residual_adaln" | "rms_silu"
    m: int                    # rows (tokens)
    k: int                    # output columns (hidden, or F for swiglu)
    frames: int = 0           # modulation table rows (rms_adaln)
    rows_per_frame: int = 0   # frame index = row // rows_per_frame
    eps: float = 1e-6
    outliers: str = ""        # "iid1pct_x20" | "cols36_x30" | ""
    cal_rows: int = 0         # calibration rows for the static amax (0: from the data itself)
    bias_std: float = 0.0     # swiglu: std of the 2F-entry bias (0: no bias)
    interleaved: bool = False  # swiglu: value/gate columns paired instead of value-first
    extra: dict = field(default_factory=dict)

    # ---- sizes -------------------------------------------------------------
    @property
    def padded_rows(self) -> int:
        if self.kind == "rms_silu":
            return self.m                      # plain scale layout: no padding rows
        return (self.m + 127) // 128 * 128

    @property
    def in_cols(self) -> int:
        return 2 * self.k if self.kind == "swiglu" else self.k

    def algorithmic_bytes(self) -> int:
        """HBM bytes one pass must move: bf16 inputs once, packed codes once,
        scale bytes over the padded rows (parameters not counted).  residual_rms: the
        fp32 stream read and written back, the bf16 branch read."""
        out = self.m * self.k // 2 + self.padded_rows * self.k // 16
        if self.kind == "ln_fp8":
            return 2 * self.m * self.k + self.m * self.k       # fp16 in, one FP8 byte out
        if self.kind in ("residual_rms", "residual_adaln"):
            return (4 + 2 + 4) * self.m * self.k + out
        return 2 * self.m * self.in_cols + out

    def param_bytes(self) -> int:
        if self.kind == "rms_adaln":
            return 2 * self.k + 2 * self.frames * 2 * self.k + 4 * self.m
        if self.kind == "swiglu" and self.bias_std > 0:
            return 2 * 2 * self.k
        if self.kind == "residual_rms":
            return (2 + 4 + 4) * self.k
        if self.kind == "residual_adaln":
            return 2 * self.k + 2 * self.frames * self.k + 2 * self.k + 2 * self.frames * 2 * self.k + 4 * self.m
        if self.kind == "rms_silu":
            return 2 * self.k
        if self.kind == "ln_fp8":
            return 2 * 4 * self.k
        return 0

    # ---- generation ----------------------------------------------------------
    def n_chunks(self, rows: int) -> int:
        return (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def _chunk_f32(self, role: int, rows: int, c: int, cols_out: np.ndarray | None,
                   head_std: np.ndarray | None) -> np.ndarray:
        seeds = np.random.SeedSequence(1000 * self.number + role).spawn(self.n_chunks(rows))
        g = np.random.Generator(np.random.PCG64(seeds[c]))
        r = min(CHUNK_ROWS, rows - c * CHUNK_ROWS)
        a = g.standard_normal((r, self.in_cols), dtype=np.float32)
        if self.outliers == "iid1pct_x20":
            mask = g.random((r, self.in_cols), dtype=np.float32) < 0.01
            a[mask] *= 20.0
        elif self.outliers == "cols36_x30":
            a[:, cols_out] *= 30.0
        if head_std is not None:
            a *= np.repeat(head_std, 128)[None, :]
        return a

    def outlier_columns(self) -> np.ndarray | None:
        if self.outliers != "cols36_x30":
            return None
        n = int(round(0.005 * self.k))
        return np.sort(rng(self.number, ROLE_OUTLIER).choice(self.k, n, replace=False))

    def head_std(self) -> np.ndarray | None:
        if self.kind != "quantize":
            return None
        heads = self.k // 128
        return (0.5 * rng(self.number, ROLE_HEADSTD).uniform(0.2, 2.0, heads)).astype(np.float32)

    def _rows_bf16(self, role: int, rows: int, chunks=None, out: np.ndarray | None = None, fp32: bool = False,
                   plain: bool = False):
        """Rows drawn in chunks; bf16 patterns, or the fp32 draws themselves with fp32.
        plain: N(0,1) without the workload's outlier or per-head recipe."""
        cols = None if plain else self.outlier_columns()
        hs = None if plain else self.head_std()
        idx = range(self.n_chunks(rows)) if chunks is None else chunks
        idx = list(idx)

        conv = to_f16 if self.kind in ("rms_silu", "ln_fp8") else to_bf16

        def one(c):
            a = self._chunk_f32(role, rows, c, cols, hs)
            return c, (a if fp32 else conv(a))

        parts = {}
        with ThreadPoolExecutor(_threads()) as ex:
            for c, a in ex.map(one, idx):
                if out is not None:
                    out[c * CHUNK_ROWS:c * CHUNK_ROWS + a.shape[0]] = a
                else:
                    parts[c] = a
        if out is not None:
            return out
        return np.concatenate([parts[c] for c in idx], axis=0)

    def x(self, out: np.ndarray | None = None) -> np.ndarray:
        """The full input [m, in_cols] as bf16 patterns."""
        if out is None:
            out = np.empty((self.m, self.in_cols), np.uint16)
        return self._rows_bf16(ROLE_X, self.m, out=out)

    # ---- residual_rms inputs -------------------------------------------------
    def h(self, out: np.ndarray | None = None) -> np.ndarray:
        """residual_rms: the fp32 residual stream [m, k]."""
        if out is None:
            out = np.empty((self.m, self.k), np.float32)
        return self._rows_bf16(ROLE_X, self.m, out=out, fp32=True)

    def o(self, out: np.ndarray | None = None) -> np.ndarray:
        """residual_rms: the bf16 branch output [m, k], N(0,1)."""
        if out is None:
            out = np.empty((self.m, self.k), np.uint16)
        return self._rows_bf16(ROLE_O, self.m, out=out, plain=True)

    def h_rows(self, rows) -> np.ndarray:
        return self.x_rows(rows, ROLE_X, fp32=True)

    def o_rows(self, rows) -> np.ndarray:
        return self.x_rows(rows, ROLE_O, plain=True)

    def calibration_h(self) -> np.ndarray:
        return self._rows_bf16(ROLE_CAL, self.cal_rows, fp32=True)

    def calibration_o(self) -> np.ndarray:
        return self._rows_bf16(ROLE_CAL_O, self.cal_rows, plain=True)

    def modulation(self) -> tuple[np.ndarray, np.ndarray]:
        """ln_fp8: the fp32 adaLN (scale, shift) vectors [k]."""
        g = rng(self.number, ROLE_TABLE)
        sc = (0.1 * g.standard_normal(self.k, dtype=np.float32)).astype(np.float32)
        sh = (0.1 * g.standard_normal(self.k, dtype=np.float32)).astype(np.float32)
        return sc, sh

    def residual_scale(self) -> np.ndarray:
        """residual_rms: the fp32 per-channel scale [k] of the branch."""
        return (0.2 * rng(self.number, ROLE_TABLE).standard_normal(self.k, dtype=np.float32)).astype(np.float32)

    def gamma(self) -> np.ndarray:
        """residual_rms: the fp32 RMSNorm weight [k]."""
        return (1.0 + 0.1 * rng(self.number, ROLE_GAMMA).standard_normal(self.k, dtype=np.float32)).astype(
            np.float32)

    def x_rows(self, rows, role: int = ROLE_X, fp32: bool = False, plain: bool = False) -> np.ndarray:
        """Rows of the input (or of another role's rows) regenerated from their chunks alone."""
        rows = np.asarray(rows, np.int64)
        chunks = sorted(set((rows // CHUNK_ROWS).tolist()))
        blocks = self._rows_bf16(role, self.m, chunks=chunks, fp32=fp32, plain=plain)
        pos = {c: i for i, c in enumerate(chunks)}
        starts = np.cumsum([0] + [min(CHUNK_ROWS, self.m - c * CHUNK_ROWS) for c in chunks])
        sel = [starts[pos[int(r // CHUNK_ROWS)]] + int(r % CHUNK_ROWS) for r in rows]
        return blocks[sel]

    def calibration_x(self) -> np.ndarray:
        return self._rows_bf16(ROLE_CAL, self.cal_rows)

    def weight(self) -> np.ndarray:
        """The RMSNorm weight [k]: bf16, or fp16 for the fp16 (rms_silu) workload."""
        conv = to_f16 if self.kind == "rms_silu" else to_bf16
        return conv(1.0 + 0.1 * rng(self.number, ROLE_W).standard_normal(self.k, dtype=np.float32))

    def bias(self) -> np.ndarray | None:
        """swiglu: the [2k] bf16 bias in the projection's column order; residual_rms: the
        [k] bf16 bias of the branch; None without a bias."""
        if self.bias_std <= 0:
            return None
        if self.kind == "residual_adaln":
            g = rng(self.number, ROLE_BIAS)
            return to_bf16(self.bias_std * g.standard_normal(self.k, dtype=np.float32))
        n = self.k if self.kind == "residual_rms" else 2 * self.k
        return to_bf16(self.bias_std * rng(self.number, ROLE_W).standard_normal(n, dtype=np.float32))

    def gate_table(self) -> np.ndarray:
        """residual_adaln: the folding block's [frames, k] bf16 gate rows (std 0.2)."""
        g = rng(self.number, ROLE_GATE)
        return to_bf16(0.2 * g.standard_normal((self.frames, self.k), dtype=np.float32))

    def table(self) -> np.ndarray:
        """[frames, 2, k] bf16: row t holds (shift, scale) of frame t."""
        t = 0.1 * rng(self.number, ROLE_TABLE).standard_normal((self.frames, 2, self.k),
                                                                dtype=np.float32)
        return to_bf16(t)

    def frame_idx(self, rows=None) -> np.ndarray:
        r = np.arange(self.m, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
        return (r // self.rows_per_frame).astype(np.int32)

    def calibration_frame_idx(self) -> np.ndarray:
        r = np.arange(self.cal_rows, dtype=np.int64)
        return ((r * self.frames) // self.cal_rows).astype(np.int32)

    def sample_rows(self, n_random: int = 8192, head: int = 4096, tail: int = 4096) -> np.ndarray:
        """First `head`, last `tail` and `n_random` seeded random rows (sorted, unique)."""
        g = np.random.Generator(np.random.PCG64(1000 * self.number + 7))
        parts = [np.arange(min(head, self.m)), np.arange(max(0, self.m - tail), self.m),
                 g.choice(self.m, size=min(n_random, self.m), replace=False)]
        return np.unique(np.concatenate(parts)).astype(np.int64)


WORKLOADS = {
    w.name: w for w in [
        Workload("rms_adaln_256x2048", 1, "rms_adaln", 256, 2048, frames=8, rows_per_frame=32,
                 outliers="iid1pct_x20"),
        Workload("quantize_63240x7168", 2, "quantize", 63240, 7168, cal_rows=8192),
        Workload("rms_adaln_63240x7168", 3, "rms_adaln", 63240, 7168, frames=31,
                 rows_per_frame=2040, outliers="cols36_x30", cal_rows=8192),
        Workload("swiglu_16384x19456", 4, "swiglu", 16384, 19456, cal_rows=2048),
        Workload("rms_adaln_300000x7168", 5, "rms_adaln", 300000, 7168, frames=147,
                 rows_per_frame=2041, outliers="cols36_x30", cal_rows=8192),
        Workload("swiglu_bias_16384x19456", 6, "swiglu", 16384, 19456, cal_rows=2048, bias_std=0.25),
        Workload("swiglu_paired_16384x19456", 7, "swiglu", 16384, 19456, cal_rows=2048, bias_std=0.25,
                 interleaved=True),
        Workload("residual_rms_63240x7168", 8, "residual_rms", 63240, 7168, outliers="cols36_x30",
                 cal_rows=8192, bias_std=0.25),
        Workload("residual_adaln_63240x7168", 9, "residual_adaln", 63240, 7168, frames=31,
                 rows_per_frame=2040, outliers="cols36_x30", cal_rows=8192, bias_std=0.25),
        Workload("rms_silu_16x120x216x192", 10, "rms_silu", 16 * 120 * 216, 192, cal_rows=32768),
        Workload("ln_fp8_63240x7168", 11, "ln_fp8", 63240, 7168, outliers="cols36_x30", cal_rows=8192),
    ]
}

BENCH_WORKLOAD = "rms_adaln_63240x7168"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def fp8_act_scale(name: str) -> float:
    """The static per-tensor FP8 scale of an ln_fp8 workload: its calibrated amax / 448."""
    return float(np.float32(calibration_amax(name)) / np.float32(448.0))


def calibration_amax(name: str) -> float:
    """The static global amax of a workload, read from the stored calibration
    file (written by tests/golden/make_calibration.py from the CPU oracle)."""
    import json
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "tests", "golden", "calibration_amax.json")
    with open(path) as f:
        data = json.load(f)
    return float(np.float32(data[name]["global_amax"]))
