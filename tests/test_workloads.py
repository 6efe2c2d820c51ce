"""Seeded input generators: determinism, shapes, chunk regeneration, calibration file."""
import json
import os

import numpy as np

import oracle
import workloads


def test_shapes_and_determinism():
    w = workloads.get("rms_adaln_256x2048")
    a, b = w.x(), w.x()
    assert a.shape == (256, 2048) and a.dtype == np.uint16
    assert np.array_equal(a, b)
    assert w.weight().shape == (2048,) and w.table().shape == (8, 2, 2048)
    assert np.array_equal(w.frame_idx(), np.arange(256) // 32)


def test_chunk_regeneration_matches_full_draw():
    w = workloads.Workload("t", 9, "rms_adaln", 9000, 512, frames=3, rows_per_frame=3000,
                           outliers="cols36_x30")
    full = w.x()
    rows = np.array([0, 1, 4095, 4096, 8191, 8192, 8999])
    assert np.array_equal(w.x_rows(rows), full[rows])


def test_outlier_recipes():
    w = workloads.get("rms_adaln_63240x7168")
    cols = w.outlier_columns()
    assert len(cols) == 36 and len(set(cols.tolist())) == 36
    w1 = workloads.get("rms_adaln_256x2048")
    x = oracle.bf16_to_f32(w1.x())
    frac_big = np.mean(np.abs(x) > 6)  # N(0,1) beyond 6 sigma is ~2e-9; outliers are x20
    assert 0.005 < frac_big < 0.015


def test_frames_cover_the_table():
    for name in ["rms_adaln_63240x7168", "rms_adaln_300000x7168"]:
        w = workloads.get(name)
        idx = w.frame_idx()
        assert idx.min() == 0 and idx.max() == w.frames - 1
        cal = w.calibration_frame_idx()
        assert cal.min() == 0 and cal.max() == w.frames - 1


def test_algorithmic_bytes():
    w = workloads.get("rms_adaln_63240x7168")
    assert w.algorithmic_bytes() == 1_161_646_080
    assert workloads.get("swiglu_16384x19456").algorithmic_bytes() == 1_454_374_912
    assert workloads.get("rms_adaln_300000x7168").algorithmic_bytes() == 5_510_414_336


def test_calibration_file_reproduces_for_the_tiny_workload():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "calibration_amax.json")
    data = json.load(open(path))
    assert set(data) == set(workloads.WORKLOADS)
    w = workloads.get("rms_adaln_256x2048")
    res = oracle.rms_adaln_rows(w.x(), w.weight(), w.table(), w.frame_idx(), w.eps, 1.0, want_y=True)
    amax = float(np.max(np.abs(oracle.bf16_to_f32(res["y"]))))
    assert amax == data[w.name]["global_amax"] == workloads.calibration_amax(w.name)


def test_packed_swiglu_workloads():
    for name, paired in [("swiglu_bias_16384x19456", False), ("swiglu_paired_16384x19456", True)]:
        w = workloads.get(name)
        assert w.interleaved == paired and w.in_cols == 2 * w.k
        b = w.bias()
        assert b.shape == (2 * w.k,) and b.dtype == np.uint16 and np.array_equal(b, w.bias())
        assert 0.2 < float(np.std(oracle.bf16_to_f32(b))) < 0.3
        assert w.algorithmic_bytes() == 1_454_374_912 and w.param_bytes() == 4 * w.k
    assert workloads.get("swiglu_16384x19456").bias() is None


def test_residual_rms_workload():
    w = workloads.get("residual_rms_63240x7168")
    assert w.algorithmic_bytes() == 10 * w.m * w.k + w.m * w.k // 2 + w.padded_rows * w.k // 16
    assert w.bias().shape == (w.k,) and w.residual_scale().dtype == np.float32 and w.gamma().shape == (w.k,)
    rows = np.array([0, 4095, 4096, 63239])
    h = w._rows_bf16(workloads.ROLE_X, w.m, chunks=[0, 1, 15], fp32=True)
    assert h.dtype == np.float32 and h.shape == (4096 * 2 + (w.m - 15 * 4096), w.k)
    cols = w.outlier_columns()
    assert np.std(h[:, cols]) > 20 and np.std(np.delete(h[:64], cols, axis=1)) < 1.1
    o = w.calibration_o()
    assert o.dtype == np.uint16 and o.shape == (w.cal_rows, w.k)
    del rows


def test_rms_silu_workload():
    w = workloads.get("rms_silu_16x120x216x192")
    assert w.m == 414720 and w.k == 192 and w.padded_rows == w.m
    assert w.algorithmic_bytes() == w.m * w.k * 2 + w.m * w.k // 2 + w.m * w.k // 16
    x = w.x_rows(np.array([0, 4096, w.m - 1]))
    xf = oracle.f16_to_f32(x)
    assert x.dtype == np.uint16 and np.all(np.isfinite(xf)) and 0.5 < float(np.std(xf)) < 1.5
    assert np.array_equal(oracle.f16_round(xf), x)                 # fp16 patterns


def test_ln_fp8_workload():
    w = workloads.get("ln_fp8_63240x7168")
    assert w.algorithmic_bytes() == 3 * w.m * w.k
    sc, sh = w.modulation()
    assert sc.dtype == np.float32 and sh.shape == (w.k,) and not np.array_equal(sc, sh)
    act = workloads.fp8_act_scale(w.name)
    assert act == np.float32(workloads.calibration_amax(w.name)) / np.float32(448.0)
