"""GPU parity of the fp32 residual stream + RMSNorm (fp32 weight) -> NVFP4 producer, static
and per-call amax, through the C ABI, against the CPU oracle on the same seeded inputs:
codes, the whole swizzled scale buffer, the bf16 side output and the updated fp32 stream
bit for bit, rstd at 0 ulp."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from util import (first_mismatch, gather_scales, oracle_residual_adaln, oracle_residual_rms, scales_from_rows,
                  to_device, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def nq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_activation_quantization_amd as mod
    return mod


def assert_equal(got, want, what):
    assert np.array_equal(got, want), "%s: %s" % (what, first_mismatch(got, want))


def u32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def case(m, k, seed, form="bias", h_std=2.0):
    g = np.random.Generator(np.random.PCG64(seed))
    h = (g.standard_normal((m, k)) * h_std).astype(np.float32)
    o = oracle.bf16_round(g.standard_normal((m, k)).astype(np.float32)) if form != "none" else None
    bias = oracle.bf16_round((0.5 * g.standard_normal(k)).astype(np.float32)) if form == "bias" else None
    scale = (0.3 * g.standard_normal(k)).astype(np.float32) if form != "none" else None
    gamma = (1 + 0.1 * g.standard_normal(k)).astype(np.float32)
    return h, o, bias, scale, gamma


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def gpu_residual(nq, h, o, bias, scale, gamma, eps, amax, y=True, dynamic=False):
    m, k = h.shape
    hd = dev_f32(h)
    residual = None if o is None else (to_device(o), None if bias is None else to_device(bias), dev_f32(scale))
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    yd = torch.empty((m, k), dtype=torch.int16, device="cuda:0") if y else None
    if dynamic:
        codes, scales, amax_t = nq.residual_rms_nvfp4_dynamic(hd, dev_f32(gamma), eps, residual=residual,
                                                               rstd_out=rstd, y_out=yd)
    else:
        codes, scales = nq.residual_rms_nvfp4(hd, dev_f32(gamma), eps, amax, residual=residual, rstd_out=rstd,
                                              y_out=yd)
        amax_t = None
    torch.cuda.synchronize()
    out = dict(codes=to_host(codes), scales=to_host(scales), y=to_host(yd) if y else None,
               rstd=rstd.cpu().numpy(), h=hd.cpu().numpy())
    if dynamic:
        out["amax"] = float(amax_t.cpu().numpy()[0])
    return out


def check(got, h, o, bias, scale, gamma, eps, amax):
    m, k = h.shape
    want = oracle_residual_rms(h, o, bias, scale, gamma, eps, amax, want_y=got["y"] is not None)
    assert_equal(u32(got["h"]), u32(want["h"]), "h")
    assert_equal(u32(got["rstd"]), u32(want["rstd"]), "rstd")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, k), "scales")


@pytest.mark.parametrize("form", ["bias", "nobias", "none"])
@pytest.mark.parametrize("m,k", [(1, 512), (127, 1024), (129, 1536), (129, 2048), (64, 3584), (200, 4608),
                                 (64, 6144), (300, 7168), (257, 8192)])
def test_shapes(nq, m, k, form):
    print("residual_rms", m, k, form, flush=True)
    h, o, bias, scale, gamma = case(m, k, 13 * m + k + len(form), form)
    for amax in [12.0, 2688.0]:
        got = gpu_residual(nq, h, o, bias, scale, gamma, 1e-6, amax)
        check(got, h, o, bias, scale, gamma, 1e-6, amax)
        if form == "none":
            assert_equal(u32(got["h"]), u32(h), "h (only read)")


def test_hand_worked_row(nq):
    blk = json.load(open(os.path.join(GOLDEN, "hand_worked_blocks.json")))["blocks"][0]
    k = 512
    gamma = np.ones(k, np.float32)
    gamma[:16] = np.array([-0.0 if v == "-0" else float(v) for v in blk["values"]], np.float32)
    h = np.full((1, k), 1.5, np.float32)
    o = oracle.bf16_round(np.full((1, k), 0.25, np.float32))
    bias = oracle.bf16_round(np.full(k, 0.25, np.float32))
    got = gpu_residual(nq, h, o, bias, np.ones(k, np.float32), gamma, 0.0, blk["global_amax"])
    assert np.all(got["h"] == 2.0) and got["rstd"][0] == 0.5
    row0 = gather_scales(got["scales"], [0], k)[0]          # row 0's bytes out of the swizzle
    assert row0[0] == blk["scale_code"] and np.all(row0[1:] == 0x23)
    assert got["codes"][0, :8].tobytes().hex() == blk["packed_hex"]
    assert np.all(got["codes"][0, 8:] == 0x77)
    # every other byte of the buffer belongs to the padding rows 1..127
    assert np.count_nonzero(got["scales"]) == np.count_nonzero(row0)


def test_special_rows(nq):
    """Zero rows (rstd = 1/sqrt(eps)), a row cancelled exactly by its branch, signed zeros,
    huge and tiny stream values, a branch that rounds onto bf16 ties."""
    m, k = 8, 1024
    h, o, bias, scale, gamma = case(m, k, 99)
    h[0] = 0.0
    o[0] = 0
    h[1] = -0.0
    h[2] = 1e30
    h[3] = 1e-30
    h[4, ::2] *= 1e4
    # row 5: h = -(o + bias) * scale exactly where representable (cancellation to +-0)
    t = oracle.bf16_to_f32(oracle.bf16_round(oracle.bf16_to_f32(o[5]) + oracle.bf16_to_f32(bias)))
    h[5] = -(t * scale)
    # row 6: o values that tie with the bias in bf16
    o[6] = oracle.bf16_round(np.full(k, 1.0 + 2.0 ** -7, np.float32))
    for eps in [1e-6, 0.5]:
        got = gpu_residual(nq, h, o, bias, scale, gamma, eps, 16.0)
        check(got, h, o, bias, scale, gamma, eps, 16.0)


@pytest.mark.parametrize("form", ["bias", "none"])
@pytest.mark.parametrize("m,k", [(1, 512), (129, 2048), (64, 3584), (200, 4608), (300, 7168), (64, 8192)])
def test_dynamic(nq, m, k, form):
    print("residual_rms_dynamic", m, k, form, flush=True)
    h, o, bias, scale, gamma = case(m, k, 7 * m + k, form)
    got = gpu_residual(nq, h, o, bias, scale, gamma, 1e-6, None, dynamic=True)
    want = oracle.residual_rms_dynamic(h, o, bias, scale, gamma, 1e-6, want_y=True,
                                       scales_rows=oracle.padded_rows(m))
    assert u32(got["amax"]) == u32(want["amax"])
    assert_equal(u32(got["h"]), u32(want["h"]), "h")      # updated once, by the second pass
    assert_equal(u32(got["rstd"]), u32(want["rstd"]), "rstd")
    assert_equal(got["y"], want["y"], "y_out")
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], want["scales"], "scales")


# --------------------------------------------------------------------------------------
# the gated residual applied by the next block's RMSNorm + adaLN
# --------------------------------------------------------------------------------------

def fold_case(m, k, seed, form="bias", frames=3):
    h, o, bias, _, _ = case(m, k, seed, form)
    g = np.random.Generator(np.random.PCG64(seed + 1))
    gate = oracle.bf16_round((0.3 * g.standard_normal((frames, k))).astype(np.float32))
    w = oracle.bf16_round((1 + 0.1 * g.standard_normal(k)).astype(np.float32))
    table = oracle.bf16_round((0.1 * g.standard_normal((frames, 2, k))).astype(np.float32))
    idx = g.integers(0, frames, m).astype(np.int32)
    return h, o, bias, gate, w, table, idx


def gpu_fold(nq, h, o, bias, gate, w, table, idx, eps, amax, y=True, dynamic=False):
    m, k = h.shape
    hd = dev_f32(h)
    residual = None if o is None else (to_device(o), None if bias is None else to_device(bias), to_device(gate))
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    yd = torch.empty((m, k), dtype=torch.int16, device="cuda:0") if y else None
    args = (hd, to_device(w), to_device(table), torch.from_numpy(idx).to("cuda:0"), eps)
    if dynamic:
        codes, scales, amax_t = nq.residual_rms_adaln_nvfp4_dynamic(*args, residual=residual, rstd_out=rstd,
                                                                     y_out=yd, status_word=status)
    else:
        codes, scales = nq.residual_rms_adaln_nvfp4(*args, amax, residual=residual, rstd_out=rstd, y_out=yd,
                                                    status_word=status)
    torch.cuda.synchronize()
    out = dict(codes=to_host(codes), scales=to_host(scales), y=to_host(yd) if y else None,
               rstd=rstd.cpu().numpy(), h=hd.cpu().numpy(), status=int(status.cpu().numpy()[0]))
    if dynamic:
        out["amax"] = float(amax_t.cpu().numpy()[0])
    return out


def check_fold(got, want, m, k):
    assert_equal(u32(got["h"]), u32(want["h"]), "h")
    assert_equal(u32(got["rstd"]), u32(want["rstd"]), "rstd")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")
    assert_equal(got["codes"], want["codes"], "codes")
    assert got["status"] == want["status"]


@pytest.mark.parametrize("form", ["bias", "nobias", "none"])
@pytest.mark.parametrize("m,k", [(1, 512), (127, 1024), (129, 1536), (129, 2048), (64, 3584), (200, 4608),
                                 (64, 6144), (300, 7168), (257, 8192)])
def test_fold_shapes(nq, m, k, form):
    print("residual_rms_adaln", m, k, form, flush=True)
    h, o, bias, gate, w, table, idx = fold_case(m, k, 17 * m + k + len(form), form)
    for amax in [12.0, 2688.0]:
        got = gpu_fold(nq, h, o, bias, gate, w, table, idx, 1e-6, amax)
        want = oracle_residual_adaln(h, o, bias, gate, w, table, idx, 1e-6, amax)
        check_fold(got, want, m, k)
        assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, k), "scales")


def test_fold_out_of_range_frames(nq):
    m, k = 300, 2048
    h, o, bias, gate, w, table, idx = fold_case(m, k, 5)
    idx[[0, 33, 64, 299]] = [3, -1, 1 << 30, -(1 << 31)]
    got = gpu_fold(nq, h, o, bias, gate, w, table, idx, 1e-6, 10.0)
    want = oracle_residual_adaln(h, o, bias, gate, w, table, idx, 1e-6, 10.0)
    assert want["status"] == 1
    check_fold(got, want, m, k)
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, k), "scales")
    for r in (0, 33, 64, 299):
        assert_equal(u32(got["h"][r]), u32(h[r]), "h row %d kept" % r)


@pytest.mark.parametrize("form", ["bias", "none"])
@pytest.mark.parametrize("m,k", [(1, 512), (129, 2048), (64, 3584), (200, 4608), (300, 7168)])
def test_fold_dynamic(nq, m, k, form):
    print("residual_rms_adaln_dynamic", m, k, form, flush=True)
    h, o, bias, gate, w, table, idx = fold_case(m, k, 3 * m + k, form)
    idx[m // 2] = 7                                         # one row out of range: y = 0
    got = gpu_fold(nq, h, o, bias, gate, w, table, idx, 1e-6, None, dynamic=True)
    want = oracle.residual_rms_adaln_dynamic(h, o, bias, gate, w, table, idx, 1e-6, want_y=True,
                                             scales_rows=oracle.padded_rows(m))
    assert u32(got["amax"]) == u32(want["amax"])
    check_fold(got, want, m, k)
    assert_equal(got["scales"], want["scales"], "scales")


# --------------------------------------------------------------------------------------
# full size, the launch configuration the benchmark times
# --------------------------------------------------------------------------------------

def test_full_residual_rms_63240x7168(nq):
    wl = workloads.get("residual_rms_63240x7168")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    h, o = wl.h(), wl.o()
    bias, scale, gamma = wl.bias(), wl.residual_scale(), wl.gamma()
    got = gpu_residual(nq, h, o, bias, scale, gamma, wl.eps, amax, y=False)
    print("oracle", flush=True)
    check(got, h, o, bias, scale, gamma, wl.eps, amax)


def test_full_residual_adaln_63240x7168(nq):
    wl = workloads.get("residual_adaln_63240x7168")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    h, o = wl.h(), wl.o()
    args = (wl.bias(), wl.gate_table(), wl.weight(), wl.table(), wl.frame_idx())
    got = gpu_fold(nq, h, o, *args, wl.eps, amax, y=False)
    print("oracle", flush=True)
    want = oracle_residual_adaln(h, o, *args, wl.eps, amax, want_y=False)
    check_fold(got, want, wl.m, wl.k)
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], wl.m, wl.k), "scales")
