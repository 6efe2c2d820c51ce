"""GPU parity: the HIP kernels, called through the C ABI (Python binding), against the
CPU oracle on the same seeded inputs.  Codes, scale bytes (the whole swizzled buffer,
padding rows included), bf16 side outputs are compared bit for bit; fp32 rstd at 0 ulp.
"""
import hashlib

import numpy as np
import pytest

import oracle
import workloads
from util import (first_mismatch, gather_scales, oracle_quantize_rows, oracle_rms_adaln, oracle_swiglu,
                  scales_from_rows, to_device, to_host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_activation_quantization_amd as mod
    return mod


def bf16(a):
    return oracle.bf16_round(np.asarray(a, np.float32))


def rand_bf16(shape, seed, scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.standard_normal(shape).astype(np.float32) * scale
    return bf16(a)


def assert_equal(got, want, what):
    assert np.array_equal(got, want), "%s: %s" % (what, first_mismatch(got, want))


# --------------------------------------------------------------------------------------
# the standalone quantizer
# --------------------------------------------------------------------------------------

def gpu_quantize(nq, x_u16, amax):
    xd = to_device(x_u16)
    codes, scales = nq.nvfp4_quantize(xd, amax)
    torch.cuda.synchronize()
    return to_host(codes), to_host(scales)


@pytest.mark.parametrize("m,k", [(1, 64), (127, 64), (128, 128), (129, 192), (300, 512), (257, 7168),
                                 (1000, 2048), (64, 19456)])
def test_quantize_shapes(nq, m, k):
    print("quantize", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(m * 7 + k))
    x = bf16(g.standard_normal((m, k)).astype(np.float32) * np.exp2(g.integers(-10, 10, (m, 1))).astype(np.float32))
    for amax in [3.0, 2688.0, 1e-3]:
        codes, scales = gpu_quantize(nq, x, amax)
        want_c, want_s = oracle.nvfp4_quantize(x, amax)
        assert_equal(codes, want_c, "codes amax=%g" % amax)
        assert_equal(scales, want_s, "scales amax=%g" % amax)


@pytest.mark.parametrize("slots", range(1, 17))
def test_quantize_every_slot_count(nq, slots):
    """Every row-piece instantiation (slots 16-byte chunks per lane, 1 .. 16): rows whose
    last slot is full (k = 512 slots) and rows whose last slot holds one 64-column group
    (k = 512 (slots - 1) + 64), over a ragged row tile."""
    m = 300
    for k in sorted({512 * slots, 512 * (slots - 1) + 64}):
        print("quantize", m, k, flush=True)
        g = np.random.Generator(np.random.PCG64(k + 11))
        x = bf16(g.standard_normal((m, k)).astype(np.float32))
        codes, scales = gpu_quantize(nq, x, 5.0)
        want_c, want_s = oracle.nvfp4_quantize(x, 5.0)
        assert_equal(codes, want_c, "codes k=%d" % k)
        assert_equal(scales, want_s, "scales k=%d" % k)


FIXED15 = np.array([0.75, -1.3125, 0.2, 2.5, -0.046875, 1.0, -3.0, 0.5, 1.75, -0.625, 0.0, 4.0,
                    -2.25, 0.09375, 1.5], np.float32)


def sweep_rows(k):
    """Rows of k values: row i sweeps finite bf16 pattern i; block b < 16 holds the fixed 15
    values with the swept one inserted at position b; later blocks hold the fixed values + 1."""
    pats = np.arange(65536, dtype=np.uint32)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)      # 65,280 finite patterns
    fixed = bf16(FIXED15)
    rows = np.empty((len(pats), k), np.uint16)
    for b in range(k // 16):
        blk = np.insert(fixed, b % 16, 0)
        rows[:, 16 * b:16 * b + 16] = blk[None, :]
        if b < 16:
            rows[:, 16 * b + b] = pats
        else:
            rows[:, 16 * b + b % 16] = bf16([1.0])[0]
    return rows


@pytest.mark.parametrize("amax", [4.0, 2688.0])
def test_quantize_every_bf16_value_at_every_position(nq, amax):
    x = sweep_rows(256)
    codes, scales = gpu_quantize(nq, x, amax)
    want_c, want_s = oracle.nvfp4_quantize(x, amax)
    assert_equal(codes, want_c, "codes")
    assert_equal(scales, want_s, "scales")


def test_quantize_empty_and_errors(nq):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    codes, scales = nq.nvfp4_quantize(x, 1.0)
    assert codes.shape == (0, 32) and scales.shape == (0, 4)
    with pytest.raises(nq.NVFP4Error) as e:
        nq.nvfp4_quantize(torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda:0"), 1.0)
    assert e.value.status == 2
    with pytest.raises(nq.NVFP4Error) as e:
        nq.nvfp4_quantize(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda:0"), float("nan"))
    assert e.value.status == 4


# --------------------------------------------------------------------------------------
# RMSNorm + adaLN
# --------------------------------------------------------------------------------------

def gpu_rms(nq, x, w, table, idx, eps, amax, y=True):
    m, k = x.shape
    xd, wd, td = to_device(x), to_device(w), to_device(table)
    idd = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to("cuda:0")
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    yd = torch.empty((m, k), dtype=torch.int16, device="cuda:0") if y else None
    st = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    codes, scales = nq.rms_adaln_nvfp4(xd, wd, td, idd, eps, amax, rstd_out=rstd, y_out=yd, status_word=st)
    torch.cuda.synchronize()
    return dict(codes=to_host(codes), scales=to_host(scales), rstd=rstd.cpu().numpy(),
                y=to_host(yd) if y else None, status=int(st.cpu().item()))


def check_rms(got, x, w, table, idx, eps, amax):
    m, k = x.shape
    want = oracle_rms_adaln(x, w, table, idx, eps, amax)
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, k), "scales")
    assert_equal(got["rstd"].view(np.uint32), want["rstd"].view(np.uint32), "rstd")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")
    assert got["status"] == want["status"]


@pytest.mark.parametrize("m,k,frames,order", [(1, 512, 1, "sorted"), (127, 512, 3, "sorted"),
                                              (129, 1024, 4, "random"), (300, 2048, 5, "sorted"),
                                              (257, 7168, 31, "sorted"), (200, 7168, 7, "random"),
                                              (150, 8192, 2, "sorted"), (70, 8704, 3, "random")])
def test_rms_adaln_shapes(nq, m, k, frames, order):
    print("rms_adaln", m, k, frames, order, flush=True)
    g = np.random.Generator(np.random.PCG64(m + k + frames))
    x = rand_bf16((m, k), m + 1, 2.0)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    if order == "sorted":
        idx = (np.arange(m) * frames // m).astype(np.int32)
    else:
        idx = g.integers(0, frames, m).astype(np.int32)
    for amax in [8.0, 2688.0]:
        got = gpu_rms(nq, x, w, table, idx, 1e-6, amax)
        check_rms(got, x, w, table, idx, 1e-6, amax)


@pytest.mark.parametrize("k", [512 * c for c in range(1, 17)])
def test_rms_adaln_every_row_length(nq, k):
    """Every row length the kernel is instantiated for (k/512 = 1 .. 16 chunks per lane)
    over 2,100 rows: 17 tiles, fewer than the CUs, so the rows run in 16-row units (two rows
    per wavefront, the next row's prefetch between them) with direct scale stores."""
    m, frames = 2100, 3
    print("rms_adaln", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(7 * k + 1))
    x = rand_bf16((m, k), k + 3, 2.0)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = (np.arange(m) * frames // m).astype(np.int32)
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 8.0)
    check_rms(got, x, w, table, idx, 1e-6, 8.0)


@pytest.fixture(scope="module")
def tile_rows():
    """32,845 rows of 8192 bf16 columns: 257 tiles of 128 rows (77 in the last), more than
    the device's 256 CUs, so RMSNorm + adaLN runs the first 256 tiles in full rounds of its
    units of 4 S rows and the last, lone tile in 8-row units (16 of them, on 16
    workgroups).  Each k takes the first k columns."""
    return rand_bf16((32845, 8192), 4242, 2.0)


@pytest.mark.parametrize("k", [512 * c for c in range(1, 17)])
def test_rms_adaln_tile_path_every_row_length(nq, tile_rows, k):
    """The tile path at every row length (the next row's prefetch across rows and units,
    frame changes inside tiles) and the 8-row units after the full rounds (the ragged last
    tile, its zero padding rows and their scale bytes as 4-byte pieces)."""
    m, frames = tile_rows.shape[0], 5
    print("rms_adaln tiles", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(11 * k + 5))
    x = np.ascontiguousarray(tile_rows[:, :k])
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = (np.arange(m) * frames // m).astype(np.int32)
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 16.0)
    check_rms(got, x, w, table, idx, 1e-6, 16.0)


@pytest.mark.parametrize("m", [9, 12, 129, 2047, 4089, 8189, 16379, 16512, 24583, 28000])
def test_rms_adaln_unit_sizes(nq, m):
    """Row counts that take each unit of a short tensor on 256 CUs: 8 rows (12, 129, 2047,
    16512), 16 (4089), 32 (8189), 64 (16379), each but the first with a ragged last unit,
    and 128-row tiles where smaller units would not unload the busiest CU (9, 24583,
    28000); unsorted frames, an out-of-range frame index and y_out."""
    k, frames = 1024, 6
    print("rms_adaln units", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(m + 17))
    x = rand_bf16((m, k), m + 19, 2.0)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = g.integers(0, frames, m).astype(np.int32)
    idx[m // 2] = frames
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 8.0)
    assert got["status"] == 1
    check_rms(got, x, w, table, idx, 1e-6, 8.0)


@pytest.mark.parametrize("m,k,rows_per_frame", [(40000, 1024, 97), (70000, 2048, 41), (33000, 8192, 13)])
def test_rms_adaln_tail_units(nq, m, k, rows_per_frame):
    """Tensors whose last round of units is short on 256 CUs, so the rows after the full
    rounds run in 8-row units (313, 547 and 258 tiles): frames change every few rows, so
    units straddle frame boundaries (restaged and unstaged rows), with out-of-range frame
    indices in the tail, the ragged last tile, rstd_out and y_out."""
    print("rms_adaln tail units", m, k, rows_per_frame, flush=True)
    frames = (m + rows_per_frame - 1) // rows_per_frame
    g = np.random.Generator(np.random.PCG64(m + k))
    x = rand_bf16((m, k), m + 3, 2.0)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = (np.arange(m) // rows_per_frame).astype(np.int32)
    idx[[m - 1000, m - 333, m - 2]] = [-1, frames, frames + 7]
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 8.0)
    assert got["status"] == 1
    check_rms(got, x, w, table, idx, 1e-6, 8.0)


def test_rms_adaln_tiny_workload(nq):
    wl = workloads.get("rms_adaln_256x2048")
    amax = workloads.calibration_amax(wl.name)
    x, w, table, idx = wl.x(), wl.weight(), wl.table(), wl.frame_idx()
    got = gpu_rms(nq, x, w, table, idx, wl.eps, amax)
    check_rms(got, x, w, table, idx, wl.eps, amax)


def test_rms_adaln_every_bf16_value_at_every_position(nq):
    x = sweep_rows(512)
    m, k = x.shape
    g = np.random.Generator(np.random.PCG64(77))
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((3, 2, k)).astype(np.float32))
    idx = (np.arange(m) % 3).astype(np.int32)
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 6.0)
    check_rms(got, x, w, table, idx, 1e-6, 6.0)


def test_rms_adaln_frame_index_out_of_range(nq):
    m, k, frames = 40, 1024, 3
    x = rand_bf16((m, k), 5)
    g = np.random.Generator(np.random.PCG64(6))
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = (np.arange(m) % frames).astype(np.int32)
    idx[[3, 17, 39]] = [-1, 3, 1 << 30]
    got = gpu_rms(nq, x, w, table, idx, 1e-6, 4.0)
    assert got["status"] == 1
    assert not got["codes"][[3, 17, 39]].any() and not got["y"][[3, 17, 39]].any()
    check_rms(got, x, w, table, idx, 1e-6, 4.0)


def test_rms_adaln_zero_rows_and_eps(nq):
    m, k = 130, 512
    x = rand_bf16((m, k), 8)
    x[5] = 0
    x[129] = 0
    w = bf16(np.ones(k, np.float32))
    table = np.zeros((1, 2, k), np.uint16)
    idx = np.zeros(m, np.int32)
    for eps in [1e-6, 0.5]:
        got = gpu_rms(nq, x, w, table, idx, eps, 4.0)
        check_rms(got, x, w, table, idx, eps, 4.0)


# --------------------------------------------------------------------------------------
# SwiGLU
# --------------------------------------------------------------------------------------

def gpu_swiglu(nq, proj, amax, y=True):
    m, two_f = proj.shape
    f = two_f // 2
    pd = to_device(proj)
    yd = torch.empty((m, f), dtype=torch.int16, device="cuda:0") if y else None
    codes, scales = nq.swiglu_nvfp4(pd, amax, y_out=yd)
    torch.cuda.synchronize()
    return dict(codes=to_host(codes), scales=to_host(scales), y=to_host(yd) if y else None)


def check_swiglu(got, proj, amax):
    m, two_f = proj.shape
    f = two_f // 2
    want = oracle_swiglu(proj[:, :f], proj[:, f:], amax)
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, f), "scales")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")


@pytest.mark.parametrize("m,f", [(1, 64), (127, 128), (129, 192), (300, 512), (64, 19456), (257, 1024),
                                 (300, 1088), (131, 2624), (130, 320), (257, 960), (129, 1792)])
def test_swiglu_shapes(nq, m, f):
    print("swiglu", m, f, flush=True)
    proj = rand_bf16((m, 2 * f), m + f, 2.0)
    for amax in [16.0, 2688.0]:
        check_swiglu(gpu_swiglu(nq, proj, amax), proj, amax)


def test_swiglu_every_gate_and_up_value(nq):
    sweep = sweep_rows(256)
    g = np.random.Generator(np.random.PCG64(9))
    other = bf16(g.standard_normal(sweep.shape).astype(np.float32))
    for name, proj in [("gate", np.concatenate([other, sweep], axis=1)),
                       ("up", np.concatenate([sweep, other], axis=1))]:
        print("swiglu sweep", name, flush=True)
        check_swiglu(gpu_swiglu(nq, proj, 8.0), proj, 8.0)


def test_swiglu_separate_views_with_row_stride(nq):
    m, f = 100, 256
    big = rand_bf16((m, 3 * f), 10)           # rows of 3f: up at column 0, gate at column 2f
    bd = to_device(big)
    up, gate = bd[:, :f], bd[:, 2 * f:]
    codes, scales = nq.swiglu_nvfp4(up, 6.0, gate=gate)
    torch.cuda.synchronize()
    want = oracle_swiglu(big[:, :f], big[:, 2 * f:], 6.0, want_y=False)
    assert_equal(to_host(codes), want["codes"], "codes")
    assert_equal(to_host(scales), scales_from_rows(want["scale_bytes"], m, f), "scales")


# --------------------------------------------------------------------------------------
# full-size workloads, the launch configuration the benchmark times
# --------------------------------------------------------------------------------------

def test_full_quantize_63240x7168(nq):
    wl = workloads.get("quantize_63240x7168")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    x = wl.x()
    codes, scales = gpu_quantize(nq, x, amax)
    print("oracle", flush=True)
    want_c, want_sb = oracle_quantize_rows(x, amax)
    assert_equal(codes, want_c, "codes")
    assert_equal(scales, scales_from_rows(want_sb, wl.m, wl.k), "scales")


def test_full_rms_adaln_63240x7168(nq):
    wl = workloads.get("rms_adaln_63240x7168")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    x, w, table, idx = wl.x(), wl.weight(), wl.table(), wl.frame_idx()
    got = gpu_rms(nq, x, w, table, idx, wl.eps, amax, y=False)
    print("oracle", flush=True)
    want = oracle_rms_adaln(x, w, table, idx, wl.eps, amax, want_y=False)
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], wl.m, wl.k), "scales")
    assert_equal(got["rstd"].view(np.uint32), want["rstd"].view(np.uint32), "rstd")


def test_full_swiglu_16384x19456(nq):
    wl = workloads.get("swiglu_16384x19456")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    proj = wl.x()
    got = gpu_swiglu(nq, proj, amax, y=False)
    print("oracle", flush=True)
    check_swiglu(got, proj, amax)


def test_full_rms_adaln_300000x7168_sampled(nq):
    """2.15e9 elements (past 2^31): first/last 4096 rows, 8192 seeded random rows and
    every padding row checked against the oracle."""
    wl = workloads.get("rms_adaln_300000x7168")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    x = np.empty((wl.m, wl.k), np.uint16)
    wl.x(out=x)
    w, table, idx = wl.weight(), wl.table(), wl.frame_idx()
    xd = to_device(x)
    del x
    m, k = wl.m, wl.k
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    codes, scales = nq.rms_adaln_nvfp4(xd, to_device(w), to_device(table),
                                       torch.from_numpy(idx).to("cuda:0"), wl.eps, amax, rstd_out=rstd)
    torch.cuda.synchronize()
    del xd
    rows = wl.sample_rows()
    print("oracle on %d rows" % len(rows), flush=True)
    xs = wl.x_rows(rows)
    want = oracle_rms_adaln(xs, w, table, idx[rows], wl.eps, amax, row_ids=rows, want_y=False)
    rows_t = torch.from_numpy(rows).to("cuda:0")
    assert_equal(to_host(codes.index_select(0, rows_t)), want["codes"], "codes")
    assert_equal(rstd.index_select(0, rows_t).cpu().numpy().view(np.uint32), want["rstd"].view(np.uint32), "rstd")
    sc = to_host(scales)
    assert_equal(gather_scales(sc, rows, k), want["scale_bytes"], "scales")
    pad_rows = np.arange(m, oracle.padded_rows(m))
    assert not gather_scales(sc, pad_rows, k).any()


# --------------------------------------------------------------------------------------
# determinism without per-call synchronisation
# --------------------------------------------------------------------------------------

def test_repeated_runs_hash_identically(nq):
    wl = workloads.get("rms_adaln_63240x7168")
    m = 8192
    x = wl.x_rows(np.arange(m))
    w, table, idx = wl.weight(), wl.table(), wl.frame_idx(np.arange(m))
    xd, wd, td = to_device(x), to_device(w), to_device(table)
    idd = torch.from_numpy(idx).to("cuda:0")
    outs = []
    for _ in range(5):
        outs.append(nq.rms_adaln_nvfp4(xd, wd, td, idd, wl.eps, 60.0))
    torch.cuda.synchronize()
    hashes = {hashlib.sha256(to_host(c).tobytes() + to_host(s).tobytes()).hexdigest() for c, s in outs}
    assert len(hashes) == 1
