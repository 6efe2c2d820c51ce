"""GPU parity of the per-call (dynamic) amax forms, called through the C ABI, against the
CPU oracle: the device amax bit for bit against the oracle's max |y|, and codes and the
whole swizzled scale buffer byte for byte against the oracle at that amax.
"""
import numpy as np
import pytest

import oracle
import workloads
from util import first_mismatch, oracle_quantize_rows, scales_from_rows, to_device, to_host

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


def assert_equal(got, want, what):
    assert np.array_equal(got, want), "%s: %s" % (what, first_mismatch(got, want))


def f32_bits(v):
    return np.float32(v).view(np.uint32)


def amax_value(t):
    return float(t.cpu().numpy()[0])


# --------------------------------------------------------------------------------------
# standalone quantize
# --------------------------------------------------------------------------------------

def check_quantize_dynamic(nq, x, amax_buf=None):
    codes, scales, amax = nq.nvfp4_quantize_dynamic(to_device(x), amax_out=amax_buf)
    torch.cuda.synchronize()
    wc, ws, wa = oracle.nvfp4_quantize_dynamic(x)
    assert f32_bits(amax_value(amax)) == f32_bits(wa), (amax_value(amax), wa)
    assert_equal(to_host(codes), wc, "codes")
    assert_equal(to_host(scales), ws, "scales")


@pytest.mark.parametrize("m,k", [(1, 64), (129, 192), (300, 512), (257, 7168), (64, 19456)])
def test_quantize_dynamic_shapes(nq, m, k):
    print("quantize_dynamic", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(m * 3 + k))
    x = bf16(g.standard_normal((m, k)).astype(np.float32) * np.exp2(g.integers(-8, 8, (m, 1))).astype(np.float32))
    check_quantize_dynamic(nq, x)


@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_quantize_dynamic_max_in_any_workgroup(nq, where):
    # the maximum sits in one row; every other workgroup holds smaller values, so the
    # result is right only if every workgroup's maximum reaches the device amax
    m, k = 5000, 1024
    print("quantize_dynamic max at", where, flush=True)
    g = np.random.Generator(np.random.PCG64(11))
    x = bf16(g.uniform(-1, 1, (m, k)).astype(np.float32))
    r = {"first": 0, "middle": m // 2 + 17, "last": m - 1}[where]
    x[r, 333] = bf16(np.float32(-1000.0 - r))
    check_quantize_dynamic(nq, x)


@pytest.mark.parametrize("pattern", [0x0000, 0x8000, 0x0003])
def test_quantize_dynamic_zero_and_underflowing_tensors(nq, pattern):
    print("quantize_dynamic degenerate", hex(pattern), flush=True)
    x = np.full((200, 128), pattern, np.uint16)
    x[::7, ::3] = 0x8000
    check_quantize_dynamic(nq, x)


def test_quantize_dynamic_reuses_the_amax_buffer(nq):
    # the buffer is cleared by each call: a second call with smaller data gets its own amax
    print("quantize_dynamic reuse", flush=True)
    buf = torch.full((1,), 1e30, dtype=torch.float32, device="cuda:0")
    g = np.random.Generator(np.random.PCG64(12))
    check_quantize_dynamic(nq, bf16(g.standard_normal((300, 512)).astype(np.float32) * 50), buf)
    check_quantize_dynamic(nq, bf16(g.standard_normal((130, 256)).astype(np.float32) * 0.01), buf)


# --------------------------------------------------------------------------------------
# RMSNorm + adaLN and SwiGLU
# --------------------------------------------------------------------------------------

def gpu_rms_dynamic(nq, x, w, table, idx, eps, y=True):
    m, k = x.shape
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    y_out = torch.empty((m, k), dtype=torch.int16, device="cuda:0") if y else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    codes, scales, amax = nq.rms_adaln_nvfp4_dynamic(to_device(x), to_device(w), to_device(table),
                                                      torch.from_numpy(idx).to("cuda:0"), eps, rstd_out=rstd,
                                                      y_out=y_out, status_word=status)
    torch.cuda.synchronize()
    return dict(codes=to_host(codes), scales=to_host(scales), amax=amax_value(amax), rstd=rstd.cpu().numpy(),
                y=to_host(y_out) if y else None, status=int(status.cpu().numpy()[0]))


@pytest.mark.parametrize("m,k,frames,order", [(129, 1024, 4, "random"), (257, 7168, 31, "sorted"),
                                              (300, 2048, 5, "bad"), (70, 8704, 3, "random")])
def test_rms_adaln_dynamic(nq, m, k, frames, order):
    print("rms_adaln_dynamic", m, k, frames, order, flush=True)
    g = np.random.Generator(np.random.PCG64(m + 2 * k + frames))
    x = bf16(g.standard_normal((m, k)).astype(np.float32) * 2)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    if order == "sorted":
        idx = (np.arange(m) * frames // m).astype(np.int32)
    else:
        idx = g.integers(0, frames, m).astype(np.int32)
    if order == "bad":
        idx[[3, 100, 299]] = [frames, -1, 1 << 30]     # rows written as zeros, y = 0
    got = gpu_rms_dynamic(nq, x, w, table, idx, 1e-6)
    want = oracle.rms_adaln_dynamic(x, w, table, idx, 1e-6, want_y=True, scales_rows=oracle.padded_rows(m))
    assert f32_bits(got["amax"]) == f32_bits(want["amax"])
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], want["scales"], "scales")
    assert_equal(got["rstd"].view(np.uint32), want["rstd"].view(np.uint32), "rstd")
    assert_equal(got["y"], want["y"], "y_out")
    assert got["status"] == want["status"]


@pytest.mark.parametrize("m,k,hot", [(32845, 1024, 32840), (40000, 512, 39999), (40000, 512, 5)])
def test_rms_adaln_dynamic_last_round(nq, m, k, hot):
    """More than one round of units with a short last round (257 and 313 tiles on 256
    CUs): the rows after the full rounds run in 8-row units, in the amax pass as in the
    producer.  The row holding max |y| sits in those rows, or in the full rounds'."""
    print("rms_adaln_dynamic last round", m, k, hot, flush=True)
    frames = 5
    g = np.random.Generator(np.random.PCG64(m + k + hot))
    xf = g.standard_normal((m, k)).astype(np.float32)
    xf[hot] *= 8
    x = bf16(xf)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = g.integers(0, frames, m).astype(np.int32)
    got = gpu_rms_dynamic(nq, x, w, table, idx, 1e-6, y=False)
    want = oracle.rms_adaln_dynamic(x, w, table, idx, 1e-6, want_y=False, scales_rows=oracle.padded_rows(m))
    assert f32_bits(got["amax"]) == f32_bits(want["amax"])
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], want["scales"], "scales")
    assert_equal(got["rstd"].view(np.uint32), want["rstd"].view(np.uint32), "rstd")


@pytest.mark.parametrize("k", [512 * c for c in range(1, 17)])
def test_rms_adaln_dynamic_every_row_length(nq, k):
    """The amax pass and the producer at every row length they are instantiated for
    (k/512 = 1 .. 16), 2,100 rows over three frames."""
    m, frames = 2100, 3
    print("rms_adaln_dynamic", m, k, flush=True)
    g = np.random.Generator(np.random.PCG64(5 * k + 2))
    x = bf16(g.standard_normal((m, k)).astype(np.float32) * 2)
    w = bf16(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = (np.arange(m) * frames // m).astype(np.int32)
    got = gpu_rms_dynamic(nq, x, w, table, idx, 1e-6, y=False)
    want = oracle.rms_adaln_dynamic(x, w, table, idx, 1e-6, want_y=False, scales_rows=oracle.padded_rows(m))
    assert f32_bits(got["amax"]) == f32_bits(want["amax"])
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], want["scales"], "scales")


@pytest.mark.parametrize("m,f", [(1, 64), (129, 192), (130, 320), (300, 512), (129, 1792), (64, 19456)])
def test_swiglu_dynamic(nq, m, f):
    print("swiglu_dynamic", m, f, flush=True)
    g = np.random.Generator(np.random.PCG64(m * 5 + f))
    proj = bf16(g.standard_normal((m, 2 * f)).astype(np.float32) * 2)
    y_out = torch.empty((m, f), dtype=torch.int16, device="cuda:0")
    codes, scales, amax = nq.swiglu_nvfp4_dynamic(to_device(proj), y_out=y_out)
    torch.cuda.synchronize()
    want = oracle.swiglu_dynamic(proj[:, :f], proj[:, f:], want_y=True, scales_rows=oracle.padded_rows(m))
    assert f32_bits(amax_value(amax)) == f32_bits(want["amax"])
    assert_equal(to_host(codes), want["codes"], "codes")
    assert_equal(to_host(scales), want["scales"], "scales")
    assert_equal(to_host(y_out), want["y"], "y_out")


# --------------------------------------------------------------------------------------
# full-size workloads
# --------------------------------------------------------------------------------------

def test_full_quantize_dynamic_63240x7168(nq):
    wl = workloads.get("quantize_63240x7168")
    print("generating", wl.name, flush=True)
    x = wl.x()
    codes, scales, amax = nq.nvfp4_quantize_dynamic(to_device(x))
    torch.cuda.synchronize()
    print("oracle", flush=True)
    want_amax = oracle.max_abs(x)
    assert f32_bits(amax_value(amax)) == f32_bits(want_amax)
    assert oracle.dynamic_global_scale(want_amax) == oracle.global_scale(want_amax)
    want_c, want_sb = oracle_quantize_rows(x, want_amax)
    assert_equal(to_host(codes), want_c, "codes")
    assert_equal(to_host(scales), scales_from_rows(want_sb, wl.m, wl.k), "scales")


def test_full_rms_adaln_dynamic_63240x7168(nq):
    wl = workloads.get("rms_adaln_63240x7168")
    print("generating", wl.name, flush=True)
    x, w, table, idx = wl.x(), wl.weight(), wl.table(), wl.frame_idx()
    got = gpu_rms_dynamic(nq, x, w, table, idx, wl.eps, y=True)
    print("oracle", flush=True)
    # the oracle's y (whose max is the amax), then its quantizer at that amax; for finite
    # 2688 / amax this is the producer at the static amax
    from util import oracle_rms_adaln
    want = oracle_rms_adaln(x, w, table, idx, wl.eps, 1.0, want_y=True)
    assert_equal(got["y"], want["y"], "y_out")
    want_amax = oracle.max_abs(want["y"])
    assert f32_bits(got["amax"]) == f32_bits(want_amax)
    want_c, want_sb = oracle_quantize_rows(want["y"], want_amax)
    assert_equal(got["codes"], want_c, "codes")
    assert_equal(got["scales"], scales_from_rows(want_sb, wl.m, wl.k), "scales")
    assert_equal(got["rstd"].view(np.uint32), want["rstd"].view(np.uint32), "rstd")


def test_full_swiglu_dynamic_16384x19456(nq):
    wl = workloads.get("swiglu_16384x19456")
    print("generating", wl.name, flush=True)
    proj = wl.x()
    f = wl.k
    y_out = torch.empty((wl.m, f), dtype=torch.int16, device="cuda:0")
    codes, scales, amax = nq.swiglu_nvfp4_dynamic(to_device(proj), y_out=y_out)
    torch.cuda.synchronize()
    print("oracle", flush=True)
    from util import oracle_swiglu
    want = oracle_swiglu(proj[:, :f], proj[:, f:], 1.0, want_y=True)
    y = to_host(y_out)
    assert_equal(y, want["y"], "y_out")
    want_amax = oracle.max_abs(want["y"])
    assert f32_bits(amax_value(amax)) == f32_bits(want_amax)
    want_c, want_sb = oracle_quantize_rows(want["y"], want_amax)
    assert_equal(to_host(codes), want_c, "codes")
    assert_equal(to_host(scales), scales_from_rows(want_sb, wl.m, f), "scales")
