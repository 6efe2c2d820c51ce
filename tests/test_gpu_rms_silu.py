"""GPU parity of the channels-last RMSNorm + SiLU -> NVFP4 producer (fp16), static and
per-call amax, through the C ABI, against the CPU oracle on the same seeded inputs: codes,
plain-order scale bytes and the fp16 side output bit for bit, rstd at 0 ulp."""
import numpy as np
import pytest

import oracle
import workloads
from util import first_mismatch, oracle_rms_silu, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def case(rows, c, seed, scale=2.0):
    g = np.random.Generator(np.random.PCG64(seed))
    x = oracle.f16_round((g.standard_normal((rows, c)) * scale).astype(np.float32))
    gamma = oracle.f16_round((1 + 0.3 * g.standard_normal(c)).astype(np.float32))
    return x, gamma


def gpu(nq, x, gamma, eps, amax, y=True, dynamic=False):
    rows, c = x.shape
    xd, gd = to_device(x), to_device(gamma)
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda:0")
    yd = torch.empty((rows, c), dtype=torch.int16, device="cuda:0") if y else None
    if dynamic:
        codes, scales, amax_t = nq.rms_silu_nvfp4_dynamic(xd, gd, eps, rstd_out=rstd, y_out=yd)
    else:
        codes, scales = nq.rms_silu_nvfp4(xd, gd, eps, amax, rstd_out=rstd, y_out=yd)
    torch.cuda.synchronize()
    out = dict(codes=to_host(codes), scales=to_host(scales), rstd=rstd.cpu().numpy(), y=to_host(yd) if y else None)
    if dynamic:
        out["amax"] = float(amax_t.cpu().numpy()[0])
    return out


def check(got, want):
    assert_equal(u32(got["rstd"]), u32(want["rstd"]), "rstd")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], want["scale_bytes"], "scales")


# c/8 chunks per row: 2 .. 64 on P lanes with one slot each (16, 32, 64, 128, 256, 512),
# on P = 2, 4, 8, 16 lanes with three slots (48, 96, 192, 384), and padded to the next
# power of two with repeated chunks (80, 160, 320, 496)
@pytest.mark.parametrize("c", [16, 32, 48, 64, 80, 96, 128, 160, 192, 256, 320, 384, 496, 512])
@pytest.mark.parametrize("rows", [1, 3, 257, 4099])
def test_shapes(nq, rows, c):
    print("rms_silu", rows, c, flush=True)
    x, gamma = case(rows, c, 31 * rows + c)
    for amax in [6.0, 2688.0]:
        check(gpu(nq, x, gamma, 1e-6, amax), oracle_rms_silu(x, gamma, 1e-6, amax))


def test_every_fp16_value_through_the_chain(nq):
    """Every finite fp16 pattern at one channel of a 192-channel row (the other channels
    random): all SiLU table entries reachable from the pattern set, and zero, subnormal and
    huge inputs through the statistic."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 10) & 0x1F) != 0x1F]
    c = 192
    g = np.random.Generator(np.random.PCG64(3))
    x = oracle.f16_round(g.standard_normal((len(pats), c)).astype(np.float32))
    x[:, 7] = pats
    gamma = oracle.f16_round((1 + 0.3 * g.standard_normal(c)).astype(np.float32))
    for eps in [1e-6, 0.25]:
        check(gpu(nq, x, gamma, eps, 16.0), oracle_rms_silu(x, gamma, eps, 16.0))


def test_gamma_reaches_every_silu_entry(nq):
    """x = 1 in every channel gives rstd = 1/sqrt(1 + eps) ~ 1, so a = fp16(fp16(rstd) *
    gamma): sweeping gamma over every finite fp16 value (192 per row) runs the product and
    the table over nearly all patterns."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    pats = pats[((pats >> 10) & 0x1F) != 0x1F]
    c = 192
    n = len(pats) // c
    x = oracle.f16_round(np.ones((1, c), np.float32))
    for i in range(0, n, 32):
        print("gamma sweep", i, flush=True)
        rows = []
        for j in range(i, min(n, i + 32)):
            gamma = pats[j * c:(j + 1) * c]
            got = gpu(nq, x, gamma, 0.0, 64.0)
            rows.append((got, oracle.rms_silu_rows(x, gamma, 0.0, 64.0, want_y=True)))
        for got, want in rows:
            check(got, want)


def test_channels_last_view(nq):
    """A 5-d channels-last tensor [frames, h, w, c]: rows are every leading index."""
    x, gamma = case(2 * 7 * 9, 96, 8)
    xd = to_device(x).view(2, 7, 9, 96)
    codes, scales = nq.rms_silu_nvfp4(xd, to_device(gamma), 1e-6, 5.0)
    torch.cuda.synchronize()
    want = oracle.rms_silu_rows(x, gamma, 1e-6, 5.0)
    assert_equal(to_host(codes), want["codes"], "codes")
    assert_equal(to_host(scales), want["scale_bytes"], "scales")


@pytest.mark.parametrize("c", [64, 80, 96, 192, 384])
@pytest.mark.parametrize("rows", [1, 300, 5000])
def test_dynamic(nq, rows, c):
    x, gamma = case(rows, c, 7 * rows + c, scale=3.0)
    got = gpu(nq, x, gamma, 1e-6, None, dynamic=True)
    want = oracle.rms_silu_dynamic(x, gamma, 1e-6, want_y=True)
    assert u32(got["amax"]) == u32(want["amax"])
    check(got, want)


@pytest.mark.parametrize("pattern", [0x0000, 0x8000])
def test_signed_zero_rows(nq, pattern):
    """Rows of +0 or of -0 only: the statistic is 0 (rstd = 1/sqrt(eps)), y is the signed
    zero that SiLU keeps, the call's own amax is 0 (global scale 0), and every code carries
    y's sign alone; the static form under a positive amax gives the same codes."""
    rows, c = 300, 192
    print("rms_silu zero rows", hex(pattern), flush=True)
    _, gamma = case(rows, c, 11)
    x = np.full((rows, c), pattern, np.uint16)
    got = gpu(nq, x, gamma, 1e-6, None, dynamic=True)
    want = oracle.rms_silu_dynamic(x, gamma, 1e-6, want_y=True)
    assert want["amax"] == 0.0 and u32(got["amax"]) == 0
    check(got, want)
    assert set(np.unique(want["codes"])) <= {0x00, 0x08, 0x80, 0x88}
    check(gpu(nq, x, gamma, 1e-6, 6.0), oracle_rms_silu(x, gamma, 1e-6, 6.0))


def test_full_rms_silu_16x120x216x192_dynamic(nq):
    wl = workloads.get("rms_silu_16x120x216x192")
    print("generating", wl.name, flush=True)
    x, gamma = wl.x(), wl.weight()
    got = gpu(nq, x, gamma, wl.eps, None, y=False, dynamic=True)
    print("oracle", flush=True)
    want = oracle.rms_silu_dynamic(x, gamma, wl.eps, want_y=False)
    assert u32(got["amax"]) == u32(want["amax"])
    check(got, want)


def test_full_rms_silu_16x120x216x192(nq):
    wl = workloads.get("rms_silu_16x120x216x192")
    amax = workloads.calibration_amax(wl.name)
    print("generating", wl.name, flush=True)
    x, gamma = wl.x(), wl.weight()
    got = gpu(nq, x, gamma, wl.eps, amax, y=False)
    print("oracle", flush=True)
    check(got, oracle_rms_silu(x, gamma, wl.eps, amax, want_y=False))
