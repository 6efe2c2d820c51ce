"""GPU parity of the LayerNorm (fp32 statistics) + adaLN -> per-tensor FP8 E4M3 producer
(fp16 rows), static and per-call scale, through the C ABI, against the CPU oracle on the
same seeded inputs: codes bit for bit, mean, rstd and the fp32 side output y at 0 ulp."""
import numpy as np
import pytest

import oracle
import workloads
from util import first_mismatch, oracle_ln_fp8, oracle_ln_fp8_amax, to_device, to_host

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


def case(m, k, seed, xscale=2.0, mscale=0.1):
    g = np.random.Generator(np.random.PCG64(seed))
    x = oracle.f16_round((g.standard_normal((m, k)) * xscale + 0.3 * g.standard_normal((m, 1))).astype(np.float32))
    sc = (mscale * g.standard_normal(k)).astype(np.float32)
    sh = (mscale * g.standard_normal(k)).astype(np.float32)
    return x, sc, sh


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def gpu(nq, x, sc, sh, eps, act_scale, y=True, dynamic=False):
    m, k = x.shape
    xd = to_device(x)
    mean = torch.empty(m, dtype=torch.float32, device="cuda:0")
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    yd = torch.empty((m, k), dtype=torch.float32, device="cuda:0") if y else None
    if dynamic:
        codes, act = nq.ln_adaln_fp8_dynamic(xd, f32_dev(sc), f32_dev(sh), eps, mean_out=mean, rstd_out=rstd,
                                             y_out=yd)
    else:
        codes = nq.ln_adaln_fp8(xd, f32_dev(sc), f32_dev(sh), eps, act_scale, mean_out=mean, rstd_out=rstd, y_out=yd)
    torch.cuda.synchronize()
    out = dict(codes=to_host(codes), mean=mean.cpu().numpy(), rstd=rstd.cpu().numpy(),
               y=yd.cpu().numpy() if y else None)
    if dynamic:
        out["act_scale"] = act.cpu().numpy()[:1]
    return out


def check(got, want):
    assert_equal(u32(got["mean"]), u32(want["mean"]), "mean")
    assert_equal(u32(got["rstd"]), u32(want["rstd"]), "rstd")
    if got["y"] is not None and want["y"] is not None:
        assert_equal(u32(got["y"]), u32(want["y"]), "y_out")
    assert_equal(got["codes"], want["codes"], "codes")


@pytest.mark.parametrize("k", [512, 1024, 3072, 4608, 7168, 8192])
@pytest.mark.parametrize("m", [1, 7, 2051, 4609])
def test_shapes(nq, m, k):
    """Row counts below, at and past one row per wavefront of the persistent grid (2048
    wavefronts on 256 CUs), so the prefetch of a wavefront's next row and the tail run."""
    print("ln_fp8", m, k, flush=True)
    x, sc, sh = case(m, k, 13 * m + k)
    for act in [0.01, 0.125]:
        inv = oracle.fp8_inverse_scale(act)
        check(gpu(nq, x, sc, sh, 1e-6, act), oracle_ln_fp8(x, sc, sh, 1e-6, inv))


@pytest.mark.parametrize("k", [512 * c for c in range(1, 17) if c not in (1, 2, 6, 9, 14, 16)])
def test_every_row_length(nq, k):
    """The row lengths test_shapes leaves out, so that every instantiation (k/512 = 1 .. 16
    chunks per lane; LDS planes past 64 KiB from 9 up) runs over 2,051 rows."""
    m = 2051
    print("ln_fp8", m, k, flush=True)
    x, sc, sh = case(m, k, 17 * k + 1)
    inv = oracle.fp8_inverse_scale(0.05)
    check(gpu(nq, x, sc, sh, 1e-6, 0.05), oracle_ln_fp8(x, sc, sh, 1e-6, inv))


@pytest.mark.parametrize("k", [512 * c for c in range(1, 17)])
def test_dynamic_every_row_length(nq, k):
    """The per-call form (amax pass, scale kernel, producer) at every row length, 2,051 rows."""
    m = 2051
    print("ln_fp8 dynamic", m, k, flush=True)
    x, sc, sh = case(m, k, 19 * k + 5, xscale=3.0, mscale=0.3)
    got = gpu(nq, x, sc, sh, 1e-6, None, dynamic=True)
    want = oracle.ln_adaln_fp8_dynamic(x, sc, sh, 1e-6)
    assert u32(got["act_scale"])[0] == u32(np.float32(want["act_scale"]))
    check(got, want)


def test_saturation_rounding_and_signed_zero(nq):
    """act_scale small enough that most |y / act_scale| pass 448 (saturated codes), large
    enough that they underflow (signed zeros), and adaLN columns with scale = -1 and
    shift = -0, where y is a zero whose sign follows (x - mean)."""
    m, k = 300, 2048
    x, sc, sh = case(m, k, 5)
    sc[::7] = -1.0
    sh[::7] = -0.0
    sh[3::7] = 0.0
    for act in [1e-3, 3e-2, 1.0, 1e6, 1e30]:
        want = oracle_ln_fp8(x, sc, sh, 1e-6, oracle.fp8_inverse_scale(act))
        check(gpu(nq, x, sc, sh, 1e-6, act), want)
    assert (want["codes"][:, ::7] == 0x80).any() and (want["codes"][:, ::7] == 0).any()


def test_constant_and_extreme_rows(nq):
    """Constant rows (variance 0: rstd = 1 / sqrt(eps), y = shift), rows of the largest fp16
    magnitudes, subnormal rows and rows with one outlier."""
    k = 4096
    g = np.random.Generator(np.random.PCG64(21))
    rows = [np.full(k, 1.5), np.full(k, -65504.0), np.zeros(k), np.full(k, 6e-8),
            np.where(g.random(k) < 0.5, 65504.0, -65504.0), g.standard_normal(k) * 1e-6,
            np.concatenate([[30000.0], g.standard_normal(k - 1)])]
    x = oracle.f16_round(np.stack(rows).astype(np.float32))
    sc = (0.2 * g.standard_normal(k)).astype(np.float32)
    sh = (0.2 * g.standard_normal(k)).astype(np.float32)
    for eps in [1e-6, 0.5]:
        check(gpu(nq, x, sc, sh, eps, 0.02), oracle_ln_fp8(x, sc, sh, eps, oracle.fp8_inverse_scale(0.02)))


@pytest.mark.parametrize("k", [1024, 7168])
@pytest.mark.parametrize("m", [1, 333, 5000])
def test_dynamic(nq, m, k):
    x, sc, sh = case(m, k, 3 * m + k, xscale=3.0, mscale=0.3)
    got = gpu(nq, x, sc, sh, 1e-6, None, dynamic=True)
    want = oracle.ln_adaln_fp8_dynamic(x, sc, sh, 1e-6)
    assert u32(got["act_scale"])[0] == u32(np.float32(want["act_scale"]))
    check(got, want)


def test_dynamic_all_zero_output(nq):
    """Every column with scale = -1 and shift = -0: y is a signed zero everywhere, the
    per-call scale is 0, and every code is the sign of y."""
    m, k = 100, 1536
    x, _, _ = case(m, k, 9)
    sc = np.full(k, -1.0, np.float32)
    sh = np.full(k, -0.0, np.float32)
    got = gpu(nq, x, sc, sh, 1e-6, None, dynamic=True)
    want = oracle.ln_adaln_fp8_dynamic(x, sc, sh, 1e-6)
    assert want["act_scale"] == 0.0 and u32(got["act_scale"])[0] == 0
    check(got, want)
    assert set(np.unique(want["codes"])) <= {0x00, 0x80}


def test_full_ln_fp8_63240x7168(nq):
    wl = workloads.get("ln_fp8_63240x7168")
    act = workloads.fp8_act_scale(wl.name)
    print("generating", wl.name, flush=True)
    x = wl.x()
    sc, sh = wl.modulation()
    got = gpu(nq, x, sc, sh, wl.eps, act, y=False)
    print("oracle", flush=True)
    check(got, oracle_ln_fp8(x, sc, sh, wl.eps, oracle.fp8_inverse_scale(act), want_y=False))


def test_full_ln_fp8_63240x7168_dynamic(nq):
    wl = workloads.get("ln_fp8_63240x7168")
    print("generating", wl.name, flush=True)
    x = wl.x()
    sc, sh = wl.modulation()
    got = gpu(nq, x, sc, sh, wl.eps, None, y=False, dynamic=True)
    print("oracle", flush=True)
    act = oracle.fp8_dynamic_scale(oracle_ln_fp8_amax(x, sc, sh, wl.eps))
    assert u32(got["act_scale"])[0] == u32(np.float32(act))
    check(got, oracle_ln_fp8(x, sc, sh, wl.eps, oracle.fp8_dynamic_inverse(act), want_y=False))
