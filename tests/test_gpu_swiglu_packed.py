"""GPU parity of the packed-projection SwiGLU forms (bias before SiLU; value-first or
paired value/gate columns), static and per-call amax, through the C ABI, against the
CPU oracle on the same seeded inputs: codes, the whole swizzled scale buffer and the
bf16 side output bit for bit."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from util import first_mismatch, oracle_swiglu_packed, scales_from_rows, to_device, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


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
    return np.asarray(v, np.float32).view(np.uint32)


def projection(m, f, seed, bias_std=0.5, scale=2.0):
    g = np.random.Generator(np.random.PCG64(seed))
    proj = bf16(g.standard_normal((m, 2 * f)).astype(np.float32) * scale)
    bias = bf16(g.standard_normal(2 * f).astype(np.float32) * bias_std) if bias_std else None
    return proj, bias


def gpu_packed(nq, proj_dev, bias, interleaved, amax, m, f, y=True):
    bd = to_device(bias) if bias is not None else None
    yd = torch.empty((m, f), dtype=torch.int16, device="cuda:0") if y else None
    codes, scales = nq.swiglu_packed_nvfp4(proj_dev, amax, bias=bd, interleaved=interleaved, y_out=yd)
    torch.cuda.synchronize()
    return dict(codes=to_host(codes), scales=to_host(scales), y=to_host(yd) if y else None)


def check(got, proj, bias, interleaved, amax):
    m, two_f = proj.shape
    f = two_f // 2
    want = oracle_swiglu_packed(proj, bias, interleaved, amax, want_y=got["y"] is not None)
    assert_equal(got["codes"], want["codes"], "codes")
    assert_equal(got["scales"], scales_from_rows(want["scale_bytes"], m, f), "scales")
    if got["y"] is not None:
        assert_equal(got["y"], want["y"], "y_out")


def _f32_list(vals):
    return np.array([-0.0 if v == "-0" else float(v) for v in vals], np.float32)


@pytest.mark.parametrize("interleaved", [False, True])
def test_hand_worked_blocks(nq, interleaved):
    d = json.load(open(os.path.join(GOLDEN, "swiglu_packed_blocks.json")))
    f, cols = d["f"], d["columns"]
    half = {}
    for key in ("value", "value_bias", "gate", "gate_bias"):
        row = np.zeros((1, f), np.float32)
        row[0, :cols] = _f32_list(d[key])
        half[key] = bf16(row)
    proj = np.empty((1, 2 * f), np.uint16)
    bias = np.empty((1, 2 * f), np.uint16)
    if interleaved:
        proj[:, 0::2], proj[:, 1::2] = half["value"], half["gate"]
        bias[:, 0::2], bias[:, 1::2] = half["value_bias"], half["gate_bias"]
    else:
        proj[:, :f], proj[:, f:] = half["value"], half["gate"]
        bias[:, :f], bias[:, f:] = half["value_bias"], half["gate_bias"]
    got = gpu_packed(nq, to_device(proj), bias.reshape(-1), interleaved, d["global_amax"], 1, f)
    want = bytes.fromhex(d["codes_hex"]) + bytes(f // 2 - len(d["codes_hex"]) // 2)
    assert got["codes"][0].tobytes() == want
    assert list(got["scales"][0, :4]) == d["scale_codes"]
    assert not got["scales"][1:].any()


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("m,f", [(1, 64), (127, 128), (129, 192), (300, 512), (64, 19456), (257, 1024),
                                 (300, 1088), (131, 2624), (130, 320), (257, 960), (129, 1792)])
def test_shapes(nq, m, f, with_bias, interleaved):
    print("swiglu_packed", m, f, "bias" if with_bias else "no bias", "paired" if interleaved else "value-first",
          flush=True)
    proj, bias = projection(m, f, 7 * m + f + 3 * interleaved, bias_std=0.5 if with_bias else 0.0)
    for amax in [16.0, 2688.0]:
        check(gpu_packed(nq, to_device(proj), bias, interleaved, amax, m, f), proj, bias, interleaved, amax)


@pytest.mark.parametrize("interleaved", [False, True])
def test_every_gate_and_value_through_the_bias(nq, interleaved):
    """Every finite bf16 pattern as gate (then as value) of one column in each row, with a
    bias that sends many of the sums onto bf16 rounding ties and past the SiLU table's
    saturating and underflowing ends."""
    f = 64
    pats = np.arange(65536, dtype=np.uint32)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    g = np.random.Generator(np.random.PCG64(77))
    for role in ("gate", "value"):
        print("swiglu_packed sweep", role, "paired" if interleaved else "value-first", flush=True)
        value = bf16(g.standard_normal((len(pats), f)).astype(np.float32))
        gate = bf16(g.standard_normal((len(pats), f)).astype(np.float32) * 3)
        (gate if role == "gate" else value)[:, 5] = pats
        bv = bf16(g.standard_normal(f).astype(np.float32))
        bg = bf16(g.standard_normal(f).astype(np.float32))
        bv[5], bg[5] = bf16([2.0 ** -7])[0], bf16([-3.0])[0]
        proj = np.empty((len(pats), 2 * f), np.uint16)
        bias = np.empty(2 * f, np.uint16)
        if interleaved:
            proj[:, 0::2], proj[:, 1::2], bias[0::2], bias[1::2] = value, gate, bv, bg
        else:
            proj[:, :f], proj[:, f:], bias[:f], bias[f:] = value, gate, bv, bg
        check(gpu_packed(nq, to_device(proj), bias, interleaved, 8.0, len(pats), f), proj, bias, interleaved, 8.0)


@pytest.mark.parametrize("interleaved", [False, True])
def test_row_strided_view(nq, interleaved):
    m, f = 100, 256
    big = bf16(np.random.Generator(np.random.PCG64(12)).standard_normal((m, 2 * f + 64)).astype(np.float32))
    _, bias = projection(1, f, 13)
    bd = to_device(big)
    got = gpu_packed(nq, bd[:, 8:8 + 2 * f], bias, interleaved, 6.0, m, f)
    check(got, np.ascontiguousarray(big[:, 8:8 + 2 * f]), bias, interleaved, 6.0)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("m,f", [(1, 64), (129, 192), (130, 320), (300, 512), (129, 1792), (64, 19456)])
def test_dynamic(nq, m, f, interleaved):
    print("swiglu_packed_dynamic", m, f, "paired" if interleaved else "value-first", flush=True)
    # a large bias so that rows past m (which load zeros) would raise the amax if counted
    proj, bias = projection(m, f, 11 * m + f + interleaved, bias_std=4.0)
    y_out = torch.empty((m, f), dtype=torch.int16, device="cuda:0")
    codes, scales, amax = nq.swiglu_packed_nvfp4_dynamic(to_device(proj), bias=to_device(bias),
                                                         interleaved=interleaved, y_out=y_out)
    torch.cuda.synchronize()
    want = oracle.swiglu_packed_dynamic(proj, bias, interleaved, want_y=True, scales_rows=oracle.padded_rows(m))
    assert f32_bits(amax.cpu().numpy()[0]) == f32_bits(want["amax"])
    assert_equal(to_host(codes), want["codes"], "codes")
    assert_equal(to_host(scales), want["scales"], "scales")
    assert_equal(to_host(y_out), want["y"], "y_out")


# --------------------------------------------------------------------------------------
# full-size workloads, the launch configuration the benchmark times
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["swiglu_bias_16384x19456", "swiglu_paired_16384x19456"])
def test_full_packed(nq, name):
    wl = workloads.get(name)
    amax = workloads.calibration_amax(name)
    print("generating", name, flush=True)
    proj, bias = wl.x(), wl.bias()
    got = gpu_packed(nq, to_device(proj), bias, wl.interleaved, amax, wl.m, wl.k, y=False)
    print("oracle", flush=True)
    check(got, proj, bias, wl.interleaved, amax)


def test_full_paired_dynamic(nq):
    wl = workloads.get("swiglu_paired_16384x19456")
    print("generating", wl.name, flush=True)
    proj, bias = wl.x(), wl.bias()
    y_out = torch.empty((wl.m, wl.k), dtype=torch.int16, device="cuda:0")
    codes, scales, amax = nq.swiglu_packed_nvfp4_dynamic(to_device(proj), bias=to_device(bias), interleaved=True,
                                                         y_out=y_out)
    torch.cuda.synchronize()
    print("oracle", flush=True)
    want = oracle_swiglu_packed(proj, bias, True, 1.0, want_y=True)
    assert_equal(to_host(y_out), want["y"], "y_out")
    want_amax = oracle.max_abs(want["y"])
    assert f32_bits(amax.cpu().numpy()[0]) == f32_bits(want_amax)
    # for a finite 2688 / amax the per-call result is the static one at that amax
    ref = oracle_swiglu_packed(proj, bias, True, want_amax, want_y=False)
    assert_equal(to_host(codes), ref["codes"], "codes")
    assert_equal(to_host(scales), scales_from_rows(ref["scale_bytes"], wl.m, wl.k), "scales")
