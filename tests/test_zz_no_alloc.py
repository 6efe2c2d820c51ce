"""The allocation-free per-call entry point rms_adaln_nvfp4_dynamic_noalloc, called through
the raw C ABI (ctypes), against rms_adaln_nvfp4_dynamic on the same inputs: codes, the whole
swizzled scale buffer, rstd_out and y_out byte for byte, on two calls in a row where the
second is smaller and has a smaller amax (a scratch word left over from the first call
would then give the second call the wrong global scale).
"""
import ctypes

import numpy as np
import pytest

from util import first_mismatch

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_activation_quantization_amd as mod
    return mod


def bf16_bits(a):
    a = np.ascontiguousarray(a, np.float32).view(np.uint32)
    return ((a + 0x7FFF + ((a >> 16) & 1)) >> 16).astype(np.uint16)


def make_case(seed, m, k, frames, scale):
    g = np.random.Generator(np.random.PCG64(seed))
    x = bf16_bits(g.standard_normal((m, k)).astype(np.float32) * np.float32(scale))
    w = bf16_bits(1 + 0.1 * g.standard_normal(k).astype(np.float32))
    table = bf16_bits(0.1 * g.standard_normal((frames, 2, k)).astype(np.float32))
    idx = g.integers(0, frames, m).astype(np.int32)
    idx.sort()
    return x, w, table, idx


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def run_both(nq, case, eps=1e-6):
    x, w, table, idx = case
    m, k = x.shape
    xd, wd, td, idd = dev(x), dev(w), dev(table), dev(idx)
    lib = nq.library()
    fn = lib.rms_adaln_nvfp4_dynamic_noalloc
    P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    fn.argtypes = [P, P, P, P, I64, I64, P, F, I64, I64, P, P, P, P, P, P]
    fn.restype = ctypes.c_int
    padded = nq.padded_rows(m)
    codes = torch.full((m, k // 2), 0x5A, dtype=torch.uint8, device="cuda:0")
    scales = torch.full((padded, k // 16), 0xA5, dtype=torch.uint8, device="cuda:0")
    rstd = torch.empty(m, dtype=torch.float32, device="cuda:0")
    y = torch.empty((m, k), dtype=torch.int16, device="cuda:0")
    tab = td.data_ptr()
    stream = torch.cuda.current_stream()
    rc = fn(xd.data_ptr(), wd.data_ptr(), tab, tab + 2 * k, 2 * k, table.shape[0], idd.data_ptr(), eps, m, k,
            codes.data_ptr(), scales.data_ptr(), rstd.data_ptr(), y.data_ptr(), None, stream.cuda_stream)
    assert rc == 0, rc
    # the existing per-call entry point, with its own amax buffer
    amax = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    rstd2 = torch.empty(m, dtype=torch.float32, device="cuda:0")
    y2 = torch.empty((m, k), dtype=torch.int16, device="cuda:0")
    c2, s2, a2 = nq.rms_adaln_nvfp4_dynamic(xd, wd, td, idd, eps, amax_out=amax, rstd_out=rstd2, y_out=y2)
    torch.cuda.synchronize()
    for got, want, what in ((codes, c2, "codes"), (scales, s2, "scales"), (rstd, rstd2, "rstd"), (y, y2, "y_out")):
        g, w_ = got.cpu().numpy(), want.cpu().numpy()
        if g.dtype == np.float32:
            g, w_ = g.view(np.uint32), w_.view(np.uint32)
        assert np.array_equal(g, w_), "%s: %s" % (what, first_mismatch(g, w_))
    return float(a2.cpu().numpy()[0])


def test_noalloc_matches_dynamic_on_two_calls(nq):
    print("noalloc: call 1 (2000 x 7168, large amax)", flush=True)
    a1 = run_both(nq, make_case(71, 2000, 7168, 3, 8.0))
    print("noalloc: call 2 (300 x 2048, small amax)", flush=True)
    a2 = run_both(nq, make_case(72, 300, 2048, 2, 0.5))
    assert a2 < a1   # the second call's own amax is the smaller one: a stale word would show


def test_noalloc_empty_and_bad_shape(nq):
    lib = nq.library()
    fn = lib.rms_adaln_nvfp4_dynamic_noalloc
    P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    fn.argtypes = [P, P, P, P, I64, I64, P, F, I64, I64, P, P, P, P, P, P]
    fn.restype = ctypes.c_int
    assert fn(None, None, None, None, 1024, 1, None, 1e-6, 0, 512, None, None, None, None, None, None) == 0
    assert fn(None, None, None, None, 1024, 1, None, 1e-6, 4, 500, None, None, None, None, None, None) == 2
