"""Every input of the gfx950 conversions the producer kernels rely on, against the CPU
oracle's encoders: the helpers of common.hpp, compiled as the kernels compile them, run
over whole fp32 bit-pattern ranges by libnvfp4act_selftest.so (NaN inputs excluded: they
are outside the contract).

  round_bf16 (v_cvt_pk_bf16_f32, zero low operand)  all 2^32 patterns vs bf16_round, and
                                                   the result's low half must be +0
  pack_bf16x2 (both operands converted)             all 2^32 patterns vs bf16_round
  e4m3_code (clamp at 448, v_cvt_pk_fp8_f32)        every non-negative pattern (2^31:
                                                   the kernels only convert sf >= 0)
                                                   vs e4m3_encode
  pack_e2m1x8 (v_cvt_scalef32_pk_fp4_f32, scale 1)  all 2^32 patterns vs e2m1_encode
  fp8_quad (med3 clamp, v_cvt_pk_fp8_f32)           all 2^32 patterns vs e4m3_encode_signed
  f16_bits (fp32 -> fp16)                           all 2^32 patterns vs f16_round

The rounding these conversions must reproduce is the one the FastVideo branch compare's
minimax_h3_swiglu_quant.cuh applies in scale_fp8 and fp4_pair (round to nearest even,
saturating), written out as the oracle's encoders.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SELFTEST = os.path.join(ROOT, "nvfp4_activation_quantization_amd", "libnvfp4act_selftest.so")
CHUNK = 1 << 26
WORKERS = max(1, min(16, os.cpu_count() or 1))   # host checks in parallel (ctypes drops the GIL)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_activation_quantization_amd  # noqa: F401  (checks the build matches the sources)
    if not os.path.exists(SELFTEST):
        raise RuntimeError("libnvfp4act_selftest.so is not built")
    lib = ctypes.CDLL(SELFTEST)
    lib.nvfp4act_selftest_convert.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
    lib.nvfp4act_selftest_convert.restype = ctypes.c_int
    lib.nvfp4act_selftest_convert_bytes.argtypes = [ctypes.c_int, ctypes.c_int64]
    lib.nvfp4act_selftest_convert_bytes.restype = ctypes.c_int64
    return lib


def inputs(first, count):
    bits = np.arange(count, dtype=np.uint32) + np.uint32(first)     # first + count <= 2^32
    keep = ~(((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x007FFFFF) != 0))   # not NaN
    return bits.view(np.float32), keep


def expected_and_got(kind, first, count, got_bytes):
    x, keep = inputs(first, count)
    if kind in (0, 1):
        want, got = oracle.bf16_round(x), got_bytes.view(np.uint16)
    elif kind == 5:
        want, got = oracle.f16_round(x), got_bytes.view(np.uint16)
    elif kind == 2:
        want, got = oracle.e4m3_encode(x), got_bytes
    elif kind == 4:
        want, got = oracle.e4m3_encode_signed(x), got_bytes
    else:
        want = oracle.e2m1_encode(x)
        got = np.empty(count, np.uint8)
        got[0::2] = got_bytes & 0x0F
        got[1::2] = got_bytes >> 4
    return want[keep], got[keep], x[keep]


def sweep(lib, kind, first, last):
    """Run conversion `kind` over the patterns [first, last) in chunks; the host checks run
    on a thread pool while the next chunk converts."""
    stream = torch.cuda.current_stream()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    nbytes = lib.nvfp4act_selftest_convert_bytes(kind, CHUNK)
    out = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    failures = []

    def check(first, got_bytes):
        want, got, x = expected_and_got(kind, first, CHUNK, got_bytes)
        bad = np.nonzero(want != got)[0]
        if bad.size:
            i = bad[0]
            failures.append("input 0x%08x: got 0x%x, want 0x%x (%d mismatches in the chunk at 0x%08x)"
                            % (x[i:i + 1].view(np.uint32)[0], got[i], want[i], bad.size, first))

    with ThreadPoolExecutor(WORKERS) as pool:
        futures = []
        for start in range(first, last, CHUNK):
            rc = lib.nvfp4act_selftest_convert(kind, start, CHUNK, out.data_ptr(), flag.data_ptr(), stream.cuda_stream)
            assert rc == 0, rc
            host = out.cpu().numpy()          # synchronizes
            futures.append(pool.submit(check, start, host))
            if len(futures) >= 2 * WORKERS:
                futures.pop(0).result()
        for f in futures:
            f.result()
    assert not failures, failures[:5]
    return int(flag.cpu().numpy()[0])


def test_round_bf16_every_input(lib):
    print("round_bf16 over all 2^32 fp32 patterns", flush=True)
    assert sweep(lib, 0, 0, 1 << 32) == 0, "a bf16 result had a nonzero low half"


def test_pack_bf16x2_every_input(lib):
    print("pack_bf16x2 over all 2^32 fp32 patterns", flush=True)
    sweep(lib, 1, 0, 1 << 32)


@pytest.mark.parametrize("part", range(2))
def test_e4m3_code_every_non_negative_input(lib, part):
    # the E4M3 encoder of the oracle searches the code table per input: the 2^31 inputs are
    # checked in two halves so that each test stays short
    first = part << 30
    print("e4m3_code over the non-negative fp32 patterns 0x%08x .. +2^30" % first, flush=True)
    sweep(lib, 2, first, first + (1 << 30))


def test_pack_e2m1x8_every_input(lib):
    print("pack_e2m1x8 over all 2^32 fp32 patterns", flush=True)
    sweep(lib, 3, 0, 1 << 32)


@pytest.mark.parametrize("part", range(4))
def test_fp8_quad_every_input(lib, part):
    first = part << 30
    print("fp8_quad over the fp32 patterns 0x%08x .. +2^30" % first, flush=True)
    sweep(lib, 4, first, first + (1 << 30))


def test_f16_bits_every_input(lib):
    print("f16_bits over all 2^32 fp32 patterns", flush=True)
    sweep(lib, 5, 0, 1 << 32)


def test_selftest_rejects_bad_ranges(lib):
    out = torch.empty(64, dtype=torch.uint8, device="cuda:0")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    assert lib.nvfp4act_selftest_convert(0, 0xFFFFFFF8, 16, out.data_ptr(), flag.data_ptr(), None) == 2
    assert lib.nvfp4act_selftest_convert(0, 0, 12, out.data_ptr(), flag.data_ptr(), None) == 2
    assert lib.nvfp4act_selftest_convert(9, 0, 16, out.data_ptr(), flag.data_ptr(), None) == 2
