"""The Python binding rejects bad arguments before any launch (CPU only).

The tensors are CPU tensors dressed as device tensors (is_cuda True, device cuda:0), and
the C library is replaced by a stub that fails the test if any entry point is called, so
a check that does not fire can never reach a kernel.  Every case has a control that
differs only in the argument under test and does reach the (stubbed) launch.
"""
import pytest
import torch

import nvfp4_activation_quantization_amd as nq


class Dev:
    """A CPU tensor that reports itself as a device tensor."""

    def __init__(self, t):
        self._t = t

    is_cuda = True
    device = torch.device("cuda", 0)

    def __getattr__(self, name):
        return getattr(self._t, name)

    @property
    def shape(self):
        return self._t.shape

    @property
    def dtype(self):
        return self._t.dtype


class Launched(Exception):
    pass


class StubLib:
    """The library's host-only helpers pass through; every other entry point raises."""
    HOST_ONLY = ("nvfp4act_padded_rows", "nvfp4act_status_string")

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in self.HOST_ONLY:
            return getattr(self._real, name)

        def entry(*args):
            raise Launched(name)
        return entry


class Stream:
    cuda_stream = 0


@pytest.fixture(autouse=True)
def stub_library(monkeypatch):
    monkeypatch.setattr(nq, "_lib", StubLib(nq._lib))


M, K = 4, 512


def dev(shape, dtype):
    return Dev(torch.zeros(shape, dtype=dtype))


def quant_outs(m=M, k=K):
    return dict(codes=dev((m, k // 2), torch.uint8), scales=dev((nq.padded_rows(m), k // 16), torch.uint8))


def rms_adaln_args(**over):
    a = dict(x=dev((M, K), torch.bfloat16), weight=dev((K,), torch.bfloat16), table=dev((3, 2, K), torch.bfloat16),
             frame_idx=dev((M,), torch.int32), eps=1e-6)
    a.update(over)
    return a


def call_rms_adaln(dynamic=False, **over):
    a = rms_adaln_args(**over)
    extra = dict(quant_outs(), stream=Stream())
    extra.update({k: v for k, v in over.items() if k in ("y_out", "rstd_out", "status_word")})
    args = (a["x"], a["weight"], a["table"], a["frame_idx"], a["eps"])
    if dynamic:
        return nq.rms_adaln_nvfp4_dynamic(*args, amax_out=dev((1,), torch.float32), **extra)
    return nq.rms_adaln_nvfp4(*args, 1.0, **extra)


@pytest.mark.parametrize("dynamic", [False, True])
def test_rms_adaln_valid_arguments_reach_the_launch(dynamic):
    with pytest.raises(Launched):
        call_rms_adaln(dynamic)
    with pytest.raises(Launched):
        call_rms_adaln(dynamic, y_out=dev((M, K), torch.bfloat16))


@pytest.mark.parametrize("dynamic", [False, True])
@pytest.mark.parametrize("dtype", [torch.uint8, torch.float32, torch.float16, torch.int32])
def test_rms_adaln_rejects_y_out_of_another_dtype(dynamic, dtype):
    with pytest.raises(ValueError, match="y_out"):
        call_rms_adaln(dynamic, y_out=dev((M, K), dtype))


@pytest.mark.parametrize("dynamic", [False, True])
def test_rms_adaln_rejects_host_frame_idx(dynamic):
    with pytest.raises(TypeError, match="frame_idx"):
        call_rms_adaln(dynamic, frame_idx=torch.zeros(M, dtype=torch.int32))


@pytest.mark.parametrize("dynamic", [False, True])
@pytest.mark.parametrize("n", [K - 1, K + 1])
def test_rms_adaln_rejects_weight_of_another_length(dynamic, n):
    with pytest.raises(ValueError, match="weight"):
        call_rms_adaln(dynamic, weight=dev((n,), torch.bfloat16))


def test_rms_adaln_rejects_frame_idx_of_another_length_or_dtype():
    with pytest.raises(ValueError, match="frame_idx"):
        call_rms_adaln(frame_idx=dev((M + 1,), torch.int32))
    with pytest.raises(ValueError, match="frame_idx"):
        call_rms_adaln(frame_idx=dev((M,), torch.int64))


def fold_call(**over):
    a = dict(h=dev((M, K), torch.float32), weight=dev((K,), torch.bfloat16), table=dev((3, 2, K), torch.bfloat16),
             frame_idx=dev((M,), torch.int32))
    a.update({k: v for k, v in over.items() if k in a})
    residual = (dev((M, K), torch.bfloat16), None, dev((3, K), torch.bfloat16))
    extra = dict(quant_outs(), stream=Stream())
    extra.update({k: v for k, v in over.items() if k == "y_out"})
    return nq.residual_rms_adaln_nvfp4(a["h"], a["weight"], a["table"], a["frame_idx"], 1e-6, 1.0,
                                       residual=residual, **extra)


def test_fold_checks_frame_idx_placement_and_contiguity():
    with pytest.raises(Launched):
        fold_call()
    with pytest.raises(TypeError, match="frame_idx"):
        fold_call(frame_idx=torch.zeros(M, dtype=torch.int32))
    strided = Dev(torch.zeros(2 * M, dtype=torch.int32)[::2])
    with pytest.raises(ValueError, match="frame_idx"):
        fold_call(frame_idx=strided)
    with pytest.raises(ValueError, match="y_out"):
        fold_call(y_out=dev((M, K), torch.uint8))


def test_swiglu_rejects_y_out_of_another_dtype():
    proj = dev((M, 2 * K), torch.bfloat16)
    with pytest.raises(Launched):
        nq.swiglu_nvfp4(proj, 1.0, y_out=dev((M, K), torch.bfloat16), stream=Stream(), **quant_outs())
    for dtype in (torch.uint8, torch.float32):
        with pytest.raises(ValueError, match="y_out"):
            nq.swiglu_nvfp4(proj, 1.0, y_out=dev((M, K), dtype), stream=Stream(), **quant_outs())
        with pytest.raises(ValueError, match="y_out"):
            nq.swiglu_packed_nvfp4(proj, 1.0, y_out=dev((M, K), dtype), stream=Stream(), **quant_outs())


def test_rms_silu_wants_an_fp16_y_out():
    x = dev((2, 3, K), torch.float16)
    gamma = dev((K,), torch.float16)
    rows = 6
    outs = dict(codes=dev((rows, K // 2), torch.uint8), scales=dev((rows, K // 16), torch.uint8), stream=Stream())
    with pytest.raises(Launched):
        nq.rms_silu_nvfp4(x, gamma, 1e-6, 1.0, y_out=dev((rows, K), torch.float16), **outs)
    for dtype in (torch.bfloat16, torch.uint8, torch.float32):
        with pytest.raises(ValueError, match="y_out"):
            nq.rms_silu_nvfp4(x, gamma, 1e-6, 1.0, y_out=dev((rows, K), dtype), **outs)


def test_ln_fp8_wants_an_fp32_y_out():
    x = dev((M, K), torch.float16)
    sc, sh = dev((K,), torch.float32), dev((K,), torch.float32)
    codes = dev((M, K), torch.uint8)
    with pytest.raises(Launched):
        nq.ln_adaln_fp8(x, sc, sh, 1e-6, 1.0, codes=codes, y_out=dev((M, K), torch.float32), stream=Stream())
    for dtype in (torch.bfloat16, torch.float16, torch.uint8):
        with pytest.raises(ValueError, match="y_out"):
            nq.ln_adaln_fp8(x, sc, sh, 1e-6, 1.0, codes=codes, y_out=dev((M, K), dtype), stream=Stream())


def test_residual_rms_wants_a_bf16_y_out():
    h = dev((M, K), torch.float32)
    gamma = dev((K,), torch.float32)
    with pytest.raises(Launched):
        nq.residual_rms_nvfp4(h, gamma, 1e-6, 1.0, y_out=dev((M, K), torch.bfloat16), stream=Stream(), **quant_outs())
    with pytest.raises(ValueError, match="y_out"):
        nq.residual_rms_nvfp4(h, gamma, 1e-6, 1.0, y_out=dev((M, K), torch.uint8), stream=Stream(), **quant_outs())
