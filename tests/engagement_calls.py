"""Child process of test_gpu_engagement.py (not a test module): one call of every entry
point of the library on small inputs, in a fixed order, then the list of kernels each call
is expected to launch, written as JSON to argv[1].  Each entry names the kernel and, for
the RMSNorm + adaLN kernel, whether it is the amax pass (its last template argument)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import nvfp4_activation_quantization_amd as nq  # noqa: E402

dev = "cuda:0"
g = torch.Generator(device=dev).manual_seed(7)
m, k, f, T = 256, 1024, 512, 3


def bf16(*shape):
    return torch.randn(*shape, generator=g, device=dev).to(torch.bfloat16)


x = bf16(m, k)
w = bf16(k)
table = (0.1 * torch.randn(T, 2, k, generator=g, device=dev)).to(torch.bfloat16)
idx = (torch.arange(m, device=dev, dtype=torch.int32) * T // m).to(torch.int32)
proj = bf16(m, 2 * f)
pbias = bf16(2 * f)
h = torch.randn(m, k, generator=g, device=dev)
o = bf16(m, k)
obias = bf16(k)
rscale = torch.randn(k, generator=g, device=dev)
gamma32 = torch.randn(k, generator=g, device=dev)
gate = (0.2 * torch.randn(T, k, generator=g, device=dev)).to(torch.bfloat16)
xs = torch.randn(2, 8, 16, 256, generator=g, device=dev).to(torch.float16)
gs = torch.randn(256, generator=g, device=dev).to(torch.float16)
xl = torch.randn(m, k, generator=g, device=dev).to(torch.float16)
sc = 0.1 * torch.randn(k, generator=g, device=dev)
sh = 0.1 * torch.randn(k, generator=g, device=dev)
torch.cuda.synchronize()

PRODUCER = [["rms_adaln_staged", "producer"]]
calls = [
    (lambda: nq.nvfp4_quantize(x, 4.0), [["quantize_kernel", None]]),
    (lambda: nq.nvfp4_quantize_dynamic(x), [["zero_amax_kernel", None], ["amax_x_kernel", None],
                                            ["quantize_kernel", None]]),
    (lambda: nq.rms_adaln_nvfp4(x, w, table, idx, 1e-6, 8.0), PRODUCER),
    (lambda: nq.rms_adaln_nvfp4_dynamic(x, w, table, idx, 1e-6),
     [["zero_amax_kernel", None], ["rms_adaln_staged", "amax"]] + PRODUCER),
    (lambda: nq.rms_adaln_nvfp4_dynamic_noalloc(x, w, table, idx, 1e-6),
     [["zero_amax_kernel", None], ["rms_adaln_staged", "amax"]] + PRODUCER),
    (lambda: nq.swiglu_nvfp4(proj, 4.0), [["swiglu_kernel", None]]),
    (lambda: nq.swiglu_nvfp4_dynamic(proj), [["zero_amax_kernel", None], ["swiglu_kernel", None],
                                             ["swiglu_kernel", None]]),
    (lambda: nq.swiglu_packed_nvfp4(proj, 4.0, bias=pbias, interleaved=True), [["swiglu_kernel", None]]),
    (lambda: nq.swiglu_packed_nvfp4_dynamic(proj, bias=pbias, interleaved=True),
     [["zero_amax_kernel", None], ["swiglu_kernel", None], ["swiglu_kernel", None]]),
    (lambda: nq.residual_rms_nvfp4(h, gamma32, 1e-6, 16.0, residual=(o, obias, rscale)),
     [["residual_rms_kernel", None]]),
    (lambda: nq.residual_rms_nvfp4_dynamic(h, gamma32, 1e-6, residual=(o, obias, rscale)),
     [["zero_amax_kernel", None], ["residual_rms_kernel", None], ["residual_rms_kernel", None]]),
    (lambda: nq.residual_rms_adaln_nvfp4(h, w, table, idx, 1e-6, 16.0, residual=(o, None, gate)),
     [["residual_rms_kernel", None]]),
    (lambda: nq.residual_rms_adaln_nvfp4_dynamic(h, w, table, idx, 1e-6, residual=(o, None, gate)),
     [["zero_amax_kernel", None], ["residual_rms_kernel", None], ["residual_rms_kernel", None]]),
    (lambda: nq.rms_silu_nvfp4(xs, gs, 1e-6, 6.0), [["rms_silu_kernel", None]]),
    (lambda: nq.rms_silu_nvfp4_dynamic(xs, gs, 1e-6), [["zero_amax_kernel", None], ["rms_silu_kernel", None],
                                                        ["rms_silu_kernel", None]]),
    (lambda: nq.ln_adaln_fp8(xl, sc, sh, 1e-6, 0.05), [["ln_fp8_kernel", None]]),
    (lambda: nq.ln_adaln_fp8_dynamic(xl, sc, sh, 1e-6), [["zero_amax_kernel", None], ["ln_fp8_kernel", None],
                                                         ["amax_to_fp8_scale_kernel", None],
                                                         ["ln_fp8_kernel", None]]),
]
expected = []
for fn, kernels in calls:
    fn()
    expected.extend(kernels)
torch.cuda.synchronize()
with open(sys.argv[1], "w") as fh:
    json.dump(expected, fh)
print("engagement calls done: %d calls, %d kernels expected" % (len(calls), len(expected)), flush=True)
