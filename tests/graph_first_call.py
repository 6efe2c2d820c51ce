"""Child process of test_gpu_graph_capture.py (not a test module): the library's first call
in this process, swiglu_nvfp4, is made under HIP graph capture; the graph is then replayed
several times, with eager work and a synchronization between replays and the input changed
in place before each, and every replay is compared with an eager call on the same input.
The per-call form (a fill kernel, the amax pass, the producer) is captured and checked the
same way.  Prints 'graph replays match' on success."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import nvfp4_activation_quantization_amd as nq  # noqa: E402

dev = "cuda:0"
m, f = 384, 1536
g = torch.Generator(device=dev).manual_seed(11)
proj = (2.0 * torch.randn(m, 2 * f, generator=g, device=dev)).to(torch.bfloat16)
codes, scales = nq.new_quantized(m, f, dev)
dcodes, dscales = nq.new_quantized(m, f, dev)
amax_out = torch.zeros(1, dtype=torch.float32, device=dev)
torch.cuda.synchronize()

static = torch.cuda.CUDAGraph()
with torch.cuda.graph(static):
    nq.swiglu_nvfp4(proj, 12.0, codes=codes, scales=scales)        # the first library call
dynamic = torch.cuda.CUDAGraph()
with torch.cuda.graph(dynamic):
    nq.swiglu_nvfp4_dynamic(proj, amax_out=amax_out, codes=dcodes, scales=dscales)

for rep in range(4):
    with torch.no_grad():
        proj.mul_(-1.5 if rep % 2 else 0.75)                        # eager work between replays
    for t, v in ((codes, 0x5A), (scales, 0xA5), (dcodes, 0x3C), (dscales, 0xC3)):
        t.fill_(v)
    amax_out.fill_(-1.0)
    torch.cuda.synchronize()
    static.replay()
    dynamic.replay()
    torch.cuda.synchronize()
    ec, es = nq.swiglu_nvfp4(proj, 12.0)
    dc, ds, damax = nq.swiglu_nvfp4_dynamic(proj)
    torch.cuda.synchronize()
    assert torch.equal(codes, ec) and torch.equal(scales, es), "static replay %d differs from the eager call" % rep
    assert torch.equal(dcodes, dc) and torch.equal(dscales, ds), "per-call replay %d differs" % rep
    assert torch.equal(amax_out, damax), "per-call replay %d amax %r vs %r" % (rep, amax_out.item(), damax.item())
    print("replay %d matches" % rep, flush=True)
print("graph replays match", flush=True)
