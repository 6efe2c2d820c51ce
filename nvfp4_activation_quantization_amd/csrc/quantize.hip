// quantize.hip -- standalone NVFP4 quantize of a bf16 tensor (the attention-output
// quantize of TensorRT-LLM PR #21483; FastVideo API page, quantize).
//
// Bandwidth-bound: 2 bytes in, 0.5625 bytes out per element.  Each 256-thread
// workgroup owns kRowsPerUnit consecutive rows (two per wavefront at a time, interleaved
// loads so each wavefront keeps 2 x kUnroll 1 KiB loads in flight).  Rows m..pad(m)-1
// only get their scale bytes zeroed.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWg = kThreads / kWave;
constexpr int kRowsPerUnit = 32;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t m,
                                                            int64_t k, int64_t padded, float global_amax,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t per) {
  __shared__ float inv_tab[128];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const GatherAddr ga = scale_gather_addresses(lane);
  const float gsf = global_scale(global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  __syncthreads();

  const int64_t unit = xcd_unit(per);
  const int64_t r0 = unit * kRowsPerUnit;
  if (r0 >= padded) return;
  const int64_t r1 = (r0 + kRowsPerUnit < padded) ? r0 + kRowsPerUnit : padded;
  const int64_t chunks = k >> 3;           // 8-element chunks per row (multiple of 8)
  const int64_t xrow = k >> 3;             // uint4 per input row
  const int64_t crow = k >> 3;             // uint32 code words per row (8 codes each)

  for (int64_t r = r0 + wave; r < r1; r += kWavesPerWg) {
    if (r >= m) {                          // padding row: scale bytes only
      zero_row_scales(scales, r, k, lane);
      continue;
    }
    const uint4* xr = x + r * xrow;
    uint32_t* cr = codes + r * crow;
    const int64_t sbase = row_scale_base(r, k);
    for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int64_t c = c0 + u * kWave + lane;
        v[u] = (c < chunks) ? load_stream(xr + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        int64_t c = c0 + u * kWave + lane;
        float y[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                      bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
        uint32_t s;
        uint32_t q = quantize_chunk(y, gsf, inv_tab, &s);
        uint32_t s4 = gather_scales4(s, ga);
        if (c < chunks) {
          cr[c] = q;
          if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(scales + sbase + c * 64) = s4;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int64_t m, int64_t k, float global_amax, void* codes,
                           void* scales, hipStream_t stream) {
  const int64_t padded = (m + 127) / 128 * 128;
  const int64_t units = (padded + kRowsPerUnit - 1) / kRowsPerUnit;
  const int64_t per = (units + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(quantize_kernel, dim3((uint32_t)(per * kXcds)), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(x), m, k, padded, global_amax,
                     static_cast<uint32_t*>(codes), static_cast<uint8_t*>(scales), per);
  return hipGetLastError();
}

}  // namespace nvfp4act
