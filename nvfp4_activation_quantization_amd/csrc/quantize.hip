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

// Launch shape (compile-time tuning knobs).
#ifndef NVFP4ACT_Q_THREADS
#define NVFP4ACT_Q_THREADS 256
#endif
#ifndef NVFP4ACT_Q_ROWS
#define NVFP4ACT_Q_ROWS 32
#endif
#ifndef NVFP4ACT_Q_UNROLL
#define NVFP4ACT_Q_UNROLL 4
#endif
#ifndef NVFP4ACT_Q_XCD_REMAP
#define NVFP4ACT_Q_XCD_REMAP 1
#endif
constexpr int kThreads = NVFP4ACT_Q_THREADS;
constexpr int kWavesPerWg = kThreads / kWave;
constexpr int kRowsPerUnit = NVFP4ACT_Q_ROWS;
constexpr int kUnroll = NVFP4ACT_Q_UNROLL;

// Quantize kChunkUnroll x 64 consecutive chunks of one row starting at chunk c0; with
// Tail, lanes whose chunk lies past the row's end do nothing visible.
template <bool Tail>
__device__ __forceinline__ void quantize_span(const NVFP4_GLOBAL uint4* xr, NVFP4_GLOBAL uint32_t* cr,
                                              NVFP4_GLOBAL uint8_t* sr, int64_t c0, int64_t chunks, int lane,
                                              float gsf, const float* inv_tab) {
  uint4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = c0 + u * kWave + lane;
    if (!Tail || c < chunks) v[u] = load_stream(reinterpret_cast<const uint4*>(xr + c));
    else v[u] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t c = c0 + u * kWave + lane;
    float y[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                  bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
    uint32_t s;
    const uint32_t q = quantize_chunk(y, gsf, inv_tab, &s);
    if (!Tail || c < chunks) {
      cr[c0 + u * kWave] = q;
      sr[(c0 / 8 + 8 * u) * 512] = (uint8_t)s;
    }
  }
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t m,
                                                            int64_t k, int64_t padded, float global_amax,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t per) {
  __shared__ float inv_tab[128];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const float gsf = global_scale(global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  __syncthreads();

#if NVFP4ACT_Q_XCD_REMAP
  const int64_t unit = xcd_unit(per);
#else
  const int64_t unit = blockIdx.x;
#endif
  const int64_t r0 = unit * kRowsPerUnit;
  if (r0 >= padded) return;
  const int64_t r1 = (r0 + kRowsPerUnit < padded) ? r0 + kRowsPerUnit : padded;
  const int64_t chunks = k >> 3;           // 8-element chunks per row (multiple of 8)
  const int64_t span = kWave * kUnroll;
  const int64_t full = chunks / span * span;

  for (int64_t r = r0 + wave; r < r1; r += kWavesPerWg) {
    if (r >= m) {                          // padding row: scale bytes only
      zero_row_scales(scales, r, k, lane);
      continue;
    }
    const NVFP4_GLOBAL uint4* xr = global_ptr(x) + r * chunks;
    NVFP4_GLOBAL uint32_t* cr = global_ptr(codes) + r * chunks + lane;
    NVFP4_GLOBAL uint8_t* sr = global_ptr(scales) + row_scale_base(r, k) + scale_lane_offset(lane);
    for (int64_t c0 = 0; c0 < full; c0 += span) quantize_span<false>(xr, cr, sr, c0, chunks, lane, gsf, inv_tab);
    if (full < chunks) quantize_span<true>(xr, cr, sr, full, chunks, lane, gsf, inv_tab);
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
