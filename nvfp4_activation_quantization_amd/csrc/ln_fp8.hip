// ln_fp8.hip -- LayerNorm (fp32 statistics) + adaLN -> per-tensor FP8 E4M3 of fp16 rows
// (FlashRT PR #142, fp16_ada_layernorm_quant_fp8: one pass, fp32 statistics, one FP8 scale
// shared by the three projections that read the result):
//   mean = sum(x) / k                        the fixed tree below (adds)
//   var  = sum((x - mean)^2) / k             the same tree (fused multiply-adds)
//   y    = (((x - mean) * rstd) * (1 + scale)) + shift     fp32, rstd = 1 / sqrt(var + eps)
//   q    = E4M3(y * inv_scale)               nearest-even, saturating at +-448
//
// The statistic tree is that of the RMSNorm producer: lane L owns the 8-element chunks
// L + 64 j, 8 accumulators over its chunks in ascending order, pairwise lane fold, then
// the butterfly over the 64 lanes.
//
// One workgroup of 8 wavefronts per CU, persistent over rows (wavefront w of workgroup b
// takes rows 8b + w, 8b + w + 8 G, ... for a grid of G workgroups, so the rows in flight
// at any time are consecutive).  The only parameters are two fp32 vectors, 1 + scale
// (computed once) and shift, staged in LDS as float2 planes (consecutive across the
// wavefront: each ds_read_b64 covers 512 contiguous bytes).  Each wavefront keeps its row
// unpacked in registers from the statistics to the output pass and loads the next row's
// 16-byte chunks at the top of each row.  The output is 1 byte an element: 8 bytes a
// chunk, one non-temporal store per lane (y, when asked for, likewise).
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;

struct LnArgs {
  const uint4* x;           // [m, k] fp16, 16-byte chunks
  const float* scale;       // [k] fp32
  const float* shift;       // [k] fp32
  float eps;
  int64_t m, k;
  float act_scale;          // static per-tensor scale (codes = E4M3(y / act_scale))
  const float* scale_dev;   // per-call: the device scale (null: static act_scale)
  float* amax_out;          // the amax pass: where max |y| is folded
  uint2* codes;             // 8 bytes per chunk
  float* mean_out;
  float* rstd_out;
  float4* y_out;            // [m, k] fp32, two float4 per chunk
};


// The inverse scale of the call: 1 / act_scale (static, checked on the host), or from the
// device scale of a per-call form: 0 when that scale is 0 or its reciprocal overflows.
__device__ __forceinline__ float call_inverse_scale(const LnArgs& a) {
  if (!a.scale_dev) return 1.0f / a.act_scale;
  const float s = *global_ptr(a.scale_dev);
  if (!(s > 0.0f)) return 0.0f;
  const float r = 1.0f / s;
  return __builtin_isinf(r) ? 0.0f : r;
}

// Unpack a row's fp16 chunks to fp32 and accumulate the lane's part of the mean's tree.
template <int CPL>
__device__ __forceinline__ void unpack_sum(const uint4 (&xr)[CPL], float (&xf)[CPL][8], float (&acc)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const uint32_t w[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xf[j][2 * q] = f16_lo(w[q]);
      xf[j][2 * q + 1] = f16_hi(w[q]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] + xf[j][e];
  }
}

enum Mode { kAmaxPass = 0, kCodes = 1, kCodesAndY = 2 };

// MODE kAmaxPass: fold max |y| into a.amax_out, write nothing else; kCodes: codes (and the
// nullable mean / rstd); kCodesAndY: also y_out.
template <int CPL, int MODE>
__global__ __launch_bounds__(kThreads) void ln_fp8_kernel(const LnArgs a) {
  constexpr bool AMAX = MODE == kAmaxPass;
  constexpr int kChunks = CPL * kWave;            // chunks per row
  constexpr int kK = kChunks * 8;
  __shared__ float amax_red[kWaves];
  extern __shared__ float2 planes[];              // 1 + scale: 4 planes of kChunks float2, then shift
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int64_t m = a.m;
  const int64_t first = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t stride = (int64_t)gridDim.x * kWaves;

  // the first row is in flight while the parameters are staged (a row past the end
  // re-reads row m - 1, which is never used)
  uint4 xr[CPL];
  {
    const int64_t r = first < m ? first : m - 1;
#pragma unroll
    for (int j = 0; j < CPL; ++j) xr[j] = load_stream(a.x + r * kChunks + lane + kWave * j);
  }
  for (int c = tid; c < kChunks; c += kThreads) {
    const float4 s0 = reinterpret_cast<const NVFP4_GLOBAL float4*>(global_ptr(a.scale))[2 * c];
    const float4 s1 = reinterpret_cast<const NVFP4_GLOBAL float4*>(global_ptr(a.scale))[2 * c + 1];
    const float4 h0 = reinterpret_cast<const NVFP4_GLOBAL float4*>(global_ptr(a.shift))[2 * c];
    const float4 h1 = reinterpret_cast<const NVFP4_GLOBAL float4*>(global_ptr(a.shift))[2 * c + 1];
    planes[c] = make_float2(1.0f + s0.x, 1.0f + s0.y);
    planes[kChunks + c] = make_float2(1.0f + s0.z, 1.0f + s0.w);
    planes[2 * kChunks + c] = make_float2(1.0f + s1.x, 1.0f + s1.y);
    planes[3 * kChunks + c] = make_float2(1.0f + s1.z, 1.0f + s1.w);
    planes[4 * kChunks + c] = make_float2(h0.x, h0.y);
    planes[5 * kChunks + c] = make_float2(h0.z, h0.w);
    planes[6 * kChunks + c] = make_float2(h1.x, h1.y);
    planes[7 * kChunks + c] = make_float2(h1.z, h1.w);
  }
  const float inv = call_inverse_scale(a);
  __syncthreads();

  // The row being worked on is unpacked at the end of the previous iteration, right after
  // this iteration's loads were waited for: the wait then sits in straight-line code after
  // the row's stores and can leave them in flight (at the loop head it would also cover
  // the stores).
  //
  // The eight wavefronts of a workgroup take the same number of iterations (that of
  // wavefront 0) and meet at a barrier after each, so that they keep working on eight
  // consecutive rows: left to drift apart they spread the rows in flight over the tensor,
  // which costs HBM efficiency.  A wavefront whose row is past the end recomputes row
  // m - 1 and stores the same bytes as the wavefront that owns it.
  float xf[CPL][8];
  float acc[8];
  unpack_sum(xr, xf, acc);
  float lane_amax = 0.0f;
  const int64_t wg_first = (int64_t)blockIdx.x * kWaves;
  const int64_t iters = wg_first < m ? (m - wg_first + stride - 1) / stride : 0;
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t r_own = first + it * stride;
    const int64_t r = r_own < m ? r_own : m - 1;
    // wide rows: keep the parameters in LDS rather than let them be hoisted into registers
    if constexpr (CPL >= 5) asm volatile("" ::: "memory");
    // the next row of this wavefront, in flight during the rest of this one
    {
      const int64_t rn = (r_own + stride < m) ? r_own + stride : m - 1;
#pragma unroll
      for (int j = 0; j < CPL; ++j) xr[j] = load_stream(a.x + rn * kChunks + lane + kWave * j);
    }
    const float sum = lane_sum_butterfly(((acc[0] + acc[1]) + (acc[2] + acc[3])) +
                                         ((acc[4] + acc[5]) + (acc[6] + acc[7])));
    const float mean = sum / (float)kK;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xf[j][e] = xf[j][e] - mean;
        acc[e] = __builtin_fmaf(xf[j][e], xf[j][e], acc[e]);
      }
    }
    const float sq = lane_sum_butterfly(((acc[0] + acc[1]) + (acc[2] + acc[3])) +
                                        ((acc[4] + acc[5]) + (acc[6] + acc[7])));
    const float rstd = 1.0f / sqrtf(sq / (float)kK + a.eps);
    if (!AMAX && lane == 0) {
      if (a.mean_out) global_ptr(a.mean_out)[r] = mean;
      if (a.rstd_out) global_ptr(a.rstd_out)[r] = rstd;
    }
    // output pass
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + kWave * j;
      const float2 o01 = planes[c], o23 = planes[kChunks + c], o45 = planes[2 * kChunks + c],
                   o67 = planes[3 * kChunks + c];
      const float2 h01 = planes[4 * kChunks + c], h23 = planes[5 * kChunks + c],
                   h45 = planes[6 * kChunks + c], h67 = planes[7 * kChunks + c];
      const float opl[8] = {o01.x, o01.y, o23.x, o23.y, o45.x, o45.y, o67.x, o67.y};
      const float sh[8] = {h01.x, h01.y, h23.x, h23.y, h45.x, h45.y, h67.x, h67.y};
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = ((xf[j][e] * rstd) * opl[e]) + sh[e];
      if (AMAX) {
        lane_amax = fold_abs8(lane_amax, y);
        continue;
      }
      const uint32_t lo = fp8_quad(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
      const uint32_t hi = fp8_quad(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
      store_stream(a.codes + r * kChunks + c, make_uint2(lo, hi));
      if (MODE == kCodesAndY) {
        store_stream(a.y_out + 2 * (r * kChunks + c), make_float4(y[0], y[1], y[2], y[3]));
        store_stream(a.y_out + 2 * (r * kChunks + c) + 1, make_float4(y[4], y[5], y[6], y[7]));
      }
    }
    // the old row's registers are free before the next row is unpacked into them
    __builtin_amdgcn_sched_barrier(0);
    unpack_sum(xr, xf, acc);
    __builtin_amdgcn_s_barrier();
  }
  if (AMAX) workgroup_max_to(a.amax_out, lane_amax, amax_red, kWaves);
}

// The per-call scale: amax (folded by the amax pass) -> amax / 448, in place.
__global__ void amax_to_fp8_scale_kernel(float* s) {
  if (threadIdx.x == 0) *global_ptr(s) = *global_ptr(s) / 448.0f;
}

template <int CPL, int MODE>
hipError_t launch_mode(const LnArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lds = (size_t)8 * CPL * kWave * sizeof(float2);
  int64_t grid = (a.m + kWaves - 1) / kWaves;
  if (grid > dev.cu_count) grid = dev.cu_count;
  hipLaunchKernelGGL((ln_fp8_kernel<CPL, MODE>), dim3((uint32_t)grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int CPL, bool AMAX>
hipError_t launch_cpl(const LnArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  if (AMAX) return launch_mode<CPL, kAmaxPass>(a, dev, stream);
  if (a.y_out) return launch_mode<CPL, kCodesAndY>(a, dev, stream);
  return launch_mode<CPL, kCodes>(a, dev, stream);
}

template <bool AMAX>
hipError_t launch_pass(const LnArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  switch (a.k / 512) {
    case 1: return launch_cpl<1, AMAX>(a, dev, stream);
    case 2: return launch_cpl<2, AMAX>(a, dev, stream);
    case 3: return launch_cpl<3, AMAX>(a, dev, stream);
    case 4: return launch_cpl<4, AMAX>(a, dev, stream);
    case 5: return launch_cpl<5, AMAX>(a, dev, stream);
    case 6: return launch_cpl<6, AMAX>(a, dev, stream);
    case 7: return launch_cpl<7, AMAX>(a, dev, stream);
    case 8: return launch_cpl<8, AMAX>(a, dev, stream);
    case 9: return launch_cpl<9, AMAX>(a, dev, stream);
    case 10: return launch_cpl<10, AMAX>(a, dev, stream);
    case 11: return launch_cpl<11, AMAX>(a, dev, stream);
    case 12: return launch_cpl<12, AMAX>(a, dev, stream);
    case 13: return launch_cpl<13, AMAX>(a, dev, stream);
    case 14: return launch_cpl<14, AMAX>(a, dev, stream);
    case 15: return launch_cpl<15, AMAX>(a, dev, stream);
    default: return launch_cpl<16, AMAX>(a, dev, stream);
  }
}

template <int CPL>
hipError_t allow_cpl() {
  const int lds = 8 * CPL * kWave * (int)sizeof(float2);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ln_fp8_kernel<CPL, kAmaxPass>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ln_fp8_kernel<CPL, kCodes>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ln_fp8_kernel<CPL, kCodesAndY>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  return e;
}

}  // namespace

hipError_t prepare_ln_fp8() {
  hipError_t e = hipSuccess;
  // 64 KiB of parameters from k = 8192 (CPL 16); smaller rows stay under the default limit
  if (e == hipSuccess) e = allow_cpl<9>();
  if (e == hipSuccess) e = allow_cpl<10>();
  if (e == hipSuccess) e = allow_cpl<11>();
  if (e == hipSuccess) e = allow_cpl<12>();
  if (e == hipSuccess) e = allow_cpl<13>();
  if (e == hipSuccess) e = allow_cpl<14>();
  if (e == hipSuccess) e = allow_cpl<15>();
  if (e == hipSuccess) e = allow_cpl<16>();
  return e;
}

hipError_t launch_ln_fp8(const LnFp8Launch& p, const DeviceInfo& dev, hipStream_t stream) {
  LnArgs a;
  a.x = static_cast<const uint4*>(p.x);
  a.scale = p.scale;
  a.shift = p.shift;
  a.eps = p.eps;
  a.m = p.m;
  a.k = p.k;
  a.act_scale = p.act_scale;
  a.scale_dev = nullptr;
  a.amax_out = nullptr;
  a.codes = static_cast<uint2*>(p.codes);
  a.mean_out = p.mean_out;
  a.rstd_out = p.rstd_out;
  a.y_out = static_cast<float4*>(static_cast<void*>(p.y_out));
  if (p.scale_dev) {
    // per-call scale: zero it, fold max |y| into it, turn it into amax / 448, quantize
    hipError_t e = launch_zero_amax(p.scale_dev, stream);
    if (e != hipSuccess) return e;
    LnArgs pass = a;
    pass.codes = nullptr;
    pass.mean_out = nullptr;
    pass.rstd_out = nullptr;
    pass.y_out = nullptr;
    pass.act_scale = 1.0f;
    pass.amax_out = p.scale_dev;
    e = launch_pass<true>(pass, dev, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(amax_to_fp8_scale_kernel, dim3(1), dim3(64), 0, stream, p.scale_dev);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.scale_dev = p.scale_dev;
  }
  return launch_pass<false>(a, dev, stream);
}

}  // namespace nvfp4act
