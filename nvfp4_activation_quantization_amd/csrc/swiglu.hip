// swiglu.hip -- SwiGLU producer -> NVFP4 (FastVideo API page, swiglu_quantize over a
// value-first [M, 2F] projection; TensorRT-LLM PR #21483, SiLU-and-mul producer):
//   y = bf16(S[gate] * up),  S[g] = bf16(g * sigmoid(g)) correctly rounded
// followed by the NVFP4 block quantizer.
//
// S is a 65,536-entry bf16 table indexed by the gate's bit pattern, built once per
// device in fp64 by silu_table_kernel.  Each workgroup (one per CU, persistent over a
// contiguous range of rows) copies the 128 KiB table into LDS; every element then costs
// one LDS lookup, one multiply and one bf16 rounding before the quantizer.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

__device__ uint16_t g_silu_table[65536];
__device__ unsigned int g_silu_ambiguous;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;
constexpr size_t kTableBytes = 65536 * sizeof(uint16_t);

// Round hi + lo to bf16, nearest-even.  lo is a tiny residual that only breaks an exact
// tie of hi; otherwise a value within 2^-36 of a midpoint (in units of the bf16 quantum)
// is counted as undecidable by the fp64 evaluation.
__device__ uint32_t round_to_bf16(double hi, double lo, unsigned int* ambiguous) {
  const uint32_t sign = __builtin_signbit(hi) ? 0x8000u : 0u;
  const double a = fabs(hi);
  if (a == 0.0) return sign;
  const int e = ilogb(a);                                // 2^e <= a < 2^(e+1)
  const int qexp = e < -126 ? -133 : e - 7;              // bf16 quantum exponent
  const double n = ldexp(a, -qexp);                      // exact scaling
  const double fl = floor(n);
  const double frac = n - fl;
  bool up;
  if (frac == 0.5 && lo != 0.0) {
    up = (lo > 0.0) == (hi > 0.0);                       // residual moves the magnitude
  } else {
    if (fabs(frac - 0.5) < 0x1p-36) atomicAdd(ambiguous, 1u);
    up = frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0);
  }
  const float v = (float)ldexp(up ? fl + 1.0 : fl, qexp); // <= 9 significant bits
  return sign | (__float_as_uint(v) >> 16);
}

// One thread per bf16 pattern.  For |g| < 2^-30, e^-g rounds to 1 in fp64 and g/2 can sit
// exactly on a bf16 midpoint; there silu(g) = g/2 + (g/2) tanh(g/2) and the second term,
// about (g/2)^2 > 0, decides the tie.
__global__ void silu_table_kernel() {
  const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= 65536u) return;
  const uint32_t ex = (g >> 7) & 0xFFu, mant = g & 0x7Fu;
  uint32_t out;
  if (ex == 0xFFu) {
    out = mant ? 0x7FC0u : ((g & 0x8000u) ? 0x8000u : 0x7F80u);
  } else {
    const double x = (double)__uint_as_float(g << 16);
    double hi, lo;
    if (fabs(x) < 0x1p-30) {
      hi = 0.5 * x;
      lo = hi * hi;
    } else {
      hi = x / (1.0 + exp(-x));
      lo = 0.0;
    }
    out = round_to_bf16(hi, lo, &g_silu_ambiguous);
  }
  g_silu_table[g] = (uint16_t)out;
}

// SwiGLU + quantize of kUnroll x 64 consecutive chunks of one row starting at chunk c0.
template <bool Tail>
__device__ __forceinline__ void swiglu_span(const NVFP4_GLOBAL uint4* ur, const NVFP4_GLOBAL uint4* gr,
                                            NVFP4_GLOBAL uint32_t* cr, NVFP4_GLOBAL uint8_t* sr,
                                            NVFP4_GLOBAL uint4* yr, int64_t c0, int64_t chunks, int lane,
                                            const uint16_t* table, float gsf, const float* inv_tab) {
  uint4 u[kUnroll], g[kUnroll];
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int64_t c = c0 + i * kWave + lane;
    if (!Tail || c < chunks) {
      u[i] = load_stream(reinterpret_cast<const uint4*>(ur + c));
      g[i] = load_stream(reinterpret_cast<const uint4*>(gr + c));
    } else {
      u[i] = make_uint4(0, 0, 0, 0);
      g[i] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int64_t c = c0 + i * kWave + lane;
    const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
    const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
    float y[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float s0 = __uint_as_float((uint32_t)table[gw[q] & 0xFFFFu] << 16);
      const float s1 = __uint_as_float((uint32_t)table[gw[q] >> 16] << 16);
      y[2 * q] = round_bf16(s0 * bf16_lo(uw[q]));
      y[2 * q + 1] = round_bf16(s1 * bf16_hi(uw[q]));
    }
    uint32_t s;
    const uint32_t code = quantize_chunk(y, gsf, inv_tab, &s);
    if (!Tail || c < chunks) {
      cr[c0 + i * kWave] = code;
      sr[(c0 / 8 + 8 * i) * 512] = (uint8_t)s;
      if (yr)
        yr[c0 + i * kWave] = make_uint4(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]),
                                        pack_exact_bf16x2(y[4], y[5]), pack_exact_bf16x2(y[6], y[7]));
    }
  }
}

__global__ __launch_bounds__(kThreads) void swiglu_kernel(const uint4* __restrict__ up,
                                                          const uint4* __restrict__ gate, int64_t ld8,
                                                          int64_t m, int64_t f, int64_t padded,
                                                          float global_amax, uint32_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint4* y_out,
                                                          int64_t rows_per_xcd) {
  extern __shared__ uint4 lds4[];
  uint16_t* table = reinterpret_cast<uint16_t*>(lds4);
  float* inv_tab = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lds4) + kTableBytes);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  const XcdSteps st = xcd_steps(rows_per_xcd, padded, kWaves);
  if (st.first >= st.end) return;                         // idle workgroup (uniform)

  const float gsf = global_scale(global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  const uint4* src = reinterpret_cast<const uint4*>(g_silu_table);
  for (int i = tid; i < (int)(kTableBytes / 16); i += kThreads) lds4[i] = src[i];
  __syncthreads();

  const int64_t chunks = f >> 3;
  const int64_t span = kWave * kUnroll;
  const int64_t full = chunks / span * span;
  for (int64_t g = st.first; g < st.end; g += st.step) {
    const int64_t r = g + wave;
    if (r >= st.end) break;
    if (r >= m) {
      zero_row_scales(scales, r, f, lane);
      continue;
    }
    const NVFP4_GLOBAL uint4* ur = global_ptr(up) + r * ld8;
    const NVFP4_GLOBAL uint4* gr = global_ptr(gate) + r * ld8;
    NVFP4_GLOBAL uint32_t* cr = global_ptr(codes) + r * chunks + lane;
    NVFP4_GLOBAL uint8_t* sr = global_ptr(scales) + row_scale_base(r, f) + scale_lane_offset(lane);
    NVFP4_GLOBAL uint4* yr = y_out ? global_ptr(y_out) + r * chunks + lane : nullptr;
    for (int64_t c0 = 0; c0 < full; c0 += span)
      swiglu_span<false>(ur, gr, cr, sr, yr, c0, chunks, lane, table, gsf, inv_tab);
    if (full < chunks) swiglu_span<true>(ur, gr, cr, sr, yr, full, chunks, lane, table, gsf, inv_tab);
  }
}

}  // namespace

hipError_t build_silu_table(unsigned int* ambiguous) {
  const unsigned int zero = 0;
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_silu_ambiguous), &zero, sizeof zero);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(silu_table_kernel, dim3(256), dim3(256), 0, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  return hipMemcpyFromSymbol(ambiguous, HIP_SYMBOL(g_silu_ambiguous), sizeof *ambiguous);
}

hipError_t prepare_swiglu() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&swiglu_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kTableBytes + 512));
}

hipError_t launch_swiglu(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f,
                         float global_amax, void* codes, void* scales, void* y_out,
                         const DeviceInfo& dev, hipStream_t stream) {
  const int64_t padded = (m + 127) / 128 * 128;
  int64_t wgs_per_xcd = 0, rows_per_xcd = 0;
  plan_xcd_steps(padded, dev.cu_count, kWaves, &wgs_per_xcd, &rows_per_xcd);
  const int64_t units = wgs_per_xcd * kXcds;
  hipLaunchKernelGGL(swiglu_kernel, dim3((uint32_t)units), dim3(kThreads), kTableBytes + 512, stream,
                     static_cast<const uint4*>(up), static_cast<const uint4*>(gate), ld / 8, m, f, padded,
                     global_amax, static_cast<uint32_t*>(codes), static_cast<uint8_t*>(scales),
                     static_cast<uint4*>(y_out), rows_per_xcd);
  return hipGetLastError();
}

}  // namespace nvfp4act
