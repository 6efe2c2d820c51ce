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

__global__ __launch_bounds__(kThreads) void swiglu_kernel(const uint4* __restrict__ up,
                                                          const uint4* __restrict__ gate, int64_t ld8,
                                                          int64_t m, int64_t f, int64_t padded,
                                                          float global_amax, uint32_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint4* y_out,
                                                          int64_t rows_per_unit, int64_t per) {
  extern __shared__ uint4 lds4[];
  uint16_t* table = reinterpret_cast<uint16_t*>(lds4);
  float* inv_tab = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lds4) + kTableBytes);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const GatherAddr ga = scale_gather_addresses(lane);

  const int64_t unit = xcd_unit(per);
  const int64_t r_begin = unit * rows_per_unit;
  if (r_begin >= padded) return;                          // idle workgroup (uniform)
  const int64_t r_end = (r_begin + rows_per_unit < padded) ? r_begin + rows_per_unit : padded;

  const float gsf = global_scale(global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  const uint4* src = reinterpret_cast<const uint4*>(g_silu_table);
  for (int i = tid; i < (int)(kTableBytes / 16); i += kThreads) lds4[i] = src[i];
  __syncthreads();

  const int64_t chunks = f >> 3;
  for (int64_t r = r_begin + wave; r < r_end; r += kWaves) {
    if (r >= m) {
      zero_row_scales(scales, r, f, lane);
      continue;
    }
    const uint4* ur = up + r * ld8;
    const uint4* gr = gate + r * ld8;
    const int64_t sbase = row_scale_base(r, f);
    for (int64_t c0 = 0; c0 < chunks; c0 += kWave * kUnroll) {
      uint4 u[kUnroll], g[kUnroll];
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const int64_t c = c0 + i * kWave + lane;
        const bool ok = c < chunks;
        u[i] = ok ? load_stream(ur + c) : make_uint4(0, 0, 0, 0);
        g[i] = ok ? load_stream(gr + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kUnroll; ++i) {
        const int64_t c = c0 + i * kWave + lane;
        const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
        const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
        float y[8];
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float s0 = __uint_as_float((uint32_t)table[gw[q] & 0xFFFFu] << 16);
          const float s1 = __uint_as_float((uint32_t)table[gw[q] >> 16] << 16);
          y[2 * q] = round_bf16(s0 * bf16_lo(uw[q]));
          y[2 * q + 1] = round_bf16(s1 * bf16_hi(uw[q]));
          p[q] = pack_exact_bf16x2(y[2 * q], y[2 * q + 1]);
        }
        uint32_t s;
        const uint32_t code = quantize_chunk(y, gsf, inv_tab, &s);
        const uint32_t s4 = gather_scales4(s, ga);
        if (c < chunks) {
          codes[r * chunks + c] = code;
          if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(scales + sbase + c * 64) = s4;
          if (y_out) y_out[r * chunks + c] = make_uint4(p[0], p[1], p[2], p[3]);
        }
      }
    }
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
  const int64_t groups = (padded + kWaves - 1) / kWaves;
  int64_t units = dev.cu_count < groups ? dev.cu_count : groups;
  const int64_t per = (units + kXcds - 1) / kXcds;
  units = per * kXcds;
  const int64_t rows_per_unit = (padded + units - 1) / units;
  hipLaunchKernelGGL(swiglu_kernel, dim3((uint32_t)units), dim3(kThreads), kTableBytes + 512, stream,
                     static_cast<const uint4*>(up), static_cast<const uint4*>(gate), ld / 8, m, f, padded,
                     global_amax, static_cast<uint32_t*>(codes), static_cast<uint8_t*>(scales),
                     static_cast<uint4*>(y_out), rows_per_unit, per);
  return hipGetLastError();
}

}  // namespace nvfp4act
