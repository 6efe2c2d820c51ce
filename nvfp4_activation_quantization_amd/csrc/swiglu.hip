// swiglu.hip -- SwiGLU producer -> NVFP4 (FastVideo API page, swiglu_quantize over a
// value-first [M, 2F] projection; TensorRT-LLM PR #21483, SiLU-and-mul producer):
//   y = bf16(S[gate] * up),  S[g] = bf16(g * sigmoid(g)) correctly rounded
// followed by the NVFP4 block quantizer.
//
// S is a 65,536-entry bf16 table indexed by the gate's bit pattern, built once per
// device in fp64 by silu_table_kernel.  Each workgroup (one per CU, persistent over a
// set of 128-row x 512-column tiles) copies the 128 KiB table into LDS; every element then
// costs one LDS lookup, one multiply and one bf16 rounding before the quantizer.  Each
// tile's scale bytes are gathered in LDS and leave with 16-byte stores.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

__device__ uint16_t g_silu_table[65536];
__device__ unsigned int g_silu_ambiguous;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kTableBytes = 65536 * sizeof(uint16_t);
constexpr int kTileCols = 512;                     // 64 chunks: one per lane per row
constexpr int kRowBatch = 4;                       // rows per wavefront in flight
constexpr int kScaleBytes = kTileCols / 64 * 512;  // 4 KiB

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

// One 128-row x kTileCols tile: each wavefront takes rows wave, wave + 16, ... (8 rows),
// kRowBatch at a time; scale bytes go to the tile's LDS block.  AMAX (the amax pass of a
// per-call scale): nothing is quantized or stored; max |y| is folded into *lane_amax.
template <bool AMAX>
__device__ __forceinline__ void swiglu_tile(const uint4* up, const uint4* gate, int64_t ld8, int64_t m,
                                            int64_t row_chunks, uint32_t* codes, uint4* y_out,
                                            int64_t tile_row, int64_t c0, int64_t tchunks, int lane, int wave,
                                            const uint16_t* table, float gsf, const float* inv_tab,
                                            uint8_t* sc_lane, float* lane_amax) {
  const int64_t r0 = tile_row << 7;
  const int64_t rows = (m - r0 < 128) ? (m - r0 > 0 ? m - r0 : 0) : 128;
  const int64_t c = c0 + lane;
  const bool lane_ok = lane < tchunks;
  for (int64_t rb = wave * kRowBatch; rb < rows; rb += kWaves * kRowBatch) {
    uint4 u[kRowBatch], g[kRowBatch];
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t r = r0 + rb + i;
      if (rb + i < rows && lane_ok) {
        u[i] = load_stream(reinterpret_cast<const uint4*>(global_ptr(up) + r * ld8 + c));
        g[i] = load_stream(reinterpret_cast<const uint4*>(global_ptr(gate) + r * ld8 + c));
      } else {
        u[i] = make_uint4(0, 0, 0, 0);
        g[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t rr = rb + i;
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
      if (AMAX) {
        // lanes past the real rows or columns loaded zeros, whose y is 0
        *lane_amax = fold_abs8(*lane_amax, y);
        continue;
      }
      uint32_t s;
      const uint32_t code = quantize_chunk(y, gsf, inv_tab, &s);
      if (rr < rows && lane_ok) {
        const int64_t r = r0 + rr;
        global_ptr(codes)[r * row_chunks + c] = code;
        sc_lane[(rr & 31) * 16 + ((rr >> 5) & 3) * 4] = (uint8_t)s;
        if (y_out)
          global_ptr(y_out)[r * row_chunks + c] =
              make_uint4(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]),
                         pack_exact_bf16x2(y[4], y[5]), pack_exact_bf16x2(y[6], y[7]));
      }
    }
  }
}

template <bool AMAX>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const uint4* __restrict__ up,
                                                          const uint4* __restrict__ gate, int64_t ld8,
                                                          int64_t m, int64_t f, float global_amax,
                                                          const float* amax_dev, float* amax_out,
                                                          uint32_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint4* y_out,
                                                          int64_t col_tiles, int64_t ntiles) {
  __shared__ float amax_red[kWaves];
  extern __shared__ uint4 lds4[];
  uint16_t* table = reinterpret_cast<uint16_t*>(lds4);
  float* inv_tab = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(lds4) + kTableBytes);
  uint4* tile_sc = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(lds4) + kTableBytes + 512);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if ((int64_t)blockIdx.x >= ntiles) return;              // idle workgroup (uniform)

  const float gsf = call_global_scale(global_amax, amax_dev);
  float lane_amax = 0.0f;
  fill_inverse_table(inv_tab, gsf, tid);
  const uint4* src = reinterpret_cast<const uint4*>(g_silu_table);
  for (int i = tid; i < (int)(kTableBytes / 16); i += kThreads) lds4[i] = src[i];
  for (int i = tid; i < kScaleBytes / 16; i += kThreads) tile_sc[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int64_t row_chunks = f >> 3;
  uint8_t* sc_lane = reinterpret_cast<uint8_t*>(tile_sc) + scale_lane_offset(lane);
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t tile_row = t / col_tiles, col_tile = t % col_tiles;
    const int64_t c0 = col_tile * (kTileCols / 8);
    const int64_t tchunks = (row_chunks - c0 < kTileCols / 8) ? row_chunks - c0 : kTileCols / 8;
    swiglu_tile<AMAX>(up, gate, ld8, m, row_chunks, codes, y_out, tile_row, c0, tchunks, lane, wave, table, gsf,
                      inv_tab, sc_lane, &lane_amax);
    if (AMAX) continue;
    __syncthreads();
    // copy the tile's scale slice out and zero it for the next tile (each thread clears
    // exactly the words it copied)
    NVFP4_GLOBAL uint4* dst = reinterpret_cast<NVFP4_GLOBAL uint4*>(
        global_ptr(scales) + (tile_row * (f >> 6) + c0 / 8) * 512);
    const int words = (int)(tchunks / 8) * 32;
    for (int i = tid; i < words; i += kThreads) {
      dst[i] = tile_sc[i];
      tile_sc[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  }
  if (AMAX) workgroup_max_to(amax_out, lane_amax, amax_red, kWaves);
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
  const int lds = (int)(kTableBytes + 512 + kScaleBytes);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&swiglu_kernel<false>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&swiglu_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  return e;
}

hipError_t launch_swiglu(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f,
                         float global_amax, float* amax_dev, void* codes, void* scales, void* y_out,
                         const DeviceInfo& dev, hipStream_t stream) {
  const int64_t tile_rows = (m + 127) / 128;
  const int64_t col_tiles = (f + kTileCols - 1) / kTileCols;
  const int64_t ntiles = tile_rows * col_tiles;
  const int64_t grid = ntiles < dev.cu_count ? ntiles : dev.cu_count;
  const size_t lds = kTableBytes + 512 + kScaleBytes;
  const uint4* u = static_cast<const uint4*>(up);
  const uint4* g = static_cast<const uint4*>(gate);
  if (amax_dev) {
    // per-call scale: zero the amax, fold max |y| into it, then quantize with it
    hipError_t e = launch_zero_amax(amax_dev, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(swiglu_kernel<true>, dim3((uint32_t)grid), dim3(kThreads), lds, stream, u, g, ld / 8, m, f,
                       global_amax, nullptr, amax_dev, nullptr, nullptr, nullptr, col_tiles, ntiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(swiglu_kernel<false>, dim3((uint32_t)grid), dim3(kThreads), lds, stream, u, g, ld / 8, m, f,
                     global_amax, amax_dev, nullptr, static_cast<uint32_t*>(codes), static_cast<uint8_t*>(scales),
                     static_cast<uint4*>(y_out), col_tiles, ntiles);
  return hipGetLastError();
}

}  // namespace nvfp4act
