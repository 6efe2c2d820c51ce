// rms_silu.hip -- channels-last RMSNorm + SiLU -> NVFP4 of fp16 activations (FlashRT PR
// #142, fp16_quant_nvfp4_ndhwc: the fused RMS_norm + SiLU + NVFP4 quantize of the VAE's
// channels-last tensors; the RMSNorm+RoPE kernel's fp32 statistics with an fp16 affine):
// per voxel row of c channels,
//   rstd = 1 / sqrt(sum(x^2) / c + eps)      fp32, the slot tree below
//   a    = fp16(fp16(x * rstd) * gamma)
//   y    = S16[a]                            S16[g] = fp16(g * sigmoid(g)) correctly rounded
// followed by the NVFP4 block quantizer over the channels.  Scale bytes are written in
// plain row order, [rows, c/16] (a channels-last operand; no GEMM swizzle).
//
// Rows are short (c <= 512 channels, 16..64 chunks of 8), so a wavefront holds several:
// with S = the smallest power of two >= c/8, lane L takes chunk L % S of row L / S, and
// lanes whose chunk lies past c/8 hold zeros.  The statistic is the fixed tree of the
// specification: each lane folds its 8 squares pairwise, then a butterfly over the S lanes
// of the row (distances 1 .. S/2).  A 16-channel block is the chunk pair on lanes (L, L^1),
// as in the other producers.
//
// One 1024-thread workgroup per CU, persistent over groups of rows; the 128 KiB fp16 SiLU
// table (built once per device in fp64, like the bf16 one) is copied into LDS; each lane's
// 8 gamma values stay in registers (a lane's chunk index never changes).
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

__device__ uint16_t g_silu16_table[65536];
__device__ unsigned int g_silu16_ambiguous;

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kTableBytes = 65536 * sizeof(uint16_t);
constexpr int kUnroll = 4;                 // row groups per wavefront in flight

// Round hi + lo to fp16, nearest-even (quantum 2^(E-10) for 2^E <= |v| < 2^(E+1), E >= -14,
// subnormal quantum 2^-24; infinity from 65520 up).  lo only breaks an exact tie of hi; a
// value within 2^-36 quanta of a midpoint is counted as undecidable by fp64.
__device__ uint32_t round_to_f16(double hi, double lo, unsigned int* ambiguous) {
  const uint32_t sign = __builtin_signbit(hi) ? 0x8000u : 0u;
  const double a = fabs(hi);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return sign | 0x7C00u;
  const int e = ilogb(a);
  const int qexp = e < -14 ? -24 : e - 10;
  const double n = ldexp(a, -qexp);
  const double fl = floor(n);
  const double frac = n - fl;
  bool up;
  if (frac == 0.5 && lo != 0.0) {
    up = (lo > 0.0) == (hi > 0.0);
  } else {
    if (fabs(frac - 0.5) < 0x1p-36) atomicAdd(ambiguous, 1u);
    up = frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0);
  }
  // the rounded magnitude (<= 11 significant bits) as fp16: exact conversion
  const _Float16 h = (_Float16)(float)ldexp(up ? fl + 1.0 : fl, qexp);
  return sign | (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// One thread per fp16 pattern; |g| < 2^-30 through g/2 + (g/2) tanh(g/2) as for bf16.
__global__ void silu16_table_kernel() {
  const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= 65536u) return;
  const uint32_t ex = (g >> 10) & 0x1Fu, mant = g & 0x3FFu;
  uint32_t out;
  if (ex == 0x1Fu) {
    out = mant ? 0x7E00u : ((g & 0x8000u) ? 0x8000u : 0x7C00u);
  } else {
    const double x = (double)(float)__builtin_bit_cast(_Float16, (uint16_t)g);
    double hi, lo;
    if (fabs(x) < 0x1p-30) {
      hi = 0.5 * x;
      lo = hi * hi;
    } else {
      hi = x / (1.0 + exp(-x));
      lo = 0.0;
    }
    out = round_to_f16(hi, lo, &g_silu16_ambiguous);
  }
  g_silu16_table[g] = (uint16_t)out;
}

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
// fp16(f) and its bit pattern (round to nearest even: the default mode)
__device__ __forceinline__ uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float round_f16(float f) { return (float)(_Float16)f; }

// Butterfly sum over the S lanes of a row (distances 1 .. S/2; S = 16, 32 or 64), as
// lane_sum_butterfly for the first log2(S) steps.
template <int S>
__device__ __forceinline__ float slot_sum_butterfly(float v) {
  uint32_t u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0xB1, 0xF, 0xF, false));
  u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x4E, 0xF, 0xF, false));
  u = __float_as_uint(v);
  int t = __builtin_amdgcn_update_dpp((int)u, (int)u, 0x104, 0xF, 0x5, false);   // banks 0, 2: lane + 4
  t = __builtin_amdgcn_update_dpp(t, (int)u, 0x114, 0xF, 0xA, false);            // banks 1, 3: lane - 4
  v = v + __uint_as_float((uint32_t)t);
  u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x128, 0xF, 0xF, false));
  if (S >= 32) {
    u = __float_as_uint(v);
    const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  }
  if (S >= 64) {
    u = __float_as_uint(v);
    const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  }
  return v;
}

struct RsArgs {
  const uint4* x;           // [rows, c] fp16, 16-byte chunks
  const uint4* gamma;       // [c] fp16
  float eps;
  int64_t rows, c;
  float global_amax;
  const float* amax_dev;    // per-call scale: the amax pass's result (null: static global_amax)
  float* amax_out;          // the amax pass: where max |y| is folded
  uint32_t* codes;          // one word (8 codes) per chunk
  uint8_t* scales;          // [rows, c/16]
  float* rstd_out;
  uint4* y_out;             // [rows, c] fp16
};

// S: slots (lanes) per row.  AMAX: the amax pass -- the same chain, no stores.
template <int S, bool AMAX>
__global__ __launch_bounds__(kThreads) void rms_silu_kernel(const RsArgs a) {
  constexpr int R = kWave / S;             // rows per wavefront step
  __shared__ float inv_tab[128];
  __shared__ float amax_red[kWaves];
  extern __shared__ uint4 lds4[];
  const uint16_t* table = reinterpret_cast<const uint16_t*>(lds4);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int chunk = lane % S, sub = lane / S;
  const int64_t chunks = a.c >> 3;
  const bool lane_ok = chunk < chunks;

  const float gsf = call_global_scale(a.global_amax, a.amax_dev);
  if (!AMAX) fill_inverse_table(inv_tab, gsf, tid);
  const uint4* src = reinterpret_cast<const uint4*>(g_silu16_table);
  for (int i = tid; i < (int)(kTableBytes / 16); i += kThreads) lds4[i] = src[i];
  uint4 gv = make_uint4(0, 0, 0, 0);
  if (lane_ok) gv = global_ptr(a.gamma)[chunk];
  const float g8[8] = {f16_lo(gv.x), f16_hi(gv.x), f16_lo(gv.y), f16_hi(gv.y),
                       f16_lo(gv.z), f16_hi(gv.z), f16_lo(gv.w), f16_hi(gv.w)};
  __syncthreads();

  float lane_amax = 0.0f;
  const int64_t groups = (a.rows + R - 1) / R;
  const int64_t step = (int64_t)gridDim.x * kWaves;
  // per-lane offsets within a row group (32-bit); the group's base is wave-uniform
  const int lane_chunk = sub * (int)chunks + chunk;
  const int lane_block = sub * (int)(a.c >> 4) + (chunk >> 1);
  for (int64_t g0 = (int64_t)blockIdx.x * kWaves + wave; g0 < groups; g0 += step * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r0 = (g0 + step * u) * R;                        // wave-uniform
      const int64_t r = r0 + sub;
      v[u] = (lane_ok && r < a.rows) ? load_stream(a.x + r0 * chunks + lane_chunk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r0 = (g0 + step * u) * R;
      const int64_t r = r0 + sub;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float x8[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x8[2 * q] = f16_lo(w[q]);
        x8[2 * q + 1] = f16_hi(w[q]);
      }
      float sq[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sq[e] = x8[e] * x8[e];         // exact for fp16 inputs
      const float lane_v = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
      const float sum = slot_sum_butterfly<S>(lane_v);
      const float rstd = 1.0f / sqrtf(sum / (float)a.c + a.eps);
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // the product rounded to fp32 first, then to fp16: without the opaque step the
        // compiler forms one v_fma_mix (a single rounding of the exact product to fp16)
        float p = x8[e] * rstd;
        asm volatile("" : "+v"(p));
        const float nn = round_f16(p);
        const uint32_t ab = f16_bits(nn * g8[e]);
        y[e] = (float)__builtin_bit_cast(_Float16, table[ab]);
      }
      const bool row_ok = r < a.rows;
      if (AMAX) {
        if (row_ok && lane_ok) lane_amax = fold_abs8(lane_amax, y);
        continue;
      }
      uint32_t s;
      const uint32_t code = quantize_chunk(y, gsf, inv_tab, &s);
      if (row_ok && lane_ok) {
        global_ptr(a.codes + r0 * chunks)[lane_chunk] = code;
        if ((chunk & 1) == 0) global_ptr(a.scales + r0 * (a.c >> 4))[lane_block] = (uint8_t)s;
        if (chunk == 0 && a.rstd_out) global_ptr(a.rstd_out)[r] = rstd;
        if (a.y_out)
          global_ptr(a.y_out + r0 * chunks)[lane_chunk] =
              make_uint4(f16_bits(y[0]) | (f16_bits(y[1]) << 16), f16_bits(y[2]) | (f16_bits(y[3]) << 16),
                         f16_bits(y[4]) | (f16_bits(y[5]) << 16), f16_bits(y[6]) | (f16_bits(y[7]) << 16));
      }
    }
  }
  if (AMAX) workgroup_max_to(a.amax_out, lane_amax, amax_red, kWaves);
}

template <int S, bool AMAX>
hipError_t launch_s(const RsArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int R = kWave / S;
  const int64_t groups = (a.rows + R - 1) / R;
  int64_t grid = (groups + kWaves - 1) / kWaves;
  if (grid > dev.cu_count) grid = dev.cu_count;
  hipLaunchKernelGGL((rms_silu_kernel<S, AMAX>), dim3((uint32_t)grid), dim3(kThreads), kTableBytes, stream, a);
  return hipGetLastError();
}

template <bool AMAX>
hipError_t launch_pass(const RsArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  const int64_t chunks = a.c >> 3;
  if (chunks <= 16) return launch_s<16, AMAX>(a, dev, stream);
  if (chunks <= 32) return launch_s<32, AMAX>(a, dev, stream);
  return launch_s<64, AMAX>(a, dev, stream);
}

template <int S, bool AMAX>
hipError_t allow_lds_s() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&rms_silu_kernel<S, AMAX>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTableBytes);
}

}  // namespace

hipError_t build_silu16_table(unsigned int* ambiguous) {
  const unsigned int zero = 0;
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_silu16_ambiguous), &zero, sizeof zero);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(silu16_table_kernel, dim3(256), dim3(256), 0, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  return hipMemcpyFromSymbol(ambiguous, HIP_SYMBOL(g_silu16_ambiguous), sizeof *ambiguous);
}

hipError_t prepare_rms_silu() {
  hipError_t e = allow_lds_s<16, false>();
  if (e == hipSuccess) e = allow_lds_s<16, true>();
  if (e == hipSuccess) e = allow_lds_s<32, false>();
  if (e == hipSuccess) e = allow_lds_s<32, true>();
  if (e == hipSuccess) e = allow_lds_s<64, false>();
  if (e == hipSuccess) e = allow_lds_s<64, true>();
  return e;
}

hipError_t launch_rms_silu(const RmsSiluLaunch& p, const DeviceInfo& dev, hipStream_t stream) {
  RsArgs a;
  a.x = static_cast<const uint4*>(p.x);
  a.gamma = static_cast<const uint4*>(p.gamma);
  a.eps = p.eps;
  a.rows = p.rows;
  a.c = p.c;
  a.global_amax = p.global_amax;
  a.amax_dev = nullptr;
  a.amax_out = nullptr;
  a.codes = static_cast<uint32_t*>(p.codes);
  a.scales = static_cast<uint8_t*>(p.scales);
  a.rstd_out = p.rstd_out;
  a.y_out = static_cast<uint4*>(p.y_out);
  if (p.amax_dev) {
    hipError_t e = launch_zero_amax(p.amax_dev, stream);
    if (e != hipSuccess) return e;
    RsArgs pass = a;
    pass.codes = nullptr;
    pass.scales = nullptr;
    pass.rstd_out = nullptr;
    pass.y_out = nullptr;
    pass.amax_out = p.amax_dev;
    e = launch_pass<true>(pass, dev, stream);
    if (e != hipSuccess) return e;
    a.amax_dev = p.amax_dev;
  }
  return launch_pass<false>(a, dev, stream);
}

}  // namespace nvfp4act
