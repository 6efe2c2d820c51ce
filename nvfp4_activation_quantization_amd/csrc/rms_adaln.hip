// rms_adaln.hip -- fused RMSNorm (fp32 statistic) + adaLN modulation -> NVFP4, the
// AdaLN RMSNorm + modulation producer of TensorRT-LLM PR #21483, with every bf16 rounding
// of the op-by-op eager path kept (FastVideo API page, module summary):
//   rstd = 1 / sqrt(sum(x^2) / k + eps)
//   y    = bf16(bf16(bf16(bf16(x * rstd) * w) * bf16(1 + scale[t])) + shift[t])
// followed by the NVFP4 block quantizer.
//
// One workgroup of 8 wavefronts per CU, persistent over a contiguous range of rows.
// The RMSNorm weight and the current frame's modulation row are staged once in LDS as
// fp32 (bf16(1 + scale) precomputed); a frame change restages it behind two barriers.
// A row whose frame is not the staged one (possible only for unsorted frame indices)
// reads its modulation row from global memory instead.  Each wavefront holds its row in
// registers between the statistic and the output pass, so x is read from HBM once.
//
// The statistic uses the fixed tree of the specification: lane L owns chunks L + 64j,
// keeps 8 accumulators (fused multiply-add), folds them pairwise, and a butterfly over the
// 64 lanes at distances 1..32 adds the lane values (every lane ends with the same sum).
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxStagedK = 8192;       // 12 * k + 512 bytes of LDS

struct RmsArgs {
  const uint4* x;
  const uint16_t* w;
  const uint16_t* shift;
  const uint16_t* scale;
  int64_t frame_stride;
  int64_t num_frames;
  const int32_t* frame_idx;
  float eps;
  int64_t m, k, padded;
  float global_amax;
  uint32_t* codes;
  uint8_t* scales;
  float* rstd_out;
  uint4* y_out;
  uint32_t* status;
  int64_t rows_per_unit, per;
};

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Round 8 fp32 values to bf16: packed words in p, the rounded values back in f.
__device__ __forceinline__ void round8(float* f, uint32_t* p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    f[2 * i] = bf16_lo(p[i]);
    f[2 * i + 1] = bf16_hi(p[i]);
  }
}

// The statistic of a row held as per-lane chunks v[0..n) (chunk L + 64j in v[j]).
template <int N>
__device__ __forceinline__ float row_rstd(const uint4* v, int n, int64_t k, float eps) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (N == 0 && j >= n) break;
    float f[8];
    unpack8(v[j], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f[e], f[e], acc[e]);
  }
  float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) s = s + __shfl_xor(s, d, kWave);
  float ms = s / (float)k;
  return 1.0f / sqrtf(ms + eps);
}

// adaLN modulation and quantization of one chunk c of row r.
//   x8   : the chunk's 8 inputs as fp32;  w8, opl8, sh8 : parameters as fp32
__device__ __forceinline__ void emit_chunk(const RmsArgs& a, int64_t r, int64_t c, int lane,
                                           const float* x8, const float* w8, const float* opl8,
                                           const float* sh8, float rstd, float gsf,
                                           const float* inv_tab, int64_t sbase) {
  float f[8];
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = x8[e] * rstd;
  round8(f, p);                                      // n  = bf16(x * rstd)
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f[e] * w8[e];
  round8(f, p);                                      // nw = bf16(n * w)
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f[e] * opl8[e];
  round8(f, p);                                      // m  = bf16(nw * bf16(1 + scale))
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = f[e] + sh8[e];
  round8(f, p);                                      // y  = bf16(m + shift)
  uint32_t s;
  uint32_t q = quantize_chunk(f, gsf, inv_tab, &s);
  uint32_t s4 = gather_scales4(s);
  a.codes[r * (a.k >> 3) + c] = q;
  if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(a.scales + sbase + c * 64) = s4;
  if (a.y_out) a.y_out[r * (a.k >> 3) + c] = make_uint4(p[0], p[1], p[2], p[3]);
}

// Write row r as zeros (frame index outside [0, num_frames)).
__device__ void zero_row(const RmsArgs& a, int64_t r, int lane) {
  const int64_t chunks = a.k >> 3;
  for (int64_t c = lane; c < chunks; c += kWave) {
    a.codes[r * chunks + c] = 0u;
    if (a.y_out) a.y_out[r * chunks + c] = make_uint4(0, 0, 0, 0);
  }
  zero_row_scales(a.scales, r, a.k, lane);
  if (lane == 0 && a.status) atomicOr(a.status, 1u);
}

__device__ __forceinline__ void load_frame_chunk(const RmsArgs& a, int64_t t, int64_t c, float* opl8,
                                                 float* sh8) {
  uint4 sc = *reinterpret_cast<const uint4*>(a.scale + t * a.frame_stride + 8 * c);
  uint4 sh = *reinterpret_cast<const uint4*>(a.shift + t * a.frame_stride + 8 * c);
  float tmp[8];
  uint32_t p[4];
  unpack8(sc, tmp);
#pragma unroll
  for (int e = 0; e < 8; ++e) tmp[e] = 1.0f + tmp[e];
  round8(tmp, p);
#pragma unroll
  for (int e = 0; e < 8; ++e) opl8[e] = tmp[e];
  unpack8(sh, sh8);
}

// ---- the staged kernel (k <= kMaxStagedK, CPL = k / 512 chunks per lane) ------------------

// A row whose frame is not the staged one: re-read x (an L2 hit in practice) and the
// frame's modulation row from global memory, one chunk at a time.
__device__ __noinline__ void emit_row_unstaged(const RmsArgs& a, int64_t r, int64_t t, int lane,
                                               const float* w_f, float rstd, float gsf,
                                               const float* inv_tab, int64_t sbase) {
  const uint4* xr = a.x + r * (a.k >> 3);
#pragma unroll 1
  for (int64_t c = lane; c < (a.k >> 3); c += kWave) {
    float x8[8], o8[8], h8[8];
    unpack8(xr[c], x8);
    load_frame_chunk(a, t, c, o8, h8);
    emit_chunk(a, r, c, lane, x8, w_f + 8 * c, o8, h8, rstd, gsf, inv_tab, sbase);
  }
}

template <int CPL>
__device__ __forceinline__ void load_row(uint4* v, const uint4* xr, int lane) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] = load_stream(xr + lane + kWave * j);
}

template <int CPL>
__global__ __launch_bounds__(kThreads) void rms_adaln_staged(RmsArgs a) {
  extern __shared__ float lds[];
  float* inv_tab = lds;
  float* w_f = lds + 128;
  float* opl_f = w_f + a.k;
  float* sh_f = opl_f + a.k;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t chunks = a.k >> 3;

  const int64_t unit = xcd_unit(a.per);
  const int64_t r_begin = unit * a.rows_per_unit;
  if (r_begin >= a.padded) return;                      // idle workgroup (uniform)
  const int64_t r_end = (r_begin + a.rows_per_unit < a.padded) ? r_begin + a.rows_per_unit : a.padded;

  // Each wavefront double-buffers its rows: the next row's loads are in flight while the
  // current row is normalised, modulated and quantized.
  uint4 cur[CPL], nxt[CPL];
  {
    const int64_t r = r_begin + wave;
    if (r < r_end && r < a.m) load_row<CPL>(cur, a.x + r * chunks, lane);
  }

  const float gsf = global_scale(a.global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  for (int64_t c = tid; c < chunks; c += kThreads) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(a.w + 8 * c), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) w_f[8 * c + e] = f[e];
  }
  __syncthreads();

  int64_t staged = -1;
  for (int64_t g = r_begin; g < r_end; g += kWaves) {
    const int64_t r = g + wave;
    const int64_t rn = r + kWaves;
    if (rn < r_end && rn < a.m) load_row<CPL>(nxt, a.x + rn * chunks, lane);

    int64_t want = staged;
    if (g < a.m) {
      int64_t t = a.frame_idx[g];
      if (t >= 0 && t < a.num_frames) want = t;
    }
    if (want != staged) {                               // uniform over the workgroup
      __syncthreads();
      for (int64_t c = tid; c < chunks; c += kThreads) {
        float o8[8], h8[8];
        load_frame_chunk(a, want, c, o8, h8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          opl_f[8 * c + e] = o8[e];
          sh_f[8 * c + e] = h8[e];
        }
      }
      __syncthreads();
      staged = want;
    }

    if (r < r_end) {
      if (r >= a.m) {
        zero_row_scales(a.scales, r, a.k, lane);
      } else {
        const float rstd = row_rstd<CPL>(cur, CPL, a.k, a.eps);
        if (lane == 0 && a.rstd_out) a.rstd_out[r] = rstd;
        const int64_t t = a.frame_idx[r];
        if (t < 0 || t >= a.num_frames) {
          zero_row(a, r, lane);
        } else {
          const int64_t sbase = row_scale_base(r, a.k);
          // Keep the row packed between the two passes: without this the compiler keeps
          // the fp32 values unpacked for the statistic alive into the output pass.
#pragma unroll
          for (int j = 0; j < CPL; ++j)
            asm volatile("" : "+v"(cur[j].x), "+v"(cur[j].y), "+v"(cur[j].z), "+v"(cur[j].w));
          if (t == staged) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              const int64_t c = lane + kWave * j;
              float x8[8];
              unpack8(cur[j], x8);
              emit_chunk(a, r, c, lane, x8, w_f + 8 * c, opl_f + 8 * c, sh_f + 8 * c, rstd, gsf,
                         inv_tab, sbase);
            }
          } else {
            emit_row_unstaged(a, r, t, lane, w_f, rstd, gsf, inv_tab, sbase);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) cur[j] = nxt[j];
  }
}

// ---- the general kernel (any k % 512 == 0): parameters from global memory, two passes ----

__global__ __launch_bounds__(256) void rms_adaln_general(RmsArgs a) {
  __shared__ float inv_tab[128];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t chunks = a.k >> 3;
  const float gsf = global_scale(a.global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= a.padded) return;
  if (r >= a.m) {
    zero_row_scales(a.scales, r, a.k, lane);
    return;
  }
  const uint4* xr = a.x + r * chunks;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t c = lane; c < chunks; c += kWave) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f[e], f[e], acc[e]);
  }
  float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) s = s + __shfl_xor(s, d, kWave);
  const float rstd = 1.0f / sqrtf(s / (float)a.k + a.eps);
  if (lane == 0 && a.rstd_out) a.rstd_out[r] = rstd;
  const int64_t t = a.frame_idx[r];
  if (t < 0 || t >= a.num_frames) {
    zero_row(a, r, lane);
    return;
  }
  const int64_t sbase = row_scale_base(r, a.k);
  for (int64_t c = lane; c < chunks; c += kWave) {
    float x8[8], w8[8], o8[8], h8[8];
    unpack8(xr[c], x8);
    unpack8(*reinterpret_cast<const uint4*>(a.w + 8 * c), w8);
    load_frame_chunk(a, t, c, o8, h8);
    emit_chunk(a, r, c, lane, x8, w8, o8, h8, rstd, gsf, inv_tab, sbase);
  }
}

template <int CPL>
hipError_t launch_staged(const RmsArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lds = (128 + 3 * (size_t)a.k) * sizeof(float);
  RmsArgs b = a;
  const int64_t groups = (a.padded + kWaves - 1) / kWaves;
  int64_t units = dev.cu_count < groups ? dev.cu_count : groups;
  b.per = (units + kXcds - 1) / kXcds;
  units = b.per * kXcds;
  b.rows_per_unit = (a.padded + units - 1) / units;
  hipLaunchKernelGGL(rms_adaln_staged<CPL>, dim3((uint32_t)units), dim3(kThreads), lds, stream, b);
  return hipGetLastError();
}

template <int CPL>
hipError_t allow_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&rms_adaln_staged<CPL>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)((128 + 3 * kMaxStagedK) * sizeof(float)));
}

}  // namespace

hipError_t prepare_rms_adaln() {
  hipError_t (*fns[16])() = {allow_lds<1>,  allow_lds<2>,  allow_lds<3>,  allow_lds<4>,
                             allow_lds<5>,  allow_lds<6>,  allow_lds<7>,  allow_lds<8>,
                             allow_lds<9>,  allow_lds<10>, allow_lds<11>, allow_lds<12>,
                             allow_lds<13>, allow_lds<14>, allow_lds<15>, allow_lds<16>};
  for (auto fn : fns) {
    hipError_t e = fn();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_rms_adaln(const void* x, const void* weight, const void* shift, const void* scale,
                            int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                            float eps, int64_t m, int64_t k, float global_amax, void* codes,
                            void* scales, float* rstd_out, void* y_out, uint32_t* status_word,
                            const DeviceInfo& dev, hipStream_t stream) {
  RmsArgs a;
  a.x = static_cast<const uint4*>(x);
  a.w = static_cast<const uint16_t*>(weight);
  a.shift = static_cast<const uint16_t*>(shift);
  a.scale = static_cast<const uint16_t*>(scale);
  a.frame_stride = frame_stride;
  a.num_frames = num_frames;
  a.frame_idx = frame_idx;
  a.eps = eps;
  a.m = m;
  a.k = k;
  a.padded = (m + 127) / 128 * 128;
  a.global_amax = global_amax;
  a.codes = static_cast<uint32_t*>(codes);
  a.scales = static_cast<uint8_t*>(scales);
  a.rstd_out = rstd_out;
  a.y_out = static_cast<uint4*>(y_out);
  a.status = status_word;
  a.rows_per_unit = 0;
  a.per = 0;
  switch (k / 512) {
    case 1: return launch_staged<1>(a, dev, stream);
    case 2: return launch_staged<2>(a, dev, stream);
    case 3: return launch_staged<3>(a, dev, stream);
    case 4: return launch_staged<4>(a, dev, stream);
    case 5: return launch_staged<5>(a, dev, stream);
    case 6: return launch_staged<6>(a, dev, stream);
    case 7: return launch_staged<7>(a, dev, stream);
    case 8: return launch_staged<8>(a, dev, stream);
    case 9: return launch_staged<9>(a, dev, stream);
    case 10: return launch_staged<10>(a, dev, stream);
    case 11: return launch_staged<11>(a, dev, stream);
    case 12: return launch_staged<12>(a, dev, stream);
    case 13: return launch_staged<13>(a, dev, stream);
    case 14: return launch_staged<14>(a, dev, stream);
    case 15: return launch_staged<15>(a, dev, stream);
    case 16: return launch_staged<16>(a, dev, stream);
    default: break;
  }
  const int64_t blocks = (a.padded + 3) / 4;
  hipLaunchKernelGGL(rms_adaln_general, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4act
