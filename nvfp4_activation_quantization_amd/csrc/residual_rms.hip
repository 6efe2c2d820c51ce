// residual_rms.hip -- fp32 residual stream + RMSNorm with an fp32 weight -> NVFP4 (FastVideo
// API page, residual_norm_quantize: the residual add of a block's branch folded into the
// norm that produces the next quantized activation):
//   t    = bf16(o + bias)                    o: the branch output (bf16), bias optional
//   h    = h + t * scale                     in place, fp32; the product is rounded first
//   rstd = 1 / sqrt(sum(h^2) / k + eps)      the quad tree below
//   y    = bf16((h * rstd) * gamma)
// followed by the NVFP4 block quantizer.  Without a branch (o null) h is only read.
//
// Bandwidth-bound: 4 + 2 bytes read and 4 written per element (the stream and the branch),
// 0.5625 bytes of codes and scales on top, about fifteen VALU operations per element.
//
// * One wavefront per row, non-persistent, four rows per workgroup: the rows r, r + 32,
//   r + 64, r + 96 of a 128-row tile whose scale bytes form the 16-byte units of the 128x4
//   layout (row_group), gathered in LDS and written whole.
// * Lane L holds the quads (4 consecutive fp32) L + 64 j of its row, j < k / 256, loaded and
//   stored as 16-byte vectors: each instruction of a wavefront covers 1 KiB of the stream,
//   512 bytes of the branch and 128 bytes of codes, all contiguous.  The whole row stays in
//   registers from the statistic to the output pass (k <= 8192).
// * The statistic: four accumulators per lane (one per position in the quad), fused
//   multiply-adds over j ascending, folded as (a0 + a1) + (a2 + a3), then the butterfly over
//   the 64 lanes -- the fixed tree of the specification for an fp32 row.
// * A 16-element block lies on the four lanes 4i .. 4i + 3: its amax is combined with two
//   DPP quad permutations, every lane of the four derives the same scale code, encodes its
//   own 4 elements (2 bytes of codes), and the first writes the scale byte into LDS.
// * The per-column parameters (scale, bias, gamma: 10 bytes a column) are read through the
//   caches: the four wavefronts of a workgroup read the same values at about the same time.
// * The updated stream leaves with non-temporal stores; with plain ones the kernel ran 25%
//   slower.  At 63,240 x 7168 it runs at the speed of a bare kernel that moves the same bytes
//   (read h and o, write h and the codes) with the same instructions and no arithmetic.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kWaves = 4;                     // rows per workgroup (r + 32 i)
constexpr int kThreads = kWaves * kWave;
constexpr int kMaxUnits = kMaxResidualK / 64;   // 16-byte scale units per row group

struct ResArgs {
  const uint4* h_in;        // the stream as 16-byte quads (the same memory as h_out)
  float4* h_out;            // where the updated stream is written (null: not written)
  const uint2* o;           // the branch, 4 bf16 per quad (null: no residual)
  const uint2* bias;        // 4 bf16 per quad (null: no bias)
  const float4* scale;      // 4 fp32 per quad
  const float4* gamma;      // 4 fp32 per quad
  float eps;
  int64_t m, k;
  float global_amax;
  const float* amax_dev;    // per-call scale: the amax pass's result (null: static global_amax)
  float* amax_out;          // the amax pass: where max |y| is folded
  uint16_t* codes;          // 2 bytes (4 E2M1 codes) per quad
  uint8_t* scales;
  float* rstd_out;
  uint2* y_out;             // 4 bf16 per quad
};

// max over the four lanes 4i .. 4i + 3 of non-negative fp32 bit patterns (DPP quad
// permutations [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ uint32_t max_over_lane_quad(uint32_t v) {
  v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  return __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
}

// Four E2M1 codes of v[0..3] in the low 16 bits (v[0] in bits 0..3); see pack_e2m1x8.
__device__ __forceinline__ uint32_t pack_e2m1x4(float v0, float v1, float v2, float v3) {
  uint32_t w = __float_as_uint(v0);       // bytes 0 and 1 are overwritten below
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, 1.0f, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v2, v3, 1.0f, 1);
}

// bf16(a + b) for the two bf16 values of a word each.
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  return pack_bf16x2(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b));
}

// QMAX: register slots (quads per lane) of the instantiation; EXACT: the row has exactly
// QMAX quads per lane, else `qpl` (<= QMAX) at run time.  RESID: a branch is added (BIAS:
// with a bias).  AMAX: the amax pass of a per-call scale -- the same rows and chain, no
// stores; each workgroup folds its max |y| into a.amax_out.
template <int QMAX, bool EXACT, bool RESID, bool BIAS, bool AMAX>
__global__ __launch_bounds__(kThreads) void residual_rms_kernel(const ResArgs a, int qpl) {
  __shared__ float inv_tab[128];
  __shared__ uint4 units[kMaxUnits];
  __shared__ float amax_red[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const RowGroup g = row_group(blockIdx.x);
  if (g.tile >= ((a.m + 127) >> 7)) return;                        // idle workgroup (uniform)
  const int nq = EXACT ? QMAX : qpl;                               // quads per lane
  const int64_t row_quads = a.k >> 2;
  const int64_t r = (g.tile << 7) + g.rr + 32 * wave;
  const bool live = r < a.m;                                       // uniform per wavefront
  const int64_t q0 = r * row_quads + lane;                         // this lane's quad j = 0

  // the row (and its branch) is in flight while the inverse-scale table is built
  uint4 hv[QMAX];
  uint2 ov[QMAX];
  if (live) {
#pragma unroll
    for (int j = 0; j < QMAX; ++j)
      if (EXACT || j < nq) hv[j] = load_stream(a.h_in + q0 + kWave * j);
    if (RESID) {
#pragma unroll
      for (int j = 0; j < QMAX; ++j)
        if (EXACT || j < nq) ov[j] = load_stream(a.o + q0 + kWave * j);
    }
  }
  const float gsf = call_global_scale(a.global_amax, a.amax_dev);
  if (!AMAX) {
    fill_inverse_table(inv_tab, gsf, tid);
    for (int i = tid; i < (int)(a.k >> 6); i += kThreads) units[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  float lane_amax = 0.0f;
  if (live) {
    // residual add and statistic
    float hp[QMAX][4];
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      if (!EXACT && j >= nq) continue;                             // uniform; keeps the unroll
      const int64_t pq = lane + kWave * j;                         // parameter quad
      float x[4] = {__uint_as_float(hv[j].x), __uint_as_float(hv[j].y), __uint_as_float(hv[j].z),
                    __uint_as_float(hv[j].w)};
      if (RESID) {
        const float4 sc = global_ptr(a.scale)[pq];
        uint32_t t0 = ov[j].x, t1 = ov[j].y;
        if (BIAS) {
          const uint2 b = global_ptr(a.bias)[pq];
          t0 = add_bf16x2(t0, b.x);
          t1 = add_bf16x2(t1, b.y);
        }
        // products rounded before the adds (no contraction: -ffp-contract=off)
        x[0] = x[0] + bf16_lo(t0) * sc.x;
        x[1] = x[1] + bf16_hi(t0) * sc.y;
        x[2] = x[2] + bf16_lo(t1) * sc.z;
        x[3] = x[3] + bf16_hi(t1) * sc.w;
        // streaming (non-temporal) stores: 1034 -> 827 us at 63240 x 7168 against plain ones
        if (!AMAX)
          store_stream(reinterpret_cast<uint4*>(a.h_out) + q0 + kWave * j,
                       make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                  __float_as_uint(x[3])));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = __builtin_fmaf(x[e], x[e], acc[e]);
        hp[j][e] = x[e];
      }
    }
    const float sum = lane_sum_butterfly((acc[0] + acc[1]) + (acc[2] + acc[3]));
    const float rstd = 1.0f / sqrtf(sum / (float)a.k + a.eps);
    if (!AMAX && lane == 0 && a.rstd_out) global_ptr(a.rstd_out)[r] = rstd;

    // output pass
    const float rcp6 = __uint_as_float(kRcp6Bits);
    uint8_t* unit_bytes = reinterpret_cast<uint8_t*>(units) + wave * 4 + ((lane >> 2) & 3) + (lane >> 4) * 16;
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      if (!EXACT && j >= nq) continue;
      const float4 gm = global_ptr(a.gamma)[lane + kWave * j];
      float y[4];
      y[0] = round_bf16((hp[j][0] * rstd) * gm.x);
      y[1] = round_bf16((hp[j][1] * rstd) * gm.y);
      y[2] = round_bf16((hp[j][2] * rstd) * gm.z);
      y[3] = round_bf16((hp[j][3] * rstd) * gm.w);
      const float am = max_abs2(abs_max3(y[0], y[1], y[2]), y[3], y[3]);
      const float bmax = __uint_as_float(max_over_lane_quad(__float_as_uint(am)));
      if (AMAX) {
        lane_amax = __builtin_fmaxf(lane_amax, bmax);
        continue;
      }
      const uint32_t s = e4m3_code(gsf * (bmax * rcp6));
      const float inv = inv_tab[s];
      const uint32_t c = pack_e2m1x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
      global_ptr(a.codes)[q0 + kWave * j] = (uint16_t)c;
      if ((lane & 3) == 0) unit_bytes[64 * j] = (uint8_t)s;          // unit (lane / 16 + 4 j)
      if (a.y_out)
        global_ptr(a.y_out)[q0 + kWave * j] =
            make_uint2(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]));
    }
  }
  if (AMAX) {
    workgroup_max_to(a.amax_out, lane_amax, amax_red, kWaves);
    return;
  }
  __syncthreads();
  // the row group's units (zero bytes for rows >= m): unit u at (tile * k/64 + u) * 512 + rr * 16
  const int64_t groups = a.k >> 6;
  NVFP4_GLOBAL uint8_t* dst = global_ptr(a.scales) + (g.tile * groups) * 512 + g.rr * 16;
  for (int i = tid; i < (int)groups; i += kThreads)
    *reinterpret_cast<NVFP4_GLOBAL uint4*>(dst + (int64_t)i * 512) = units[i];
}

template <int QMAX, bool EXACT, bool AMAX>
hipError_t launch_q(const ResArgs& a, int qpl, int64_t blocks, hipStream_t stream) {
  const dim3 grid((uint32_t)blocks), block(kThreads);
  if (!a.o)
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, false, false, AMAX>), grid, block, 0, stream, a, qpl);
  else if (!a.bias)
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, true, false, AMAX>), grid, block, 0, stream, a, qpl);
  else
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, true, true, AMAX>), grid, block, 0, stream, a, qpl);
  return hipGetLastError();
}

template <bool AMAX>
hipError_t launch_pass(const ResArgs& a, hipStream_t stream) {
  const int qpl = (int)(a.k / 256);
  const int64_t blocks = row_group_blocks(a.m);
  if (qpl == 28) return launch_q<28, true, AMAX>(a, qpl, blocks, stream);     // k = 7168
  if (qpl <= 8) return launch_q<8, false, AMAX>(a, qpl, blocks, stream);
  if (qpl <= 16) return launch_q<16, false, AMAX>(a, qpl, blocks, stream);
  return launch_q<32, false, AMAX>(a, qpl, blocks, stream);
}

}  // namespace

hipError_t launch_residual_rms(const ResidualLaunch& p, hipStream_t stream) {
  ResArgs a;
  a.h_in = static_cast<const uint4*>(static_cast<const void*>(p.h));
  a.h_out = p.o ? reinterpret_cast<float4*>(p.h) : nullptr;
  a.o = static_cast<const uint2*>(p.o);
  a.bias = static_cast<const uint2*>(p.bias);
  a.scale = reinterpret_cast<const float4*>(p.scale);
  a.gamma = reinterpret_cast<const float4*>(p.gamma);
  a.eps = p.eps;
  a.m = p.m;
  a.k = p.k;
  a.global_amax = p.global_amax;
  a.amax_dev = nullptr;
  a.amax_out = nullptr;
  a.codes = static_cast<uint16_t*>(p.codes);
  a.scales = static_cast<uint8_t*>(p.scales);
  a.rstd_out = p.rstd_out;
  a.y_out = static_cast<uint2*>(p.y_out);
  if (p.amax_dev) {
    // per-call scale: zero the amax, fold max |y| into it (nothing is written, h included),
    // then run the producer with the global scale taken from it
    hipError_t e = launch_zero_amax(p.amax_dev, stream);
    if (e != hipSuccess) return e;
    ResArgs pass = a;
    pass.h_out = nullptr;
    pass.codes = nullptr;
    pass.scales = nullptr;
    pass.rstd_out = nullptr;
    pass.y_out = nullptr;
    pass.amax_out = p.amax_dev;
    e = launch_pass<true>(pass, stream);
    if (e != hipSuccess) return e;
    a.amax_dev = p.amax_dev;
  }
  return launch_pass<false>(a, stream);
}

}  // namespace nvfp4act
