// residual_rms.hip -- fp32 residual stream + RMSNorm with an fp32 weight -> NVFP4 (FastVideo
// API page, residual_norm_quantize: the residual add of a block's branch folded into the
// norm that produces the next quantized activation):
//   t    = bf16(o + bias)                    o: the branch output (bf16), bias optional
//   h    = h + t * scale                     in place, fp32; the product is rounded first
//   rstd = 1 / sqrt(sum(h^2) / k + eps)      the quad tree below
//   y    = bf16((h * rstd) * gamma)
// followed by the NVFP4 block quantizer.  Without a branch (o null) h is only read.
//
// The MOD form folds a DiT block's gated MLP residual into the next block's RMSNorm +
// adaLN producer (TensorRT-LLM PR #21483, Summary: the folding block reads its gate from
// its own AdaLN table, shift and scale from the next block's): with t = frame_idx[r],
//   h = h + bf16(o + bias) * gate[t]         (the gate a bf16 row of the block's own table)
//   y = bf16(bf16(bf16(bf16(h * rstd) * w) * bf16(1 + scale[t])) + shift[t])
// A row whose frame index lies outside [0, num_frames) keeps its h, is written as zeros
// and raises bit 0 of the status word.
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
  // MOD: the tables (4 bf16 per quad; strides in quads)
  const uint2* gate;        // the folding block's gate rows: gate + t * gate_stride4
  int64_t gate_stride4;
  const uint2* w;           // RMSNorm weight
  const uint2* shift;       // the next block's rows: shift + t * frame_stride4
  const uint2* mscale;      // ... and scale + t * frame_stride4
  int64_t frame_stride4;
  int64_t num_frames;
  const int32_t* frame_idx;
  uint32_t* status;
};


// s_waitcnt vmcnt(N) (N < 64), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// The four bf16 of a quad (lo, hi of two words) as fp32.
__device__ __forceinline__ void unpack4(const uint2& v, float* f) {
  f[0] = bf16_lo(v.x);
  f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y);
  f[3] = bf16_hi(v.y);
}

// Where the MOD form reads its per-column parameters, quad pq of the row's frame t: the
// global tables (Global; the residual pass always reads these), or, for the output pass,
// the workgroup's LDS copy of frame t's rows (Staged: weight, scale and shift, k/4 quads
// each).
struct GlobalParams {
  const ResArgs* a;
  int64_t t;
  __device__ __forceinline__ uint2 gate(int64_t pq) const { return global_ptr(a->gate)[t * a->gate_stride4 + pq]; }
  __device__ __forceinline__ uint2 bias(int64_t pq) const { return global_ptr(a->bias)[pq]; }
  __device__ __forceinline__ uint2 w(int64_t pq) const { return global_ptr(a->w)[pq]; }
  __device__ __forceinline__ uint2 scale(int64_t pq) const {
    return global_ptr(a->mscale)[t * a->frame_stride4 + pq];
  }
  __device__ __forceinline__ uint2 shift(int64_t pq) const {
    return global_ptr(a->shift)[t * a->frame_stride4 + pq];
  }
};

struct StagedParams {
  const uint2* lds;         // 3 planes of `quads` uint2: w, scale, shift
  int quads;
  __device__ __forceinline__ uint2 w(int64_t pq) const { return lds[pq]; }
  __device__ __forceinline__ uint2 scale(int64_t pq) const { return lds[quads + pq]; }
  __device__ __forceinline__ uint2 shift(int64_t pq) const { return lds[2 * quads + pq]; }
};

constexpr int kStagedPlanes = 3;

// Stage frame t's output-pass rows of the MOD form into LDS: weight, scale and shift, k bf16
// each, copied by global_load_lds_dwordx4 -- 1 KiB per wavefront instruction, lane i's 16
// bytes landing at the instruction's LDS base + 16 i -- so no registers hold them.  Issued
// after the row's own loads, they travel while the residual pass runs; the caller waits
// for them (vmcnt) and synchronises the workgroup before the output pass.
__device__ __forceinline__ void stage_params(const ResArgs& a, int64_t t, uint2* lds, int wave, int lane) {
  const int per = (int)(a.k >> 9);                 // 1 KiB pieces per plane (k % 512 == 0)
  const uint2* src[kStagedPlanes] = {a.w, a.mscale + t * a.frame_stride4, a.shift + t * a.frame_stride4};
  for (int n = wave; n < kStagedPlanes * per; n += kWaves) {
    const int plane = n / per, part = n - plane * per;
    const char* gsrc = reinterpret_cast<const char*>(src[plane]) + ((int64_t)part * 64 + lane) * 16;
    char* ldst = reinterpret_cast<char*>(lds) + (int64_t)plane * (a.k * 2) + part * 1024;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)ldst, 16, 0, 0);
  }
}

// The residual add (RESID) and the statistic of one row whose loads were issued; the
// updated values stay in hp.  Returns rstd.  (Whether a row is added is decided once per row
// by the caller: a run-time test inside the unrolled loop splits it into blocks at whose
// joins the compiler waits for every memory operation in flight, stores included.)
template <int QMAX, bool EXACT, bool RESID, bool BIAS, bool MOD, bool AMAX, class P>
__device__ __forceinline__ float residual_pass(const ResArgs& a, const P& par, int nq, int64_t r, int64_t q0,
                                               int lane, const uint4* hv, const uint2* ov, float (*hp)[4]) {
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    if (!EXACT && j >= nq) continue;                               // uniform; keeps the unroll
    const int64_t pq = lane + kWave * j;                           // parameter quad
    float x[4] = {__uint_as_float(hv[j].x), __uint_as_float(hv[j].y), __uint_as_float(hv[j].z),
                  __uint_as_float(hv[j].w)};
    if (RESID) {
      float sc[4];
      if (MOD) {
        unpack4(par.gate(pq), sc);
      } else {
        const float4 v = global_ptr(a.scale)[pq];
        sc[0] = v.x;
        sc[1] = v.y;
        sc[2] = v.z;
        sc[3] = v.w;
      }
      uint32_t t0 = ov[j].x, t1 = ov[j].y;
      if (BIAS) {
        uint2 b;
        if (MOD) b = par.bias(pq);
        else b = global_ptr(a.bias)[pq];
        t0 = add_bf16x2(t0, b.x);
        t1 = add_bf16x2(t1, b.y);
      }
      // products rounded before the adds (no contraction: -ffp-contract=off)
      x[0] = x[0] + bf16_lo(t0) * sc[0];
      x[1] = x[1] + bf16_hi(t0) * sc[1];
      x[2] = x[2] + bf16_lo(t1) * sc[2];
      x[3] = x[3] + bf16_hi(t1) * sc[3];
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
  return rstd;
}

// The output pass of one row: y, the block scales (into the LDS units) and codes.  P: where
// the MOD form's parameters come from.
template <int QMAX, bool EXACT, bool MOD, bool AMAX, class P>
__device__ __forceinline__ void output_pass(const ResArgs& a, const P& par, int nq, int64_t q0, int lane, int wave,
                                            float rstd, float (*hp)[4], float gsf, const float* inv_tab,
                                            uint4* units, float* lane_amax) {
  const float rcp6 = __uint_as_float(kRcp6Bits);
  uint8_t* unit_bytes = reinterpret_cast<uint8_t*>(units) + wave * 4 + ((lane >> 2) & 3) + (lane >> 4) * 16;
#pragma unroll
  for (int j = 0; j < QMAX; ++j) {
    if (!EXACT && j >= nq) continue;
    const int64_t pq = lane + kWave * j;
    float y[4];
    if (MOD) {
      float w4[4], sc4[4], sh4[4];
      unpack4(par.w(pq), w4);
      unpack4(par.scale(pq), sc4);
      unpack4(par.shift(pq), sh4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float n = round_bf16(hp[j][e] * rstd);
        const float nw = round_bf16(n * w4[e]);
        const float mm = round_bf16(nw * round_bf16(1.0f + sc4[e]));
        y[e] = round_bf16(mm + sh4[e]);
      }
    } else {
      const float4 gm = global_ptr(a.gamma)[pq];
      y[0] = round_bf16((hp[j][0] * rstd) * gm.x);
      y[1] = round_bf16((hp[j][1] * rstd) * gm.y);
      y[2] = round_bf16((hp[j][2] * rstd) * gm.z);
      y[3] = round_bf16((hp[j][3] * rstd) * gm.w);
    }
    const float am = max_abs2(abs_max3(y[0], y[1], y[2]), y[3], y[3]);
    const float bmax = __uint_as_float(max_over_lane_quad(__float_as_uint(am)));
    if (AMAX) {
      *lane_amax = __builtin_fmaxf(*lane_amax, bmax);
      continue;
    }
    const uint32_t s = e4m3_code(gsf * (bmax * rcp6));
    const float inv = inv_tab[s];
    const uint32_t c = pack_e2m1x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
    global_ptr(a.codes)[q0 + kWave * j] = (uint16_t)c;
    if ((lane & 3) == 0) unit_bytes[64 * j] = (uint8_t)s;            // unit (lane / 16 + 4 j)
    if (a.y_out)
      global_ptr(a.y_out)[q0 + kWave * j] =
          make_uint2(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]));
  }
}

// QMAX: register slots (quads per lane) of the instantiation; EXACT: the row has exactly
// QMAX quads per lane, else `qpl` (<= QMAX) at run time.  RESID: a branch is added (BIAS:
// with a bias).  MOD: the gated, adaLN form; the workgroup stages the output-pass rows of
// the frame of its first row in LDS (dynamic LDS, 6 bytes per column) while the residual
// pass runs, and a wavefront whose row has another frame (only where a frame boundary
// falls inside the workgroup's rows) reads the global tables instead.  AMAX: the amax pass
// of a per-call scale -- the same rows and chain, no stores; each workgroup folds its
// max |y| into a.amax_out.
template <int QMAX, bool EXACT, bool RESID, bool BIAS, bool MOD, bool AMAX>
__global__ __launch_bounds__(kThreads) void residual_rms_kernel(const ResArgs a, int qpl) {
  __shared__ float inv_tab[128];
  __shared__ uint4 units[kMaxUnits];
  __shared__ float amax_red[kWaves];
  extern __shared__ __align__(16) uint2 staged[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const RowGroup g = row_group(blockIdx.x);
  if (g.tile >= ((a.m + 127) >> 7)) return;                        // idle workgroup (uniform)
  const int nq = EXACT ? QMAX : qpl;                               // quads per lane
  const int64_t row_quads = a.k >> 2;
  const int64_t r0 = (g.tile << 7) + g.rr;                         // the workgroup's first row
  const int64_t r = r0 + 32 * wave;
  const bool live = r < a.m;                                       // uniform per wavefront
  const int64_t q0 = r * row_quads + lane;                         // this lane's quad j = 0
  // MOD: the row's frame (uniform per wavefront); a row outside [0, num_frames) keeps h.
  // The workgroup stages the frame of its first row when that one is live and valid.
  int64_t t = 0, t0 = -1;
  bool frame_ok = true;
  if (MOD) {
    if (r0 < a.m) {
      const int64_t f0 = global_ptr(a.frame_idx)[r0];
      if (f0 >= 0 && f0 < a.num_frames) t0 = f0;
    }
    if (live) {
      t = global_ptr(a.frame_idx)[r];
      frame_ok = t >= 0 && t < a.num_frames;
    }
  }
  const bool add = RESID && frame_ok;
  const bool staging = MOD && t0 >= 0;                             // uniform per workgroup

  // the per-call amax (dynamic form), the row and its branch, then the staged rows: all in
  // flight while the inverse-scale table is built
  const float amax_in = a.amax_dev ? *global_ptr(a.amax_dev) : 0.0f;
  uint4 hv[QMAX];
  uint2 ov[QMAX];
  if (live) {
#pragma unroll
    for (int j = 0; j < QMAX; ++j)
      if (EXACT || j < nq) hv[j] = load_stream(a.h_in + q0 + kWave * j);
    if (add) {
#pragma unroll
      for (int j = 0; j < QMAX; ++j)
        if (EXACT || j < nq) ov[j] = load_stream(a.o + q0 + kWave * j);
    }
  }
  if (staging) stage_params(a, t0, staged, wave, lane);
  const float gsf = a.amax_dev ? dynamic_global_scale(amax_in) : global_scale(a.global_amax);
  if (!AMAX) {
    fill_inverse_table(inv_tab, gsf, tid);
    for (int i = tid; i < (int)(a.k >> 6); i += kThreads) units[i] = make_uint4(0, 0, 0, 0);
  }

  float hp[QMAX][4];
  float rstd = 0.0f;
  const bool use_staged = MOD && staging && t == t0;              // uniform per wavefront
  const StagedParams spar{staged, (int)row_quads};
  const GlobalParams gpar{&a, t};
  if (live) {
    if (add)
      rstd = residual_pass<QMAX, EXACT, RESID, BIAS, MOD, AMAX>(a, gpar, nq, r, q0, lane, hv, ov, hp);
    else
      rstd = residual_pass<QMAX, EXACT, false, false, MOD, AMAX>(a, gpar, nq, r, q0, lane, hv, ov, hp);
  }

  if (staging) {
    // every wavefront's share of the staged rows has landed
    wait_vmcnt<0>();
    __syncthreads();
  } else if (!AMAX) {
    // a barrier ordering LDS only: __syncthreads would also wait for the stream's stores
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  float lane_amax = 0.0f;
  if (live) {
    if (!frame_ok) {
      // zeros for the row (its scale bytes stay zero in the LDS units)
      if (!AMAX) {
#pragma unroll
        for (int j = 0; j < QMAX; ++j) {
          if (!EXACT && j >= nq) continue;
          global_ptr(a.codes)[q0 + kWave * j] = (uint16_t)0;
          if (a.y_out) global_ptr(a.y_out)[q0 + kWave * j] = make_uint2(0, 0);
        }
        if (lane == 0 && a.status) atomicOr(global_ptr(a.status), 1u);
      }
    } else if (use_staged) {
      output_pass<QMAX, EXACT, MOD, AMAX>(a, spar, nq, q0, lane, wave, rstd, hp, gsf, inv_tab, units, &lane_amax);
    } else {
      output_pass<QMAX, EXACT, MOD, AMAX>(a, gpar, nq, q0, lane, wave, rstd, hp, gsf, inv_tab, units, &lane_amax);
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

// Dynamic LDS of the MOD form: the staged planes of k bf16.
constexpr size_t staged_bytes(int64_t k) { return (size_t)(kStagedPlanes * 2 * k); }

template <int QMAX, bool EXACT, bool MOD, bool AMAX>
hipError_t launch_q(const ResArgs& a, int qpl, int64_t blocks, hipStream_t stream) {
  const dim3 grid((uint32_t)blocks), block(kThreads);
  const size_t lds = MOD ? staged_bytes(a.k) : 0;
  if (!a.o)
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, false, false, MOD, AMAX>), grid, block, lds, stream, a,
                       qpl);
  else if (!a.bias)
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, true, false, MOD, AMAX>), grid, block, lds, stream, a,
                       qpl);
  else
    hipLaunchKernelGGL((residual_rms_kernel<QMAX, EXACT, true, true, MOD, AMAX>), grid, block, lds, stream, a,
                       qpl);
  return hipGetLastError();
}

template <int QMAX, bool EXACT, bool AMAX>
hipError_t allow_staged() {
  const int lds = (int)staged_bytes(kMaxResidualK);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&residual_rms_kernel<QMAX, EXACT, false, false, true, AMAX>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&residual_rms_kernel<QMAX, EXACT, true, false, true, AMAX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&residual_rms_kernel<QMAX, EXACT, true, true, true, AMAX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  return e;
}

template <bool MOD, bool AMAX>
hipError_t launch_pass(const ResArgs& a, hipStream_t stream) {
  const int qpl = (int)(a.k / 256);
  const int64_t blocks = row_group_blocks(a.m);
  if (qpl == 28) return launch_q<28, true, MOD, AMAX>(a, qpl, blocks, stream);     // k = 7168
  if (qpl <= 8) return launch_q<8, false, MOD, AMAX>(a, qpl, blocks, stream);
  if (qpl <= 16) return launch_q<16, false, MOD, AMAX>(a, qpl, blocks, stream);
  return launch_q<32, false, MOD, AMAX>(a, qpl, blocks, stream);
}

template <bool AMAX>
hipError_t launch_pass(const ResArgs& a, bool mod, hipStream_t stream) {
  return mod ? launch_pass<true, AMAX>(a, stream) : launch_pass<false, AMAX>(a, stream);
}

}  // namespace

hipError_t prepare_residual_rms() {
  hipError_t e = allow_staged<28, true, false>();
  if (e == hipSuccess) e = allow_staged<28, true, true>();
  if (e == hipSuccess) e = allow_staged<8, false, false>();
  if (e == hipSuccess) e = allow_staged<8, false, true>();
  if (e == hipSuccess) e = allow_staged<16, false, false>();
  if (e == hipSuccess) e = allow_staged<16, false, true>();
  if (e == hipSuccess) e = allow_staged<32, false, false>();
  if (e == hipSuccess) e = allow_staged<32, false, true>();
  return e;
}

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
  a.gate = static_cast<const uint2*>(p.gate);
  a.gate_stride4 = p.gate_stride / 4;
  a.w = static_cast<const uint2*>(p.weight);
  a.shift = static_cast<const uint2*>(p.shift);
  a.mscale = static_cast<const uint2*>(p.mod_scale);
  a.frame_stride4 = p.frame_stride / 4;
  a.num_frames = p.num_frames;
  a.frame_idx = p.frame_idx;
  a.status = p.status_word;
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
    pass.status = nullptr;
    pass.amax_out = p.amax_dev;
    e = launch_pass<true>(pass, p.mod, stream);
    if (e != hipSuccess) return e;
    a.amax_dev = p.amax_dev;
  }
  return launch_pass<false>(a, p.mod, stream);
}

}  // namespace nvfp4act
