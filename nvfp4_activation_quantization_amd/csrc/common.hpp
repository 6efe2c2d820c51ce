// common.hpp -- device building blocks shared by the NVFP4 producer kernels.
//
// The NVFP4 format (FastVideo API page "fastvideo.models.vaes.minimax_h3_nvfp4_fused",
// module summary and new_quantized; FastVideo branch compare, minimax_h3_swiglu_quant.cuh,
// quant_probe): 16-element blocks, an E4M3 block scale under a global fp32 scale, E2M1
// element codes packed two per byte (even column low), scales in the 128x4 swizzle.
//
// Work decomposition used by every kernel: one 64-lane wavefront owns one row at a
// time.  The row is cut into 8-element chunks (16 bytes of bf16); lane L handles chunks
// L, L+64, L+128, ... so each wavefront load is a contiguous 1 KiB.  A 16-element block is
// chunk pair (2b, 2b+1), i.e. lanes (L, L^1): its amax is exchanged with one DPP move.
// Four consecutive blocks live on lanes 8q..8q+7; lane 8q assembles their four scale
// bytes and writes them as one 32-bit word, which in the swizzled layout is contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4act {

// Pointers known to address global memory: loads and stores through them compile to
// global_* instructions rather than flat_* (pointers that reach a kernel inside a struct
// argument are otherwise treated as generic).  The qualifier only exists for the gfx950
// pass; the host pass of the same source sees plain pointers.
#if defined(__HIP_DEVICE_COMPILE__)
#define NVFP4_GLOBAL __attribute__((address_space(1)))
#else
#define NVFP4_GLOBAL
#endif

template <class T>
__device__ __forceinline__ NVFP4_GLOBAL T* global_ptr(T* p) {
  return (NVFP4_GLOBAL T*)p;
}

constexpr int kWave = 64;
constexpr uint32_t kRcp6Bits = 0x3E2AAAABu;   // fp32 nearest to 1/6

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- bf16 ----------------------------------------------------------------------------

// The two bf16 values of a packed word as exact fp32 (element 0 in the low half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// The low and high fp16 halves of a word as fp32 (exact).
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// The fp16 bit pattern of fp16(f), round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Round two fp32 values to bf16 (nearest, ties to even; gfx950 v_cvt_pk_bf16_f32,
// which matches the integer rule on every non-NaN fp32 input) and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf16(a + b) for the two bf16 values of a word each (an eager bf16 tensor add).
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b) {
  return pack_bf16x2(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b));
}

// bf16(f) as an fp32 value, in one instruction: converting the pair (0, f) puts bf16(f)
// in the upper half and +0 in the lower half, which is exactly the fp32 encoding of the
// rounded value.
__device__ __forceinline__ float round_bf16(float f) {
  return __uint_as_float(pack_bf16x2(0.0f, f));
}

// Pack two values that are already bf16-exact fp32 numbers (upper halves of a and b).
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// ---- E4M3 / E2M1 ---------------------------------------------------------------------

// E4M3 code of a non-negative fp32, nearest-even, saturating at 448.  v_cvt_pk_fp8_f32
// rounds to nearest-even on gfx950 (OCP E4M3) but turns values beyond 448 into NaN, so
// the input is clamped first.  The pair (c, 0) converts to (code, 0x00) in the low half
// and the upper half comes from the zero `old` operand, so the word is the code itself.
__device__ __forceinline__ uint32_t e4m3_code(float sf) {
  float c = __builtin_fminf(sf, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false);
}

// Four signed E4M3 codes (nearest-even, saturating at +-448), a in the low byte.
// v_cvt_pk_fp8_f32 rounds to nearest-even but turns magnitudes beyond 448 into NaN, so the
// values are clamped first (v_med3 keeps the sign of zero).
__device__ __forceinline__ uint32_t fp8_quad(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Exact value of an E4M3 code 0..126: exponent field 0 is m * 2^-9, else 2^(e-7)(1+m/8).
__device__ __forceinline__ float e4m3_value(uint32_t s) {
  uint32_t e = (s >> 3) & 15u, mant = s & 7u;
  if (e == 0) return (float)mant * 0.001953125f;
  return __uint_as_float(((e + 120u) << 23) | (mant << 20));
}

// Eight E2M1 codes of v[0..7] packed into one word (v[0] in bits 0..3).  The gfx950
// scaled fp4 conversion with scale 1.0 rounds nearest-even, saturates at 6 and keeps
// the sign of zero, like the specification, on every non-NaN fp32 input.
__device__ __forceinline__ uint32_t pack_e2m1x8(const float* v) {
  uint32_t w = __float_as_uint(v[0]);     // every byte is overwritten below
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---- cross-lane ----------------------------------------------------------------------

// max(v, value of lane L^1) for non-negative fp32 bit patterns (DPP quad_perm
// [1,0,3,2]; with 0, the identity of the unsigned max, as the old value the move folds
// into the max as one DPP instruction).
__device__ __forceinline__ uint32_t max_with_lane_xor1(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  return __builtin_elementwise_max(v, o);
}

// max(|a|, |b|, |c|) and max(t, |b|, |c|) as single v_max3_f32 instructions with abs
// source modifiers.  (Written out because the compiler lowers fabs of a value that was
// bit-cast from an integer, as every bf16-rounded value here is, to a separate AND.)
// Inputs are finite, where this equals the IEEE maximum of the magnitudes.
__device__ __forceinline__ float abs_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_abs2(float t, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(t), "v"(b), "v"(c));
  return r;
}

// ---- global scale and inverse-scale table ----------------------------------------------

// gsf = 2688 / global_amax, IEEE fp32 (every lane computes the same value).
__device__ __forceinline__ float global_scale(float global_amax) { return 2688.0f / global_amax; }

// Global scale of a per-call amax measured on the tensor (FlashRT dynamic per-call
// activation scale; FastVideo API page, NVFP4DecoderLinear act_scale="dynamic"): 2688 / a
// when that is positive and finite, else 0 (every block scale 0, every code a signed zero).
__device__ __forceinline__ float dynamic_global_scale(float a) {
  if (!(a > 0.0f)) return 0.0f;
  const float g = 2688.0f / a;
  return __builtin_isfinite(g) ? g : 0.0f;
}

// The global scale of a call: from the static amax, or, when amax_dev is not null, from
// the amax a preceding pass left in device memory.
__device__ __forceinline__ float call_global_scale(float global_amax, const float* amax_dev) {
  return amax_dev ? dynamic_global_scale(*global_ptr(amax_dev)) : global_scale(global_amax);
}

// Fill inv[0..127] with gsf / dec(s) (0 for s == 0); needs a barrier before use.
__device__ __forceinline__ void fill_inverse_table(float* inv, float gsf, int tid) {
  if (tid < 128) inv[tid] = (tid == 0) ? 0.0f : gsf / e4m3_value((uint32_t)tid);
}

// ---- the block quantizer for one chunk --------------------------------------------------

// The E4M3 scale code of the 16-element block whose halves y[0..7] are on lanes L and L^1
// (the same value on both lanes of the pair).
__device__ __forceinline__ uint32_t block_scale_code(const float* y, float gsf) {
  float amax = abs_max3(y[0], y[1], y[2]);
  amax = max_abs2(amax, y[3], y[4]);
  amax = max_abs2(amax, y[5], y[6]);
  amax = max_abs2(amax, y[7], y[7]);
  // the partner lane's half: amax >= 0, so the larger bit pattern is the larger value
  amax = __uint_as_float(max_with_lane_xor1(__float_as_uint(amax)));
  const float rcp6 = __uint_as_float(kRcp6Bits);
  return e4m3_code(gsf * (amax * rcp6));
}

// The packed E2M1 codes of y[0..7] under the inverse scale inv (gsf / dec(s), or 0).
__device__ __forceinline__ uint32_t encode_chunk(const float* y, float inv) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = y[i] * inv;
  return pack_e2m1x8(v);
}

// y[0..7]: this lane's half of a 16-element block (its partner lane L^1 holds the other
// half).  Returns the packed codes of the 8 elements and sets *scale to the block's
// E4M3 code (the same value on both lanes of the pair).
__device__ __forceinline__ uint32_t quantize_chunk(const float* y, float gsf, const float* inv_tab,
                                                   uint32_t* scale) {
  float amax = abs_max3(y[0], y[1], y[2]);
  amax = max_abs2(amax, y[3], y[4]);
  amax = max_abs2(amax, y[5], y[6]);
  amax = max_abs2(amax, y[7], y[7]);
  // the partner lane's half: amax >= 0, so the larger bit pattern is the larger value
  amax = __uint_as_float(max_with_lane_xor1(__float_as_uint(amax)));
  const float rcp6 = __uint_as_float(kRcp6Bits);
  const uint32_t s = e4m3_code(gsf * (amax * rcp6));
  const float inv = inv_tab[s];
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = y[i] * inv;
  *scale = s;
  return pack_e2m1x8(v);
}

// Where a lane writes its block's scale byte.  Chunk c = lane + 64 j holds half of block
// b = c / 2, whose byte sits at row_scale_base + (c / 8) * 512 + (c / 2) % 4, i.e. at
// row_scale_base + scale_lane_offset(lane) + 4096 j.  Both lanes of a block store the same
// byte to the same address, so no cross-lane gather is needed.
__device__ __forceinline__ int64_t scale_lane_offset(int lane) {
  return (int64_t)(lane >> 3) * 512 + ((lane >> 1) & 3);
}

// Byte offset, in the swizzled scale buffer, of block 0 of row r (k columns); block b
// (b % 4 == 0) of the row is at row_scale_base(r, k) + (b / 4) * 512.
__device__ __forceinline__ int64_t row_scale_base(int64_t r, int64_t k) {
  return (r >> 7) * (k >> 6) * 512 + (r & 31) * 16 + ((r >> 5) & 3) * 4;
}

// Zero the scale bytes of row r (a padding row, or a row written as zeros).
__device__ __forceinline__ void zero_row_scales(uint8_t* scales, int64_t r, int64_t k, int lane) {
  NVFP4_GLOBAL uint8_t* base = global_ptr(scales) + row_scale_base(r, k);
  for (int64_t q = lane; q < (k >> 6); q += kWave)
    *reinterpret_cast<NVFP4_GLOBAL uint32_t*>(base + q * 512) = 0u;
}

// ---- cross-lane sum ---------------------------------------------------------------------

// Butterfly sum over the 64 lanes: for s = 1, 2, 4, 8, 16, 32 every lane replaces v by
// v + v[lane ^ s] (IEEE fp32 adds; both lanes of a pair compute the same sum, so every
// lane ends with the same value).  The partner values come from DPP and the gfx950 row
// swaps rather than LDS permutes: s = 1, 2 are quad permutations; s = 4 is row_shl:4 on
// the even 4-lane banks of each 16-lane row and row_shr:4 on the odd ones; s = 8 is
// row_ror:8; s = 16 and 32 use v_permlane16_swap / v_permlane32_swap, whose two results
// are the lane's value and its partner's.  The quad and row_ror steps read every lane of
// the row (no masked banks), so their moves fold into one v_add_f32_dpp each.
__device__ __forceinline__ float lane_sum_butterfly(float v) {
  uint32_t u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  u = __float_as_uint(v);
  int t = __builtin_amdgcn_update_dpp((int)u, (int)u, 0x104, 0xF, 0x5, false);   // banks 0, 2: lane + 4
  t = __builtin_amdgcn_update_dpp(t, (int)u, 0x114, 0xF, 0xA, false);            // banks 1, 3: lane - 4
  v = v + __uint_as_float((uint32_t)t);
  u = __float_as_uint(v);
  v = v + __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x128, 0xF, 0xF, true));
  u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  u = __float_as_uint(v);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

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

// ---- amax reduction --------------------------------------------------------------------

// max(|a|, |b|, ..) of the eight values of a chunk folded into t (t >= 0).
__device__ __forceinline__ float fold_abs8(float t, const float* y) {
  t = max_abs2(t, y[0], y[1]);
  t = max_abs2(t, y[2], y[3]);
  t = max_abs2(t, y[4], y[5]);
  return max_abs2(t, y[6], y[7]);
}

// Workgroup maximum of the non-negative values v, folded into *dst with one device-scope
// atomic max per workgroup (the maximum is exact and order-free, so the result does not
// depend on which workgroup arrives first).  red: `waves` floats of LDS.  Every thread of
// the workgroup must call it.
__device__ __forceinline__ void workgroup_max_to(float* dst, float v, float* red, int waves) {
  uint32_t u = __float_as_uint(v);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) u = __builtin_elementwise_max(u, (uint32_t)__shfl_xor((int)u, d));
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) red[wave] = __uint_as_float(u);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int w = 0; w < waves; ++w) m = __builtin_elementwise_max(m, __float_as_uint(red[w]));
    __hip_atomic_fetch_max(reinterpret_cast<NVFP4_GLOBAL uint32_t*>(global_ptr(dst)), m, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- streaming loads ------------------------------------------------------------------

// 16-byte load that is not expected to be re-read (non-temporal hint).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const NVFP4_GLOBAL u32x4*>(global_ptr(p)));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16-, 4- and 2-byte stores that are not expected to be re-read soon (non-temporal hint).
__device__ __forceinline__ void store_stream(uint4* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<NVFP4_GLOBAL u32x4*>(global_ptr(p)));
}

__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, global_ptr(p));
}

__device__ __forceinline__ void store_stream(uint16_t* p, uint16_t v) {
  __builtin_nontemporal_store(v, global_ptr(p));
}

__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const NVFP4_GLOBAL u32x2*>(global_ptr(p)));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ void store_stream(uint2* p, const uint2& v) {
  const u32x2 w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<NVFP4_GLOBAL u32x2*>(global_ptr(p)));
}

__device__ __forceinline__ void store_stream(float4* p, const float4& v) {
  const u32x4 w = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_nontemporal_store(w, reinterpret_cast<NVFP4_GLOBAL u32x4*>(global_ptr(p)));
}

// ---- workgroup -> row-group mapping ----------------------------------------------------

// A workgroup of four wavefronts owns the rows r, r + 32, r + 64, r + 96 of a 128-row tile
// (r = tile * 128 + rr, rr < 32): in the 128x4 swizzled scale layout those rows' scale bytes
// of four consecutive blocks form one contiguous 16-byte unit, which the workgroup can
// gather in LDS and write whole.  The eight workgroups rr = 8p .. 8p + 7 of a tile fill the
// same 128-byte lines of the scale buffer; workgroups are dealt round-robin over the 8 XCDs
// (each with its own L2), so block indices are arranged to put those eight consecutively
// on one XCD, and each line is completed in one L2 before it is written back.
//
// Row group of workgroup b: unit group u = b / 64 * 8 + b % 8 (tile u / 4, rr block u % 4),
// rr = 8 (u % 4) + (b / 8) % 8.  For a fixed u the eight values of (b / 8) % 8 share b % 8.
struct RowGroup {
  int64_t tile;
  int rr;
};

__device__ __forceinline__ RowGroup row_group(int64_t b) {
  const int64_t u = (b >> 6) * 8 + (b & 7);
  RowGroup g;
  g.tile = u >> 2;
  g.rr = (int)((u & 3) * 8 + ((b >> 3) & 7));
  return g;
}

// Workgroups to launch for m rows: whole groups of 64 covering the tiles' 4 row groups each
// (the surplus workgroups find a tile past the end and return).
inline int64_t row_group_blocks(int64_t m) {
  const int64_t unit_groups = (m + 127) / 128 * 4;
  return (unit_groups + 7) / 8 * 64;
}

}  // namespace nvfp4act
