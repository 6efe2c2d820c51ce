// selftest.hip -- libnvfp4act_selftest.so: diagnostics beside the product library (not part
// of its C ABI; loaded by the test suite and the benchmark only).
//
// 1. nvfp4act_selftest_convert: runs one of the conversion helpers the producer kernels use
//    (common.hpp, compiled the same way) over a contiguous range of fp32 bit patterns, so
//    that a test can compare every input of a conversion with the CPU definition:
//      kind 0  round_bf16(x)                  (v_cvt_pk_bf16_f32 with a zero low operand)
//      kind 1  pack_bf16x2(x[2i], x[2i+1])    (both operands converted)
//      kind 2  e4m3_code(x), x >= 0           (clamp at 448, then v_cvt_pk_fp8_f32)
//      kind 3  pack_e2m1x8(x[8i .. 8i+7])     (v_cvt_scalef32_pk_fp4_f32, scale 1.0)
//      kind 4  fp8_quad(x[4i .. 4i+3])        (signed E4M3 with med3 clamping)
//      kind 5  f16_bits(x)                    (fp32 -> fp16, nearest even)
// 2. nvfp4act_selftest_stream: the memory traffic of an [m, k] bf16 NVFP4 producer (a 2-byte
//    element read, half a byte of codes and 1/16 byte of swizzled scale written per
//    element) with no arithmetic, launched like the standalone quantize kernel (one row per
//    wavefront, four rows per workgroup forming whole scale units): what the memory system
//    delivers for this read/write mix, the practical ceiling the benchmark reports.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

using namespace nvfp4act;

namespace {

constexpr int kConvThreads = 256;

// Thread t handles the eight inputs first + 8t .. first + 8t + 7 of the range.
__global__ __launch_bounds__(kConvThreads) void convert_kernel(int kind, uint32_t first, int64_t groups, void* out,
                                                               unsigned int* bad_low_half) {
  const int64_t t = (int64_t)blockIdx.x * kConvThreads + threadIdx.x;
  if (t >= groups) return;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(first + (uint32_t)(8 * t + e));
  if (kind == 0) {
    uint16_t* o = static_cast<uint16_t*>(out) + 8 * t;
    unsigned int bad = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = __float_as_uint(round_bf16(x[e]));
      o[e] = (uint16_t)(b >> 16);
      bad |= b & 0xFFFFu;   // the low half must be +0: the value is the fp32 encoding of the bf16
    }
    if (bad) atomicOr(bad_low_half, 1u);
  } else if (kind == 1) {
    uint32_t* o = static_cast<uint32_t*>(out) + 4 * t;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(x[2 * p], x[2 * p + 1]);
  } else if (kind == 2) {
    uint8_t* o = static_cast<uint8_t*>(out) + 8 * t;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (uint8_t)e4m3_code(x[e]);
  } else if (kind == 3) {
    static_cast<uint32_t*>(out)[t] = pack_e2m1x8(x);
  } else if (kind == 4) {
    uint32_t* o = static_cast<uint32_t*>(out) + 2 * t;
    o[0] = fp8_quad(x[0], x[1], x[2], x[3]);
    o[1] = fp8_quad(x[4], x[5], x[6], x[7]);
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + 8 * t;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (uint16_t)f16_bits(x[e]);
  }
}

// One row of k = 64 * CPL bf16 per wavefront; a workgroup of four wavefronts owns rows
// r, r + 32, r + 64, r + 96 of a 128-row tile (one scale unit per four blocks); codes are the
// XOR of the loaded words (a value that depends on every byte read), scale units carry
// bytes of those codes.  Rows past m write zero scale bytes.
template <int CPL>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ x, int64_t m, uint32_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  constexpr int kChunks = CPL * kWave;
  __shared__ uint32_t sc[4][kChunks / 8];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const RowGroup g = row_group(blockIdx.x);
  const int64_t padded = (m + 127) / 128 * 128;
  if (g.tile * 128 >= padded) return;                    // uniform for the workgroup
  const int64_t r = g.tile * 128 + g.rr + 32 * wave;
  uint4 v[CPL];
  const int64_t rr = r < m ? r : m - 1;
#pragma unroll
  for (int j = 0; j < CPL; ++j) v[j] = load_stream(x + rr * kChunks + lane + kWave * j);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const uint32_t q = v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (r < m) store_stream(codes + r * kChunks + lane + kWave * j, q);
    if ((lane & 7) == 0) sc[wave][(lane >> 3) + 8 * j] = r < m ? q : 0u;
  }
  __syncthreads();
  for (int q = tid; q < kChunks / 8; q += 256) {
    const uint4 u = make_uint4(sc[0][q], sc[1][q], sc[2][q], sc[3][q]);
    // a plain store, as the producers use for scales: a 16-byte piece of a cache line must
    // meet the other pieces in L2 (a non-temporal store sends it on alone)
    *reinterpret_cast<NVFP4_GLOBAL uint4*>(global_ptr(scales) + g.tile * (kChunks / 8) * 512 + (int64_t)q * 512 +
                                           g.rr * 16) = u;
  }
}

}  // namespace

extern "C" {

// Bytes of output for `count` inputs of a conversion kind (count a multiple of 8), or -1.
int64_t nvfp4act_selftest_convert_bytes(int kind, int64_t count) {
  if (count < 0 || count % 8 != 0) return -1;
  switch (kind) {
    case 0: case 1: case 5: return 2 * count;
    case 2: case 4: return count;
    case 3: return count / 2;
    default: return -1;
  }
}

// Runs conversion `kind` over the fp32 bit patterns first .. first + count - 1 (count a
// positive multiple of 8, first + count <= 2^32) into the device buffer out (size
// nvfp4act_selftest_convert_bytes), one element per input in input order (kind 3: nibble i
// of word w is input 8w + i).  flag: one device uint32 that kind 0 ORs 1 into when a result
// has a nonzero low half.  Returns 0, 2 for bad arguments, or 6 for a launch error.
int nvfp4act_selftest_convert(int kind, uint32_t first, int64_t count, void* out, unsigned int* flag, void* stream) {
  if (nvfp4act_selftest_convert_bytes(kind, count) < 0 || count == 0 || !out || !flag) return 2;
  if ((int64_t)first + count > ((int64_t)1 << 32)) return 2;
  const int64_t groups = count / 8;
  const int64_t blocks = (groups + kConvThreads - 1) / kConvThreads;
  hipLaunchKernelGGL(convert_kernel, dim3((uint32_t)blocks), dim3(kConvThreads), 0, static_cast<hipStream_t>(stream),
                     kind, first, groups, out, flag);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// The bare traffic of an [m, k] producer call (see the file comment; k a multiple of 512, at
// most 8192): x [m, k] bf16, codes [m, k/2] bytes, scales [pad(m), k/16] bytes, all 16-byte
// aligned device memory.  Returns 0, 2 for bad arguments, or 6 for a launch error.
int nvfp4act_selftest_stream(const void* x, int64_t m, int64_t k, void* codes, void* scales, void* stream) {
  if (k <= 0 || k % 512 != 0 || k > 8192 || m <= 0 || !x || !codes || !scales) return 2;
  void (*kernels[16])(const uint4*, int64_t, uint32_t*, uint8_t*) = {
      stream_kernel<1>,  stream_kernel<2>,  stream_kernel<3>,  stream_kernel<4>,  stream_kernel<5>,  stream_kernel<6>,
      stream_kernel<7>,  stream_kernel<8>,  stream_kernel<9>,  stream_kernel<10>, stream_kernel<11>, stream_kernel<12>,
      stream_kernel<13>, stream_kernel<14>, stream_kernel<15>, stream_kernel<16>};
  hipLaunchKernelGGL(kernels[k / 512 - 1], dim3((uint32_t)row_group_blocks(m)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(x), m, static_cast<uint32_t*>(codes),
                     static_cast<uint8_t*>(scales));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
