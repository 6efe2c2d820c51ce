// quantize.hip -- standalone NVFP4 quantize of a bf16 tensor (the attention-output
// quantize of TensorRT-LLM PR #21483; FastVideo API page, quantize).
//
// Bandwidth-bound: 2 bytes in, 0.5625 bytes out per element, a few VALU operations per
// element.  The launch is shaped for HBM streaming rather than for reuse:
//
// * One wavefront per row, non-persistent.  A wavefront issues the 16-byte loads of a whole
//   row piece (up to 1024 chunks = 8192 columns, 16 per lane) at once, quantizes it and
//   exits; workgroups are dispatched in row order, so the rows being read at any moment
//   form one compact window of the tensor and finished wavefronts are replaced at once.
//
// * A workgroup of four wavefronts owns the four rows r, r + 32, r + 64, r + 96 of a 128-row
//   tile (r = tile * 128 + rr, rr < 32).  In the 128x4 swizzled scale layout those rows'
//   scale bytes of four consecutive blocks form one contiguous 16-byte unit (row-group
//   major, then block), so the workgroup gathers the units of each row piece in LDS and
//   writes each with one 16-byte store; padding rows (>= m) contribute zero bytes.
//
// * The eight workgroups rr = 8p .. 8p + 7 of a tile fill the same 128-byte lines of the
//   scale buffer.  Block indices are arranged so that those eight are consecutive on one
//   XCD (workgroups are dealt round-robin over the 8 XCDs), so each line is completed in
//   one L2 before it is written back.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kWaves = 4;                  // rows per workgroup (r + 32 i)
constexpr int kThreads = kWaves * kWave;
constexpr int kPieceSlots = 16;            // chunks per lane per row piece (8192 columns)

// The 16-byte loads of SLOTS chunk slots (lane + 64 j, j < SLOTS) of a row from chunk c0.
template <int SLOTS>
__device__ __forceinline__ void load_piece(const NVFP4_GLOBAL uint4* xr, int64_t c0, int64_t chunks, int lane,
                                           uint4* v) {
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int64_t c = c0 + lane + kWave * j;
    v[j] = (c < chunks) ? load_stream(reinterpret_cast<const uint4*>(xr + c)) : make_uint4(0, 0, 0, 0);
  }
}

// Quantize the loaded piece and gather its scale bytes in the workgroup's LDS units of this
// piece (unit (c - c0) / 8, byte wave * 4 + block % 4).
template <int SLOTS>
__device__ __forceinline__ void quantize_piece(const uint4* v, NVFP4_GLOBAL uint32_t* cr, int64_t c0, int64_t chunks,
                                               int lane, int wave, float gsf, const float* inv_tab, uint8_t* units) {
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    const int64_t c = c0 + lane + kWave * j;
    float y[8] = {bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y), bf16_hi(v[j].y),
                  bf16_lo(v[j].z), bf16_hi(v[j].z), bf16_lo(v[j].w), bf16_hi(v[j].w)};
    const uint32_t s = block_scale_code(y, gsf);
    const uint32_t q = encode_chunk(y, inv_tab[s]);
    if (c < chunks) {
      cr[c] = q;
      units[((c - c0) >> 3) * 16 + wave * 4 + ((c >> 1) & 3)] = (uint8_t)s;
    }
  }
}

template <int SLOTS>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t m, int64_t k,
                                                            float global_amax, const float* amax_dev,
                                                            uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  constexpr int kPieceChunks = kWave * SLOTS;       // chunks per row piece
  constexpr int kPieceUnits = kPieceChunks / 8;     // 16-byte units per row-group piece
  __shared__ float inv_tab[128];
  __shared__ uint4 units[kPieceUnits];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const RowGroup g = row_group(blockIdx.x);
  const int64_t ntiles = (m + 127) >> 7;
  if (g.tile >= ntiles) return;                                     // idle workgroup (uniform)
  const int64_t chunks = k >> 3;
  const int64_t groups = k >> 6;                                    // 16-byte units per row group
  const int64_t r = (g.tile << 7) + g.rr + 32 * wave;
  const NVFP4_GLOBAL uint4* xr = global_ptr(x) + r * chunks;
  NVFP4_GLOBAL uint32_t* cr = global_ptr(codes) + r * chunks;
  // unit q of this row group sits at ((tile * k / 64) + q) * 512 + rr * 16
  NVFP4_GLOBAL uint8_t* dst = global_ptr(scales) + (g.tile * groups) * 512 + g.rr * 16;

  // the first piece is in flight while the inverse-scale table is built
  uint4 v[SLOTS];
  if (r < m) load_piece<SLOTS>(xr, 0, chunks, lane, v);
  const float gsf = call_global_scale(global_amax, amax_dev);
  fill_inverse_table(inv_tab, gsf, tid);
  for (int i = tid; i < kPieceUnits; i += kThreads) units[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  for (int64_t c0 = 0; c0 < chunks; c0 += kPieceChunks) {
    if (r < m) {
      if (c0 > 0) load_piece<SLOTS>(xr, c0, chunks, lane, v);
      quantize_piece<SLOTS>(v, cr, c0, chunks, lane, wave, gsf, inv_tab, reinterpret_cast<uint8_t*>(units));
    }
    __syncthreads();
    // the piece's units (zero bytes for rows >= m); each thread clears what it copied
    const int64_t q0 = c0 >> 3;
    for (int i = tid; i < kPieceUnits && q0 + i < groups; i += kThreads) {
      *reinterpret_cast<NVFP4_GLOBAL uint4*>(dst + (q0 + i) * 512) = units[i];
      units[i] = make_uint4(0, 0, 0, 0);
    }
    if (c0 + kPieceChunks < chunks) __syncthreads();
  }
}

template <int SLOTS>
hipError_t launch_slots(const uint4* x, int64_t m, int64_t k, float global_amax, const float* amax_dev,
                        uint32_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t blocks = row_group_blocks(m);
  hipLaunchKernelGGL((quantize_kernel<SLOTS>), dim3((uint32_t)blocks), dim3(kThreads), 0, stream, x, m, k,
                     global_amax, amax_dev, codes, scales);
  return hipGetLastError();
}

// ---- the amax pass of the per-call scale: max |x| over the tensor ----------------------
//
// A read-only stream over all m * k / 8 chunks: one workgroup per CU, each taking a
// contiguous run of 64 KiB steps (16-byte loads, kAmaxUnroll per thread in flight, 8 KiB
// apart); each workgroup folds its maximum into *amax with one atomic.  Two workgroups per
// CU striding over the whole tensor instead (each thread's loads 2 MiB apart) measured
// 148 us at 63,240 x 7168 against 131 here; the strided form also swung by 8 % with the
// grid size (1 MiB and 2 MiB strides the slowest).
constexpr int kAmaxThreads = 512;
constexpr int kAmaxUnroll = 8;
constexpr int64_t kAmaxStep = (int64_t)kAmaxThreads * kAmaxUnroll;   // chunks per workgroup step

__global__ __launch_bounds__(kAmaxThreads) void amax_x_kernel(const uint4* __restrict__ x, int64_t chunks,
                                                              float* amax) {
  __shared__ float red[kAmaxThreads / kWave];
  const int64_t steps = (chunks + kAmaxStep - 1) / kAmaxStep;
  const int64_t s0 = blockIdx.x * steps / gridDim.x, s1 = (blockIdx.x + 1) * steps / gridDim.x;
  float t = 0.0f;
  for (int64_t s = s0; s < s1; ++s) {
    const int64_t c = s * kAmaxStep + threadIdx.x;
    uint4 v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      v[u] = (c + kAmaxThreads * u < chunks) ? load_stream(x + c + kAmaxThreads * u) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const float y[8] = {bf16_lo(v[u].x), bf16_hi(v[u].x), bf16_lo(v[u].y), bf16_hi(v[u].y),
                          bf16_lo(v[u].z), bf16_hi(v[u].z), bf16_lo(v[u].w), bf16_hi(v[u].w)};
      t = fold_abs8(t, y);
    }
  }
  workgroup_max_to(amax, t, red, kAmaxThreads / kWave);
}

// *amax = 0 (the start of an amax pass), as a kernel so that the call stays capturable.
__global__ void zero_amax_kernel(float* amax) {
  if (threadIdx.x == 0) *global_ptr(amax) = 0.0f;
}

}  // namespace

hipError_t launch_zero_amax(float* amax, hipStream_t stream) {
  hipLaunchKernelGGL(zero_amax_kernel, dim3(1), dim3(64), 0, stream, amax);
  return hipGetLastError();
}

hipError_t launch_amax_x(const void* x, int64_t m, int64_t k, float* amax, const DeviceInfo& dev,
                         hipStream_t stream) {
  const int64_t chunks = m * (k / 8);
  int64_t blocks = (chunks + kAmaxStep - 1) / kAmaxStep;
  if (blocks > dev.cu_count) blocks = dev.cu_count;
  hipLaunchKernelGGL(amax_x_kernel, dim3((uint32_t)blocks), dim3(kAmaxThreads), 0, stream,
                     static_cast<const uint4*>(x), chunks, amax);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int64_t m, int64_t k, float global_amax, const float* amax_dev,
                           void* codes, void* scales, hipStream_t stream) {
  const uint4* xv = static_cast<const uint4*>(x);
  uint32_t* cv = static_cast<uint32_t*>(codes);
  uint8_t* sv = static_cast<uint8_t*>(scales);
  // chunk slots per lane: the whole row when it has at most 1024 chunks, else pieces of 16
  const int64_t slots = (k / 8 + kWave - 1) / kWave;
  switch (slots < kPieceSlots ? slots : kPieceSlots) {
    case 1: return launch_slots<1>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 2: return launch_slots<2>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 3: return launch_slots<3>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 4: return launch_slots<4>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 5: return launch_slots<5>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 6: return launch_slots<6>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 7: return launch_slots<7>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 8: return launch_slots<8>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 9: return launch_slots<9>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 10: return launch_slots<10>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 11: return launch_slots<11>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 12: return launch_slots<12>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 13: return launch_slots<13>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 14: return launch_slots<14>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    case 15: return launch_slots<15>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
    default: return launch_slots<16>(xv, m, k, global_amax, amax_dev, cv, sv, stream);
  }
}

}  // namespace nvfp4act
