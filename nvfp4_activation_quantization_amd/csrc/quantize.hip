// quantize.hip -- standalone NVFP4 quantize of a bf16 tensor (the attention-output
// quantize of TensorRT-LLM PR #21483; FastVideo API page, quantize).
//
// Bandwidth-bound: 2 bytes in, 0.5625 bytes out per element.  The tensor is cut into
// tiles of 128 rows x 1024 columns (the last column tile may be narrower).  One
// 256-thread workgroup per tile: each wavefront takes 32 of the rows, kRowBatch rows at a
// time so 2 x kRowBatch 1 KiB loads per wavefront are in flight.  The tile's scale bytes
// (16 groups of 4 blocks x 128 rows = 8 KiB, contiguous in the swizzled layout) are
// gathered in LDS and written out with 16-byte stores; rows m..pad(m)-1 stay zero.
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerWg = kThreads / kWave;
constexpr int kTileCols = 1024;                    // 128 chunks: 2 per lane per row
constexpr int kChunkSlots = kTileCols / 8 / kWave;  // 2
constexpr int kRowBatch = 4;                       // rows per wavefront in flight
constexpr int kScaleBytes = kTileCols / 64 * 512;  // 8 KiB

__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint4* __restrict__ x, int64_t m, int64_t k,
                                                            float global_amax, uint32_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t col_tiles) {
  __shared__ float inv_tab[128];
  __shared__ uint4 tile_sc[kScaleBytes / 16];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const float gsf = global_scale(global_amax);
  fill_inverse_table(inv_tab, gsf, tid);
  for (int i = tid; i < kScaleBytes / 16; i += kThreads) tile_sc[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int64_t tile_row = blockIdx.x / col_tiles;
  const int64_t col_tile = blockIdx.x % col_tiles;
  const int64_t c0 = col_tile * (kTileCols / 8);                 // first chunk of the tile
  const int64_t row_chunks = k >> 3;
  const int64_t tchunks = (row_chunks - c0 < kTileCols / 8) ? row_chunks - c0 : kTileCols / 8;
  const int64_t r0 = tile_row << 7;
  const int64_t rows = (m - r0 < 128) ? (m - r0 > 0 ? m - r0 : 0) : 128;   // real rows of the tile
  uint8_t* sc_lane = reinterpret_cast<uint8_t*>(tile_sc) + scale_lane_offset(lane);

  for (int64_t rb = wave * kRowBatch; rb < rows; rb += kWavesPerWg * kRowBatch) {
    uint4 v[kRowBatch][kChunkSlots];
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t rr = rb + i;
#pragma unroll
      for (int j = 0; j < kChunkSlots; ++j) {
        const int64_t c = j * kWave + lane;
        if (rr < rows && c < tchunks)
          v[i][j] = load_stream(reinterpret_cast<const uint4*>(global_ptr(x) + (r0 + rr) * row_chunks + c0 + c));
        else
          v[i][j] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int64_t rr = rb + i;
      const int row_part = (int)((rr & 31) * 16 + ((rr >> 5) & 3) * 4);
#pragma unroll
      for (int j = 0; j < kChunkSlots; ++j) {
        const int64_t c = j * kWave + lane;
        float y[8] = {bf16_lo(v[i][j].x), bf16_hi(v[i][j].x), bf16_lo(v[i][j].y), bf16_hi(v[i][j].y),
                      bf16_lo(v[i][j].z), bf16_hi(v[i][j].z), bf16_lo(v[i][j].w), bf16_hi(v[i][j].w)};
        uint32_t s;
        const uint32_t q = quantize_chunk(y, gsf, inv_tab, &s);
        if (rr < rows && c < tchunks) {
          global_ptr(codes)[(r0 + rr) * row_chunks + c0 + c] = q;
          sc_lane[row_part + 4096 * j] = (uint8_t)s;
        }
      }
    }
  }
  __syncthreads();
  // the tile's scale slice: (tchunks / 8) groups of 512 bytes, contiguous in the layout
  NVFP4_GLOBAL uint4* dst = reinterpret_cast<NVFP4_GLOBAL uint4*>(
      global_ptr(scales) + (tile_row * (k >> 6) + c0 / 8) * 512);
  const int words = (int)(tchunks / 8) * 32;
  for (int i = tid; i < words; i += kThreads) dst[i] = tile_sc[i];
}

}  // namespace

hipError_t launch_quantize(const void* x, int64_t m, int64_t k, float global_amax, void* codes,
                           void* scales, hipStream_t stream) {
  const int64_t tile_rows = (m + 127) / 128;
  const int64_t col_tiles = (k + kTileCols - 1) / kTileCols;
  hipLaunchKernelGGL(quantize_kernel, dim3((uint32_t)(tile_rows * col_tiles)), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(x), m, k, global_amax, static_cast<uint32_t*>(codes),
                     static_cast<uint8_t*>(scales), col_tiles);
  return hipGetLastError();
}

}  // namespace nvfp4act
