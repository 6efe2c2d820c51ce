// swiglu.hip -- SwiGLU producer -> NVFP4 (FastVideo API page, swiglu_quantize over a
// value-first [M, 2F] projection; TensorRT-LLM PR #21483, SiLU-and-mul producer):
//   y = bf16(S[gate] * up),  S[g] = bf16(g * sigmoid(g)) correctly rounded
// followed by the NVFP4 block quantizer.  Two forms of the same kernel widen it:
// a bias added to value and gate before SiLU (swiglu_quantize's bias, as a bf16 add:
// up = bf16(up + bias_up), gate = bf16(gate + bias_gate)), and the paired column layout of
// the FastVideo branch compare's quant_probe (value of column j at 2j, gate at 2j + 1).
//
// S is a 65,536-entry bf16 table indexed by the gate's bit pattern, generated when the
// library is built (silu_tables_gen.cpp: fp64 evaluation, nearest-even, the build fails on
// an entry fp64 cannot decide) and loaded with the code object.  Each workgroup (one per CU, persistent over a
// set of 128-row x 512-column tiles) copies the 128 KiB table into its static LDS; every
// element then costs one LDS lookup, one multiply and one bf16 rounding before the
// quantizer.  Each tile's scale bytes are gathered in LDS and leave with 16-byte stores;
// codes are written with non-temporal stores (plain ones measured faster only for 16,384 to
// 24,576 rows, by 2.5 %, and 1 to 7 % slower at 4,096, 8,192, 32,768 and 49,152 rows and in
// the paired and bias forms).
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

__device__ const uint16_t g_silu_table[65536] = {
#include "silu_bf16.inc"
};

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kTableBytes = 65536 * sizeof(uint16_t);
constexpr int kTileCols = 512;                     // 64 chunks: one per lane per row
constexpr int kRowBatch = 4;                       // rows per wavefront in flight
constexpr int kScaleBytes = kTileCols / 64 * 512;  // 4 KiB

// The kernel arguments.  Two-pointer / value-first form: value row r at up + r*ld8 and gate
// row r at gate + r*ld8 (uint4 units).  Paired form: row r of the projection at up + r*ld8,
// output chunk c (8 columns) in its uint4s 2c and 2c+1, each 32-bit word holding one column's
// value (low half) and gate (high half); gate is unused.  bias_up / bias_gate: the bf16 bias
// of the value and gate columns (value-first), or bias_up alone as one paired row.
struct SwArgs {
  const uint4* up;
  const uint4* gate;
  const uint4* bias_up;
  const uint4* bias_gate;
  int64_t ld8, m, f;
  float global_amax;
  const float* amax_dev;
  float* amax_out;
  uint32_t* codes;
  uint8_t* scales;
  uint4* y_out;
  int64_t col_tiles, ntiles;
};

__device__ __forceinline__ uint32_t words_at(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}


// One batch: kRowBatch rows of one lane's chunk of a 128-row x kTileCols tile (wavefront w
// takes rows 4w .. 4w + 3 in batch 0 and 64 + 4w .. in batch 1), with the lane's 16 bias
// values.  Rows past the tensor repeat row m - 1 and lanes past the tile's chunks repeat
// the tile's last chunk pair (same parity), so every lane loads, computes and stores like
// a real one and the loop has no divergent branch; the duplicates store the same bytes
// as the lanes they repeat.
struct Batch {
  uint4 u[kRowBatch], g[kRowBatch];
  uint4 b0, b1;
};

struct TileAt {
  int64_t r0, c0, c;   // first row, first chunk, this lane's chunk (value-first)
  int64_t q[2];        // paired: this lane's two 16-byte column quads (row-relative index)
  int64_t tchunks;
};

__device__ __forceinline__ TileAt tile_at(const SwArgs& a, int64_t t, int lane) {
  const int64_t row_chunks = a.f >> 3;
  const int64_t tile_row = t / a.col_tiles, col_tile = t % a.col_tiles;
  TileAt o;
  o.r0 = tile_row << 7;
  o.c0 = col_tile * (kTileCols / 8);
  o.tchunks = (row_chunks - o.c0 < kTileCols / 8) ? row_chunks - o.c0 : kTileCols / 8;   // even
  o.c = o.c0 + (lane < o.tchunks ? lane : o.tchunks - 2 + (lane & 1));
  // paired: the tile row is 2 tchunks quads of four (value, gate) columns; lane L takes quads
  // L and L + 64, and a lane past the end repeats the last four quads (same position in its
  // block and pair)
  const int64_t nq = 2 * o.tchunks;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t k = lane + kWave * h;
    o.q[h] = 2 * o.c0 + (k < nq ? k : nq - 4 + (lane & 3));
  }
  return o;
}

template <bool PAIRED, bool BIAS>
__device__ __forceinline__ void load_batch(const SwArgs& a, const TileAt& at, int rb, Batch& b) {
#pragma unroll
  for (int i = 0; i < kRowBatch; ++i) {
    const int64_t r_own = at.r0 + rb + i;
    const int64_t r = r_own < a.m ? r_own : a.m - 1;
    if (PAIRED) {
      // quads L and L + 64: each load instruction reads 1 KiB contiguous
      b.u[i] = load_stream(a.up + r * a.ld8 + at.q[0]);
      b.g[i] = load_stream(a.up + r * a.ld8 + at.q[1]);
    } else {
      b.u[i] = load_stream(a.up + r * a.ld8 + at.c);
      b.g[i] = load_stream(a.gate + r * a.ld8 + at.c);
    }
  }
  if (BIAS) {
    if (PAIRED) {
      b.b0 = global_ptr(a.bias_up)[at.q[0]];
      b.b1 = global_ptr(a.bias_up)[at.q[1]];
    } else {
      b.b0 = global_ptr(a.bias_up)[at.c];
      b.b1 = global_ptr(a.bias_gate)[at.c];
    }
  }
}

// Quantize one batch; scale bytes go to the tile's LDS block (zero for rows past m).
// AMAX (the amax pass of a per-call scale): nothing is quantized or stored; max |y| is
// folded into *lane_amax.
template <bool AMAX, bool PAIRED, bool BIAS>
__device__ __forceinline__ void compute_batch(const SwArgs& a, const TileAt& at, int rb, const Batch& b,
                                              const uint16_t* table, float gsf, const float* inv_tab,
                                              uint8_t* tile_bytes, float* lane_amax) {
  const int64_t row_chunks = a.f >> 3;
  if (PAIRED) {
    // a 16-column block is the four quads of lanes 4i .. 4i + 3; each lane encodes its four
    // columns into 16 bits, and the lane pair (2i, 2i + 1) stores the 32-bit word of both
#pragma unroll
    for (int i = 0; i < kRowBatch; ++i) {
      const int rr = rb + i;
      const int64_t r_own = at.r0 + rr;
      const int64_t r = r_own < a.m ? r_own : a.m - 1;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 v = h == 0 ? b.u[i] : b.g[i];
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w = words_at(v, e);
          if (BIAS) w = add_bf16x2(w, words_at(h == 0 ? b.b0 : b.b1, e));
          const float s = __uint_as_float((uint32_t)table[w >> 16] << 16);
          y[e] = round_bf16(s * bf16_lo(w));
        }
        if (AMAX) {
          *lane_amax = max_abs2(max_abs2(*lane_amax, y[0], y[1]), y[2], y[3]);
          continue;
        }
        float am = max_abs2(max_abs2(0.0f, y[0], y[1]), y[2], y[3]);
        am = __uint_as_float(max_over_lane_quad(__float_as_uint(am)));
        const uint32_t s = e4m3_code(gsf * (am * __uint_as_float(kRcp6Bits)));
        const float inv = inv_tab[s];
        const uint32_t c16 = pack_e2m1x4(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv) & 0xFFFFu;
        const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)c16, 0xB1, 0xF, 0xF, true);
        const uint32_t word = (at.q[h] & 1) ? (other | (c16 << 16)) : (c16 | (other << 16));
        store_stream(reinterpret_cast<uint32_t*>(a.codes) + r * row_chunks + (at.q[h] >> 1), word);
        const int bt = (int)((at.q[h] - 2 * at.c0) >> 2);          // block within the tile
        tile_bytes[(bt >> 2) * 512 + (bt & 3) + (rr & 31) * 16 + ((rr >> 5) & 3) * 4] =
            r_own < a.m ? (uint8_t)s : (uint8_t)0;
        if (a.y_out)
          reinterpret_cast<NVFP4_GLOBAL uint2*>(global_ptr(a.y_out))[r * (a.f >> 2) + at.q[h]] =
              make_uint2(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]));
      }
    }
    return;
  }
  uint8_t* sc = tile_bytes + scale_lane_offset((int)(at.c - at.c0));
#pragma unroll
  for (int i = 0; i < kRowBatch; ++i) {
    const int rr = rb + i;
    float y[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t uw = words_at(b.u[i], q), gw = words_at(b.g[i], q);
      if (BIAS) {
        uw = add_bf16x2(uw, words_at(b.b0, q));
        gw = add_bf16x2(gw, words_at(b.b1, q));
      }
      const float s0 = __uint_as_float((uint32_t)table[gw & 0xFFFFu] << 16);
      const float s1 = __uint_as_float((uint32_t)table[gw >> 16] << 16);
      y[2 * q] = round_bf16(s0 * bf16_lo(uw));
      y[2 * q + 1] = round_bf16(s1 * bf16_hi(uw));
    }
    if (AMAX) {
      *lane_amax = fold_abs8(*lane_amax, y);
      continue;
    }
    uint32_t s;
    const uint32_t code = quantize_chunk(y, gsf, inv_tab, &s);
    const int64_t r_own = at.r0 + rr;
    const int64_t r = r_own < a.m ? r_own : a.m - 1;
    store_stream(reinterpret_cast<uint32_t*>(a.codes) + r * row_chunks + at.c, code);
    sc[(rr & 31) * 16 + ((rr >> 5) & 3) * 4] = r_own < a.m ? (uint8_t)s : (uint8_t)0;
    if (a.y_out)
      global_ptr(a.y_out)[r * row_chunks + at.c] =
          make_uint4(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]),
                     pack_exact_bf16x2(y[4], y[5]), pack_exact_bf16x2(y[6], y[7]));
  }
}

// A barrier that orders LDS only: __syncthreads would also wait for the prefetched loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One workgroup per CU, persistent over tiles t, t + grid, ...; each wavefront holds two
// batch buffers: while one batch is computed, the next one (the tile's second batch, or the
// next tile's first) is loading.
template <bool AMAX, bool PAIRED, bool BIAS>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const SwArgs a) {
  __shared__ float amax_red[kWaves];
  __shared__ uint4 lds4[kTableBytes / 16];
  __shared__ float inv_tab[128];
  __shared__ uint4 tile_sc[kScaleBytes / 16];
  uint16_t* table = reinterpret_cast<uint16_t*>(lds4);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if ((int64_t)blockIdx.x >= a.ntiles) return;            // idle workgroup (uniform)
  const int rb0 = wave * kRowBatch, rb1 = kWaves * kRowBatch + wave * kRowBatch;

  Batch A, B;
  TileAt at = tile_at(a, blockIdx.x, lane);
  load_batch<PAIRED, BIAS>(a, at, rb0, A);

  const float gsf = call_global_scale(a.global_amax, a.amax_dev);
  float lane_amax = 0.0f;
  fill_inverse_table(inv_tab, gsf, tid);
  const uint4* src = reinterpret_cast<const uint4*>(g_silu_table);
  for (int i = tid; i < (int)(kTableBytes / 16); i += kThreads) lds4[i] = src[i];
  for (int i = tid; i < kScaleBytes / 16; i += kThreads) tile_sc[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  uint8_t* tile_bytes = reinterpret_cast<uint8_t*>(tile_sc);
  for (int64_t t = blockIdx.x; t < a.ntiles; t += gridDim.x) {
    const int64_t tn = t + gridDim.x < a.ntiles ? t + gridDim.x : a.ntiles - 1;
    const TileAt next = tile_at(a, tn, lane);
    // the loads go out at a raised wavefront priority, ahead of other wavefronts' encoding
    __builtin_amdgcn_s_setprio(1);
    load_batch<PAIRED, BIAS>(a, at, rb1, B);
    __builtin_amdgcn_s_setprio(0);
    compute_batch<AMAX, PAIRED, BIAS>(a, at, rb0, A, table, gsf, inv_tab, tile_bytes, &lane_amax);
    __builtin_amdgcn_s_setprio(1);
    load_batch<PAIRED, BIAS>(a, next, rb0, A);
    __builtin_amdgcn_s_setprio(0);
    compute_batch<AMAX, PAIRED, BIAS>(a, at, rb1, B, table, gsf, inv_tab, tile_bytes, &lane_amax);
    if (!AMAX) {
      lds_barrier();
      // copy the tile's scale slice out and zero it for the next tile (each thread clears
      // exactly the words it copied)
      NVFP4_GLOBAL uint4* dst = reinterpret_cast<NVFP4_GLOBAL uint4*>(
          global_ptr(a.scales) + ((at.r0 >> 7) * (a.f >> 6) + at.c0 / 8) * 512);
      const int words = (int)(at.tchunks / 8) * 32;
      for (int i = tid; i < words; i += kThreads) {
        dst[i] = tile_sc[i];
        tile_sc[i] = make_uint4(0, 0, 0, 0);
      }
      lds_barrier();
    }
    at = next;
  }
  if (AMAX) workgroup_max_to(a.amax_out, lane_amax, amax_red, kWaves);
}

template <bool AMAX, bool PAIRED, bool BIAS>
hipError_t allow_lds() {
  (void)&swiglu_kernel<AMAX, PAIRED, BIAS>;   // static LDS only: nothing to allow
  return hipSuccess;
}

template <bool PAIRED, bool BIAS>
hipError_t launch_form(SwArgs a, int64_t grid, hipStream_t stream) {
  if (a.amax_out) {
    // per-call scale: zero the amax, fold max |y| into it, then quantize with it
    hipError_t e = launch_zero_amax(a.amax_out, stream);
    if (e != hipSuccess) return e;
    SwArgs p = a;
    p.amax_dev = nullptr;
    p.codes = nullptr;
    p.scales = nullptr;
    p.y_out = nullptr;
    hipLaunchKernelGGL((swiglu_kernel<true, PAIRED, BIAS>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.amax_dev = a.amax_out;
    a.amax_out = nullptr;
  }
  hipLaunchKernelGGL((swiglu_kernel<false, PAIRED, BIAS>), dim3((uint32_t)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t prepare_swiglu() {
  hipError_t e = allow_lds<false, false, false>();
  if (e == hipSuccess) e = allow_lds<true, false, false>();
  if (e == hipSuccess) e = allow_lds<false, false, true>();
  if (e == hipSuccess) e = allow_lds<true, false, true>();
  if (e == hipSuccess) e = allow_lds<false, true, false>();
  if (e == hipSuccess) e = allow_lds<true, true, false>();
  if (e == hipSuccess) e = allow_lds<false, true, true>();
  if (e == hipSuccess) e = allow_lds<true, true, true>();
  return e;
}

hipError_t launch_swiglu(const SwigluLaunch& p, const DeviceInfo& dev, hipStream_t stream) {
  const int64_t tile_rows = (p.m + 127) / 128;
  const int64_t col_tiles = (p.f + kTileCols - 1) / kTileCols;
  const int64_t ntiles = tile_rows * col_tiles;
  const int64_t grid = ntiles < dev.cu_count ? ntiles : dev.cu_count;
  SwArgs a;
  a.up = static_cast<const uint4*>(p.up);
  a.gate = static_cast<const uint4*>(p.gate);
  a.bias_up = static_cast<const uint4*>(p.bias_up);
  a.bias_gate = static_cast<const uint4*>(p.bias_gate);
  a.ld8 = p.ld / 8;
  a.m = p.m;
  a.f = p.f;
  a.global_amax = p.global_amax;
  a.amax_dev = nullptr;
  a.amax_out = p.amax_dev;
  a.codes = static_cast<uint32_t*>(p.codes);
  a.scales = static_cast<uint8_t*>(p.scales);
  a.y_out = static_cast<uint4*>(p.y_out);
  a.col_tiles = col_tiles;
  a.ntiles = ntiles;
  const bool bias = p.bias_up != nullptr;
  if (p.paired) return bias ? launch_form<true, true>(a, grid, stream) : launch_form<true, false>(a, grid, stream);
  return bias ? launch_form<false, true>(a, grid, stream) : launch_form<false, false>(a, grid, stream);
}

}  // namespace nvfp4act
