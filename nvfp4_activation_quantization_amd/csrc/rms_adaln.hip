// rms_adaln.hip -- fused RMSNorm (fp32 statistic) + adaLN modulation -> NVFP4, the
// AdaLN RMSNorm + modulation producer of TensorRT-LLM PR #21483, with every bf16 rounding
// of the op-by-op eager path kept (FastVideo API page, module summary):
//   rstd = 1 / sqrt(sum(x^2) / k + eps)
//   y    = bf16(bf16(bf16(bf16(x * rstd) * w) * bf16(1 + scale[t])) + shift[t])
// followed by the NVFP4 block quantizer.
//
// One workgroup per CU, persistent over a contiguous range of rows.  The RMSNorm weight
// and the current frame's modulation row are staged once in LDS as fp32 (bf16(1 + scale)
// precomputed); a frame change restages them behind two barriers.  A row whose frame is
// not the staged one (possible only for unsorted frame indices) reads its modulation row
// from global memory instead.  Each wavefront holds its row in registers between the
// statistic and the output pass, so x is read from HBM once.
//
// The statistic uses the fixed tree of the specification: lane L owns chunks L + 64j,
// keeps 8 accumulators (fused multiply-add), folds them pairwise, and a butterfly over the
// 64 lanes at distances 1..32 adds the lane values (every lane ends with the same sum).
#include "common.hpp"
#include "kernels.hpp"

namespace nvfp4act {

namespace {




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
  const float* amax_dev;   // per-call scale: the amax pass's result (null: static global_amax)
  float* amax_out;         // the amax pass: where max |y| is folded
  int unit_shift;          // staged kernel: 7 for a full-size tensor (4S-row units), else a short tensor's
                           // contiguous units of 1 << unit_shift rows (3 .. 6)
  int64_t head_units;      // full-size tensor: the units of 4S rows; the rows after them form 8-row units
};

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// The 8 values of a chunk from its four float2 planes (elements 0-1, 2-3, 4-5, 6-7).
__device__ __forceinline__ void split8(const float2& a, const float2& b, const float2& c, const float2& d,
                                       float* f) {
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y; f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// Store the 8 values of chunk c into four float2 planes of `chunks` entries each.
__device__ __forceinline__ void store_planes(float2* planes, int chunks, int c, const float* f) {
  planes[c] = make_float2(f[0], f[1]);
  planes[chunks + c] = make_float2(f[2], f[3]);
  planes[2 * chunks + c] = make_float2(f[4], f[5]);
  planes[3 * chunks + c] = make_float2(f[6], f[7]);
}

// y = bf16(bf16(bf16(bf16(x * rstd) * w) * opl) + shift) for the 8 elements of a chunk.
// Every rounding is v_cvt_pk_bf16_f32 with a zero low operand, whose result is the fp32
// encoding of the rounded value (round_bf16).  Each step is issued for all eight elements
// before the next one starts: left to itself the scheduler runs the eight dependent chains
// one after another when registers are scarce, and a wavefront then waits on every result.
// A scheduling barrier that no vector ALU instruction may cross (memory, LDS and scalar
// instructions may) separates the steps; inline assembly would order them too, but the
// compiler pads the uses of an assembly result with wait states.  The operations are those
// of the definition, in its order, so the results are the same bits.
#define NVFP4_STEP_FENCE() __builtin_amdgcn_sched_barrier(0x3F4)
__device__ __forceinline__ void modulate8(const float* x8, const float* w8, const float* o8,
                                          const float* h8, float rstd, float* y) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = x8[e] * rstd;
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = round_bf16(t[e]);
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = t[e] * w8[e];
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = round_bf16(t[e]);
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = t[e] * o8[e];
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = round_bf16(t[e]);
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = t[e] + h8[e];
  NVFP4_STEP_FENCE();
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = round_bf16(t[e]);
  NVFP4_STEP_FENCE();
}

// Per-row output cursors of one lane: chunk j of the lane is chunk c = lane + 64 j.
struct RowOut {
  NVFP4_GLOBAL uint32_t* codes;    // codes of chunk c at codes[64 j]
  NVFP4_GLOBAL uint8_t* scales;    // scale byte of chunk c's block at scales[4096 j]
  NVFP4_GLOBAL uint4* y;           // y_out of chunk c at y[64 j], or null
  uint8_t* scales_lds;             // the same byte in the unit's padded LDS block, at [lds_chunk_stride(CPL) j] (TILE)
};

// Units of a full-size tensor (see the staged kernel): S consecutive rows of each of the
// four 32-row groups of a 128-row tile, 4 S rows in all; S = 16 from k = 2048 to 7680, 8 at
// k = 8192 (where two 16-row blocks do not fit beside the parameters), 32 below 2048.
// Smaller units keep the rows in flight closer together but restage the frame's modulation
// row more often when frames change every few thousand rows (measured at 63,240 x 7168, 31
// frames: 229 us with S = 16, 231 with 8, 234 in 128-row tiles; at 300,000 x 7168: 1,056 /
// 1,043 / 1,077; k = 4096 prefers 16, k <= 2048 is within 1 % either way).  The unit's
// scale bytes are 16 S contiguous bytes of each column group's 512-byte swizzled run; its
// LDS block holds them padded to 16 S + 16 bytes per group, so that the eight column groups
// one wavefront writes for a chunk fall in different banks.
constexpr int unit_rows_per_group(int cpl) { return cpl >= 16 ? 8 : cpl >= 4 ? 16 : 32; }
constexpr int lds_group_bytes(int cpl) { return 16 * unit_rows_per_group(cpl) + 16; }
constexpr int lds_chunk_stride(int cpl) { return 8 * lds_group_bytes(cpl); }   // chunk j + 1: 8 groups on

__device__ __forceinline__ RowOut make_row_out(uint32_t* codes, uint8_t* scales, uint4* y_out, int64_t k,
                                               int64_t r, int lane) {
  const int64_t chunks = k >> 3;
  RowOut o;
  o.codes = global_ptr(codes) + r * chunks + lane;
  o.scales = global_ptr(scales) + row_scale_base(r, k) + scale_lane_offset(lane);
  o.y = y_out ? global_ptr(y_out) + r * chunks + lane : nullptr;
  o.scales_lds = nullptr;
  return o;
}

__device__ __forceinline__ RowOut row_out(const RmsArgs& a, int64_t r, int lane) {
  return make_row_out(a.codes, a.scales, a.y_out, a.k, r, lane);
}

// Quantize chunk j of a row and store its codes, its block's scale byte (into the unit's
// LDS block with TILE, else to memory) and, with Y, y_out.  No branches, so consecutive
// chunks can be scheduled together.
template <bool Y, bool TILE>
__device__ __forceinline__ void emit_chunk(const RowOut& o, int j, const float* y, float gsf,
                                           const float* inv_tab, int lds_stride) {
  uint32_t s;
  const uint32_t q = quantize_chunk(y, gsf, inv_tab, &s);
  o.codes[kWave * j] = q;
  if (TILE) o.scales_lds[lds_stride * j] = (uint8_t)s;
  else o.scales[(int64_t)4096 * j] = (uint8_t)s;
  if (Y)
    o.y[kWave * j] = make_uint4(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]),
                                pack_exact_bf16x2(y[4], y[5]), pack_exact_bf16x2(y[6], y[7]));
}

// lds_stride: with tile (the unit's LDS scale block), the byte distance between a lane's
// chunks in that block
__device__ __forceinline__ void store_chunk(const RowOut& o, int j, const float* y, float gsf,
                                            const float* inv_tab, bool tile, int lds_stride) {
  if (tile) {
    if (o.y) emit_chunk<true, true>(o, j, y, gsf, inv_tab, lds_stride);
    else emit_chunk<false, true>(o, j, y, gsf, inv_tab, lds_stride);
  } else {
    if (o.y) emit_chunk<true, false>(o, j, y, gsf, inv_tab, 0);
    else emit_chunk<false, false>(o, j, y, gsf, inv_tab, 0);
  }
}

// Write row r as zeros (frame index outside [0, num_frames)); its scale bytes go to
// memory only when they are not gathered in a zeroed LDS block.
__device__ void zero_row(const RmsArgs& a, int64_t r, int lane, bool scales_too) {
  const int64_t chunks = a.k >> 3;
  for (int64_t c = lane; c < chunks; c += kWave) {
    global_ptr(a.codes)[r * chunks + c] = 0u;
    if (a.y_out) global_ptr(a.y_out)[r * chunks + c] = make_uint4(0, 0, 0, 0);
  }
  if (scales_too) zero_row_scales(a.scales, r, a.k, lane);
  if (lane == 0 && a.status) atomicOr(a.status, 1u);
}

// The modulation row of frame t, chunk c, as fp32: o8 = bf16(1 + scale), h8 = shift.
__device__ __forceinline__ void load_frame_chunk(const uint16_t* shift, const uint16_t* scale,
                                                 int64_t frame_stride, int64_t t, int64_t c, float* o8,
                                                 float* h8) {
  const uint4 sc = *reinterpret_cast<const NVFP4_GLOBAL uint4*>(global_ptr(scale) + t * frame_stride + 8 * c);
  const uint4 sh = *reinterpret_cast<const NVFP4_GLOBAL uint4*>(global_ptr(shift) + t * frame_stride + 8 * c);
  unpack8(sc, o8);
#pragma unroll
  for (int e = 0; e < 8; ++e) o8[e] = round_bf16(1.0f + o8[e]);
  unpack8(sh, h8);
}

__device__ __forceinline__ void load_frame_chunk(const RmsArgs& a, int64_t t, int64_t c, float* o8,
                                                 float* h8) {
  load_frame_chunk(a.shift, a.scale, a.frame_stride, t, c, o8, h8);
}

// A row whose frame is not the staged one: re-read x (an L2 hit in practice) and the
// frame's modulation row from global memory, one chunk at a time.  Out of line and with
// plain arguments, so the kernel's hot loop is not shaped by this rare path.  In the amax
// pass (amax_only) nothing is stored and the lane's max |y| is returned (else 0).
__device__ __noinline__ float emit_row_unstaged(const uint4* x, const uint16_t* shift, const uint16_t* scale,
                                                int64_t frame_stride, RowOut o, int64_t k, int64_t r, int64_t t,
                                                const float2* wp, float rstd, float gsf,
                                                const float* inv_tab, bool tile, int lds_stride, bool amax_only) {
  const int lane = threadIdx.x & (kWave - 1);
  const NVFP4_GLOBAL uint4* xr = global_ptr(x) + r * (k >> 3);
  float lane_amax = 0.0f;
#pragma unroll 1
  for (int j = 0; j < (int)(k >> 9); ++j) {
    const int64_t c = lane + (int64_t)kWave * j;
    float x8[8], w8[8], o8[8], h8[8], y[8];
    unpack8(xr[c], x8);
    const int chunks = (int)(k >> 3);
    split8(wp[c], wp[chunks + c], wp[2 * chunks + c], wp[3 * chunks + c], w8);
    load_frame_chunk(shift, scale, frame_stride, t, c, o8, h8);
    modulate8(x8, w8, o8, h8, rstd, y);
    if (amax_only) lane_amax = fold_abs8(lane_amax, y);
    else store_chunk(o, j, y, gsf, inv_tab, tile, lds_stride);
  }
  return lane_amax;
}

// The float2 at byte offset base + off of the dynamic LDS block.
__device__ __forceinline__ float2 lds_f2(const float4* lds, uint32_t base, uint32_t off) {
  return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(lds) + base + off);
}

// The twelve float2 parameter values of chunk j (weight, 1 + scale, shift; four planes
// each) from the LDS plane bases of this lane.
__device__ __forceinline__ void load_params(const float4* lds, uint32_t pw, uint32_t po, uint32_t ph,
                                            uint32_t plane, int j, float2* p) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p[q] = lds_f2(lds, pw, q * plane + 512 * j);
    p[4 + q] = lds_f2(lds, po, q * plane + 512 * j);
    p[8 + q] = lds_f2(lds, ph, q * plane + 512 * j);
  }
}

// Encode chunk j (its y, scale code s and inverse scale inv) and store its codes, its
// block's scale byte (into the unit's LDS block with TILE, else to memory) and, with Y,
// y_out.
template <int CPL, bool Y, bool TILE>
__device__ __forceinline__ void emit_encoded(const RowOut& o, int j, const float* y, float inv, uint32_t s) {
  __builtin_nontemporal_store(encode_chunk(y, inv), o.codes + kWave * j);   // not read back
  if (TILE) o.scales_lds[lds_chunk_stride(CPL) * j] = (uint8_t)s;
  else o.scales[(int64_t)4096 * j] = (uint8_t)s;
  if (Y)
    o.y[kWave * j] = make_uint4(pack_exact_bf16x2(y[0], y[1]), pack_exact_bf16x2(y[2], y[3]),
                                pack_exact_bf16x2(y[4], y[5]), pack_exact_bf16x2(y[6], y[7]));
}

// The CPL chunks of a row, issued in chunk order: every path that loads a row then leaves
// chunk 0 oldest, which lets the compiler wait for each chunk of the next statistic
// separately instead of for (nearly) every outstanding load and store at its start.
template <int CPL>
__device__ __forceinline__ void load_row(uint4* v, const NVFP4_GLOBAL uint4* xr, int lane) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    v[j] = load_stream(reinterpret_cast<const uint4*>(xr + lane + kWave * j));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- the staged kernel (k <= 8192, CPL = k / 512 chunks per lane) -------------------------
//
// One workgroup of 8 wavefronts per CU, persistent over units of 4 S rows (unit v, v +
// grid, ...; see unit_row): the eight rows in flight at any time are consecutive and share
// a frame except at frame boundaries, every wavefront has the same S / 2 rows of work per
// unit, and consecutive units run on consecutive CUs.  The rows after the last full round
// of units run in 8-row units, a contiguous run of them per workgroup, when that takes rows
// off the busiest CU.  A tensor with fewer 128-row tiles than CUs is cut into contiguous
// units instead (64 rows down to 8, one row per wavefront), enough of them to occupy the
// CUs, and stores its scale bytes directly.
//
// Each wavefront keeps its current row unpacked to fp32 in registers (8 CPL values per
// lane) from the statistic to the output pass, so every element is unpacked once.  The
// packed registers (4 CPL) are free once the statistic has unpacked them: in the output
// pass the loads of the next row's chunks are issued as chunks are modulated (one per
// chunk, or two for k <= 4096, into the registers each modulated chunk frees), so the next
// row arrives during the rest of the pass.
//
// LDS: inverse-scale table (128 fp32); twelve fp32 planes of float2 indexed by chunk (weight
// elements 0-1, 2-3, 4-5, 6-7, then bf16(1 + scale) and shift alike), so each ds_read_b64
// of a wavefront is one contiguous 512 bytes; and, with TILE, two scale blocks of a unit
// (the unit's 16 S bytes of each column group, padded to 16 S + 16: unpadded, the eight
// groups a wavefront writes for one chunk would share one LDS bank) and two blocks of the
// unit's 4 S rstd values.  With TILE the scale bytes are gathered in LDS and leave as
// whole 128-byte lines, 16 bytes per store (padding rows stay zero); without TILE (the
// amax pass, or a short tensor's small units) each byte is stored directly.

constexpr int kStagedWaves = 8;

// AMAX: the amax pass of a per-call scale -- the same rows and chain, no quantizer and no
// stores; each workgroup folds its max |y| into a.amax_out (rows with an out-of-range frame
// have y = 0 and contribute nothing).
template <int CPL, bool Y, bool TILE, bool AMAX>
__global__ __launch_bounds__(kStagedWaves * kWave) void rms_adaln_staged(RmsArgs a, const int32_t* __restrict__ frame_idx) {
  static_assert(!(AMAX && (TILE || Y)), "the amax pass writes no outputs");
  __shared__ float amax_red[kStagedWaves];
  constexpr int WAVES = kStagedWaves;
  constexpr int kThreads = WAVES * kWave;
  constexpr int kChunks = CPL * kWave;          // chunks per row (k / 8)
  constexpr int kGroups = kChunks / 8;           // 512-byte column groups of the swizzled layout (k/64)
  constexpr int kS = unit_rows_per_group(CPL);    // a full-size unit: kS rows of each 32-row group
  constexpr int kGroupBytes = lds_group_bytes(CPL);
  constexpr int kUnitLdsBytes = kGroups * kGroupBytes;     // one unit's scale block
  constexpr int kK = kChunks * 8;
  extern __shared__ float4 lds4[];
  float* inv_tab = reinterpret_cast<float*>(lds4);
  float2* wp = reinterpret_cast<float2*>(lds4 + 32);   // after 128 floats = 32 float4
  float2* op = wp + 4 * kChunks;
  float2* hp = op + 4 * kChunks;
  // TILE: two unit scale blocks (used in turn, so one barrier per unit suffices), then
  // two blocks of the unit's 4 kS rstd values
  uint8_t* unit_sc = reinterpret_cast<uint8_t*>(hp + 4 * kChunks);
  float* rstd_unit = reinterpret_cast<float*>(unit_sc + 2 * kUnitLdsBytes);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const NVFP4_GLOBAL uint4* x = global_ptr(a.x);
  const int64_t m = a.m;
  // Units of rows.  A full-size tensor (unit_shift 7) is cut into units of 4 kS rows: unit
  // v holds rows kS j .. kS j + kS - 1 (j = v mod 32 / kS) of each 32-row group of tile
  // v / (32 / kS).  Those rows own 16 kS contiguous bytes of every column group's 512-byte
  // run in the swizzled scale layout (whole 128-byte lines), and consecutive units run on
  // consecutive CUs, so the rows in flight stay within a window of 4 kS rows per CU.  The
  // unit's n-th eight rows (n = 0 .. kS / 2 - 1) are consecutive: item 8 n + w of the unit is
  // row s = (8 n + w) mod kS of group (8 n + w) / kS, taken by wavefront w.  When the units
  // would leave a last round that keeps some CUs busy while others idle, only the first
  // head_units are such units and the tiles after them run in units of 8 consecutive rows,
  // one per wavefront, whose scale bytes are 4-byte pieces of the swizzled layout.  Units
  // of 4 kS rows go round-robin over the workgroups; each workgroup then takes a contiguous
  // run of the 8-row units (the pieces of one 128-byte line come mostly from one CU, where
  // the cache merges them).  A short tensor runs in contiguous units of 2^unit_shift rows
  // (8 .. 64), 2^unit_shift / 8 per wavefront, round-robin.
  constexpr int kUnitsPerTile = 32 / kS;
  // Next-row loads issued per modulated chunk of the output pass.  Two per chunk put the
  // whole next row in flight by mid-pass, which short rows need (random input, 63,240 /
  // 150,000 rows: k = 2048 82.0 -> 78.9 / 180.6 -> 172.9 us, k = 3072 110.9 -> 107.4 /
  // 246.0 -> 243.3, k = 4096 136.0 -> 133.4 / 309.3 -> 301.2); from k = 5120 on, where the
  // pass is long, it gains nothing and costs 1 % at k = 7168 (229.6 -> 233.1 us).  The amax
  // pass, whose output pass has no quantizer and no stores, takes two at every k (whole
  // per-call form at 63,240 / 300,000 x 7168: 403.8 -> 402.3 / 1,849 -> 1,839 us).
  constexpr int kAhead = (AMAX || CPL <= 8) ? 2 : 1;
  const bool quarter = TILE || a.unit_shift == 7;
  const int ushift = a.unit_shift;
  const int64_t head = quarter ? a.head_units : 0;
  const int64_t nunits = quarter ? head + ((a.padded - head * 4 * kS) >> 3) : a.padded >> ushift;
  const int64_t nrr = quarter ? head : nunits;          // units taken round-robin
  const int64_t bid = blockIdx.x, nwg = gridDim.x;
  const int64_t mine_rr = nrr > bid ? (nrr - bid + nwg - 1) / nwg : 0;
  const int64_t t0 = bid * (nunits - nrr) / nwg, t1 = (bid + 1) * (nunits - nrr) / nwg;
  const int64_t mine = mine_rr + (t1 - t0);
  if (mine == 0) return;                                 // idle workgroup (uniform)
  auto unit_of = [&](int64_t n) -> int64_t { return n < mine_rr ? bid + n * nwg : nrr + t0 + (n - mine_rr); };
  auto unit_row = [&](int64_t v, int n, int w) -> int64_t {
    if (!quarter) return (v << ushift) + WAVES * n + w;
    if (v < head) {
      const int item = 8 * n + w;
      return (v / kUnitsPerTile) * 128 + 32 * (item / kS) + kS * (int)(v % kUnitsPerTile) + item % kS;
    }
    return (head / kUnitsPerTile) * 128 + 8 * (v - head) + w;   // an 8-row unit (n == 0)
  };
  // Byte offsets of this lane's chunk 0 in the weight, 1 + scale and shift planes.  The
  // four planes of one parameter and their 64-lane steps then lie within the 16-bit
  // immediate offset of one ds_read_b64 base; hiding the three bases from the optimiser
  // keeps it from materialising one address per plane and chunk (the planes together span
  // more than the immediate range).  Each read is 8 bytes per lane, consecutive across
  // the wavefront: ds_read_b64 runs at twice the LDS bandwidth of ds_read_b128 on gfx950.
  constexpr uint32_t kPlane = kChunks * 8;
  uint32_t pw = 512 + 8 * lane, po = pw + 4 * kPlane, ph = pw + 8 * kPlane;
  asm volatile("" : "+v"(pw), "+v"(po), "+v"(ph));

  // The first row of this wavefront is in flight while the parameters are staged (loads
  // are unconditional: a row past the end re-reads row m - 1, which is never used).
  uint4 xr[CPL];
  {
    const int64_t r0 = unit_row(unit_of(0), 0, wave);
    load_row<CPL>(xr, x + (r0 < m ? r0 : m - 1) * kChunks, lane);
  }

  // The weight and the first row group's frame are staged together, so a workgroup with
  // one unit (a short tensor) waits for one round of global loads before its first row
  // instead of two (the frame used to be staged behind a barrier of its own).
  int64_t staged = -1;
  {
    const int64_t g0 = unit_row(unit_of(0), 0, 0);
    if (g0 < m) {
      const int64_t t = frame_idx[g0];
      if (t >= 0 && t < a.num_frames) staged = t;
    }
  }
  const float gsf = call_global_scale(a.global_amax, a.amax_dev);
  float lane_amax = 0.0f;
  fill_inverse_table(inv_tab, gsf, tid);
  for (int c = tid; c < kChunks; c += kThreads) {
    float f[8], o8[8], h8[8];
    unpack8(*reinterpret_cast<const NVFP4_GLOBAL uint4*>(global_ptr(a.w) + 8 * c), f);
    if (staged >= 0) load_frame_chunk(a, staged, c, o8, h8);
    store_planes(wp, kChunks, c, f);
    if (staged >= 0) {
      store_planes(op, kChunks, c, o8);
      store_planes(hp, kChunks, c, h8);
    }
  }
  if (TILE)
    for (int i = tid; i < 2 * kUnitLdsBytes / 16; i += kThreads)
      reinterpret_cast<uint4*>(unit_sc)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  int par = 0;                                          // TILE: the unit's scale block
  for (int64_t n = 0; n < mine; ++n) {
    const int64_t v = unit_of(n);
    // this wave's row in the next unit (after the last unit: any row, loaded and not used)
    const int64_t next_first = n + 1 < mine ? unit_row(unit_of(n + 1), 0, wave) : m - 1;
    const int rows_per_wave = !quarter ? (1 << ushift) / WAVES : v < head ? kS / 2 : 1;
    for (int i = 0; i < rows_per_wave; ++i) {
      const int64_t g = unit_row(v, i, 0);             // the first row of the 8 in flight
      // restage the modulation row when the group's first row needs another frame (uniform)
      int64_t want = staged;
      if (g < m) {
        const int64_t t = frame_idx[g];
        if (t >= 0 && t < a.num_frames) want = t;
      }
      if (want != staged) {
        __syncthreads();
        for (int c = tid; c < kChunks; c += kThreads) {
          float o8[8], h8[8];
          load_frame_chunk(a, want, c, o8, h8);
          store_planes(op, kChunks, c, o8);
          store_planes(hp, kChunks, c, h8);
        }
        __syncthreads();
        staged = want;
      }
      const int64_t r = unit_row(v, i, wave);
      if (r >= m) {                        // a padding row (and so is every later row)
        if (!TILE && !AMAX) zero_row_scales(a.scales, r, kK, lane);   // TILE: already zero in LDS
        continue;
      }
      // this wavefront's next row (loaded chunk by chunk during the output pass)
      int64_t rn = (i + 1 < rows_per_wave) ? unit_row(v, i + 1, wave) : next_first;
      rn = rn < m ? rn : m - 1;
      // the row arrived during the previous row's output pass: unpack it once and take the
      // statistic; the next row's chunks are loaded into the packed registers one by one in
      // the output pass, each as soon as the chunk that occupied its place is modulated
      float xf[CPL][8];
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        unpack8(xr[j], xf[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(xf[j][e], xf[j][e], acc[e]);
      }
      const NVFP4_GLOBAL uint4* xn = x + rn * kChunks;
      const float sum = lane_sum_butterfly(((acc[0] + acc[1]) + (acc[2] + acc[3])) +
                                           ((acc[4] + acc[5]) + (acc[6] + acc[7])));
      const float rstd = 1.0f / sqrtf(sum / (float)kK + a.eps);
      // rstd_out: with TILE gathered per unit in LDS and written at the unit's end
      // (4-byte stores one row apart, each leaving a partial cache line, cost up to 7 % of
      // the kernel's time at k = 2048), else stored directly
      if (!AMAX && a.rstd_out && lane == 0) {
        if (TILE) rstd_unit[4 * kS * par + 8 * i + wave] = rstd;
        else global_ptr(a.rstd_out)[r] = rstd;
      }
      const int64_t t = frame_idx[r];
      if (t < 0 || t >= a.num_frames) {
        if (!AMAX) zero_row(a, r, lane, !TILE);
        load_row<CPL>(xr, xn, lane);
        continue;
      }
      RowOut o = row_out(a, r, lane);
      // item 8 i + w (row s of group g) sits at byte 16 s + 4 g of the unit's bytes in a column
      // group (an 8-row unit: row w at byte 4 w)
      if (TILE) {
        const int item = 8 * i + wave;
        const int at = v < head ? 16 * (item % kS) + 4 * (item / kS) : 4 * wave;
        o.scales_lds = unit_sc + par * kUnitLdsBytes + (lane >> 3) * kGroupBytes + at + ((lane >> 1) & 3);
      }
      if (t != staged) {
        const float u = emit_row_unstaged(a.x, a.shift, a.scale, a.frame_stride, o, kK, r, t, wp, rstd, gsf,
                                          inv_tab, TILE, lds_chunk_stride(CPL), AMAX);
        lane_amax = __builtin_fmaxf(lane_amax, u);
        load_row<CPL>(xr, xn, lane);
        continue;
      }
      // Output pass, software-pipelined over the lane's chunks: the parameters of chunk j + 1
      // are read from LDS while chunk j is modulated, and chunk j's inverse scale (an LDS
      // table lookup) is consumed only after chunk j + 1 has been modulated, so neither LDS
      // round trip sits on the critical path of a chunk.
      float2 pc[12], pn[12];
      load_params(lds4, pw, po, ph, kPlane, 0, pc);
      float yp[8];
      uint32_t sp = 0;
      float invp = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        if (j + 1 < CPL) load_params(lds4, pw, po, ph, kPlane, j + 1, pn);
        float w8[8], o8[8], h8[8], y[8];
        split8(pc[0], pc[1], pc[2], pc[3], w8);
        split8(pc[4], pc[5], pc[6], pc[7], o8);
        split8(pc[8], pc[9], pc[10], pc[11], h8);
        modulate8(xf[j], w8, o8, h8, rstd, y);
        // the next row's chunks: kAhead per modulated chunk (the freed registers of one fp32
        // chunk hold two packed ones), so that the last of them leave early in the pass
#pragma unroll
        for (int q = kAhead * j; q < kAhead * j + kAhead; ++q)
          if (q < CPL) xr[q] = load_stream(reinterpret_cast<const uint4*>(xn + lane + kWave * q));
        if (AMAX) {
          lane_amax = fold_abs8(lane_amax, y);
          if (j + 1 < CPL) {
#pragma unroll
            for (int q = 0; q < 12; ++q) pc[q] = pn[q];
          }
          continue;
        }
        const uint32_t s = block_scale_code(y, gsf);
        const float inv = inv_tab[s];
        if (j > 0) emit_encoded<CPL, Y, TILE>(o, j - 1, yp, invp, sp);
#pragma unroll
        for (int e = 0; e < 8; ++e) yp[e] = y[e];
        sp = s;
        invp = inv;
        if (j + 1 < CPL) {
#pragma unroll
          for (int q = 0; q < 12; ++q) pc[q] = pn[q];
        }
      }
      if (!AMAX) emit_encoded<CPL, Y, TILE>(o, CPL - 1, yp, invp, sp);
    }
    if (TILE) {
      // the unit's scale block is complete: copy its 128-byte lines out and zero them (each
      // thread clears exactly the words it copied); the next unit fills the other block, and
      // this one is filled again only after the next unit's barrier, when every thread has
      // finished copying it
      __syncthreads();
      uint8_t* blk = unit_sc + par * kUnitLdsBytes;
      if (v < head) {
        NVFP4_GLOBAL uint8_t* dst =
            global_ptr(a.scales) + (v / kUnitsPerTile) * kGroups * 512 + 16 * kS * (int)(v % kUnitsPerTile);
        for (int q = tid; q < kGroups * kS; q += kThreads) {
          uint4* src = reinterpret_cast<uint4*>(blk + (q / kS) * kGroupBytes + 16 * (q % kS));
          *reinterpret_cast<NVFP4_GLOBAL uint4*>(dst + (int64_t)(q / kS) * 512 + 16 * (q % kS)) = *src;
          *src = make_uint4(0, 0, 0, 0);
        }
        if (a.rstd_out && tid < 4 * kS) {
          // item tid of the unit: row tid mod kS of group tid / kS
          const int64_t rr =
              (v / kUnitsPerTile) * 128 + 32 * (tid / kS) + kS * (int)(v % kUnitsPerTile) + tid % kS;
          if (rr < m) global_ptr(a.rstd_out)[rr] = rstd_unit[4 * kS * par + tid];
        }
      } else {
        // rows r0 .. r0 + 7 (one 8-row block of a 32-row group): row r0 + w's 4 bytes of a
        // column group go to byte 16 (r mod 32) + 4 (r mod 128 / 32) of its 512-byte run
        const int64_t r0 = (head / kUnitsPerTile) * 128 + 8 * (v - head);
        NVFP4_GLOBAL uint8_t* dst = global_ptr(a.scales) + (r0 >> 7) * kGroups * 512 +
                                    16 * (int)(r0 & 31) + 4 * (int)((r0 >> 5) & 3);
        for (int q = tid; q < kGroups * 8; q += kThreads) {
          uint32_t* src = reinterpret_cast<uint32_t*>(blk + (q >> 3) * kGroupBytes + 4 * (q & 7));
          *reinterpret_cast<NVFP4_GLOBAL uint32_t*>(dst + (int64_t)(q >> 3) * 512 + 16 * (q & 7)) = *src;
          *src = 0;
        }
        if (a.rstd_out && tid < 8 && r0 + tid < m) global_ptr(a.rstd_out)[r0 + tid] = rstd_unit[4 * kS * par + tid];
      }
      par ^= 1;
    }
  }
  if (AMAX) workgroup_max_to(a.amax_out, lane_amax, amax_red, kStagedWaves);
}

// ---- the general kernel (any k % 512 == 0): parameters from global memory, two passes ----

// Row r of the general kernel; returns the lane's max |y| in the amax pass (else 0).
template <bool AMAX>
__device__ __forceinline__ float general_row(const RmsArgs& a, int64_t r, int lane, float gsf, const float* inv_tab) {
  const int64_t chunks = a.k >> 3;
  if (r >= a.padded) return 0.0f;
  if (r >= a.m) {
    if (!AMAX) zero_row_scales(a.scales, r, a.k, lane);
    return 0.0f;
  }
  const NVFP4_GLOBAL uint4* xr = global_ptr(a.x) + r * chunks;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t c = lane; c < chunks; c += kWave) {
    float f[8];
    unpack8(xr[c], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(f[e], f[e], acc[e]);
  }
  const float s = lane_sum_butterfly(((acc[0] + acc[1]) + (acc[2] + acc[3])) +
                                     ((acc[4] + acc[5]) + (acc[6] + acc[7])));
  const float rstd = 1.0f / sqrtf(s / (float)a.k + a.eps);
  if (!AMAX && lane == 0 && a.rstd_out) global_ptr(a.rstd_out)[r] = rstd;
  const int64_t t = global_ptr(a.frame_idx)[r];
  if (t < 0 || t >= a.num_frames) {
    if (!AMAX) zero_row(a, r, lane, true);
    return 0.0f;
  }
  const RowOut o = row_out(a, r, lane);
  float lane_amax = 0.0f;
  for (int j = 0; j < (int)(chunks >> 6); ++j) {
    const int64_t c = lane + (int64_t)kWave * j;
    float x8[8], w8[8], o8[8], h8[8], y[8];
    unpack8(xr[c], x8);
    unpack8(*reinterpret_cast<const NVFP4_GLOBAL uint4*>(global_ptr(a.w) + 8 * c), w8);
    load_frame_chunk(a, t, c, o8, h8);
    modulate8(x8, w8, o8, h8, rstd, y);
    if (AMAX) lane_amax = fold_abs8(lane_amax, y);
    else store_chunk(o, j, y, gsf, inv_tab, false, 0);
  }
  return lane_amax;
}

template <bool AMAX>
__global__ __launch_bounds__(256) void rms_adaln_general(RmsArgs a) {
  __shared__ float inv_tab[128];
  __shared__ float amax_red[4];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float gsf = call_global_scale(a.global_amax, a.amax_dev);
  fill_inverse_table(inv_tab, gsf, tid);
  __syncthreads();
  const float lane_amax = general_row<AMAX>(a, (int64_t)blockIdx.x * 4 + wave, lane, gsf, inv_tab);
  if (AMAX) workgroup_max_to(a.amax_out, lane_amax, amax_red, 4);
}

// Two 32-row units' scale blocks are staged in LDS beside the parameters (TILE), which fits
// for every k of the staged kernel.
// Dynamic LDS cap: the 160 KiB of a CU less a little for the kernels' static arrays.
constexpr size_t kLdsLimit = 160 * 1024 - 256;
inline size_t staged_lds_bytes(int64_t k, bool tile) {
  const int cpl = (int)(k / 512);
  return 512 + 12 * (size_t)k +
         (tile ? 2 * (size_t)(k / 64) * lds_group_bytes(cpl) + 2 * 4 * unit_rows_per_group(cpl) * sizeof(float) : 0);
}

template <int CPL>
hipError_t launch_staged(const RmsArgs& a, bool amax_pass, const DeviceInfo& dev, hipStream_t stream) {
  // A tensor of fewer 128-row tiles than CUs leaves CUs idle; it runs in smaller units
  // instead (64 rows down to 8, one per wavefront), without the LDS scale tile, when that
  // takes the rows of the busiest CU to 3/4 of what 128-row tiles give it or fewer
  // (measured: a row costs up to ~20 % more without the tile).  The unit is the one with
  // the fewest rows of x on the busiest CU, the larger one on equal counts; padding rows
  // (only scale bytes to zero) are not counted.
  RmsArgs s = a;
  s.unit_shift = 7;
  if ((a.padded >> 7) < dev.cu_count) {
    auto busiest = [&](int u) {
      const int64_t units = (a.m + (1 << u) - 1) >> u;
      const int64_t rows = ((units + dev.cu_count - 1) / dev.cu_count) << u;
      return rows < a.m ? rows : a.m;
    };
    int best = 7;
    for (int u = 6; u >= 3; --u)
      if (busiest(u) < busiest(best)) best = u;
    if (4 * busiest(best) <= 3 * busiest(7)) s.unit_shift = best;
  }
  // A full-size tensor whose units of 4S rows leave a last round that keeps some CUs busy
  // while others idle runs its full rounds (down to a whole tile) in those units and the
  // tiles after them in 8-row units over every CU, when that takes at least S rows off the
  // busiest CU.  An 8-row unit ends with a barrier after one row per wavefront, so a tail
  // that saves less costs more than it gains (measured on random input with four frames:
  // 63,240 x 7168, 8 of 64 rows saved, 227 -> 235 us; 40,000 x 7168, 32 saved,
  // 161 -> 151 us).
  constexpr int kS = unit_rows_per_group(CPL), kPerTile = 32 / kS;
  s.head_units = (a.padded >> 7) * kPerTile;
  if (s.unit_shift == 7) {
    const int64_t cus = dev.cu_count, rounds = s.head_units / cus;
    const int64_t head = rounds * cus / kPerTile * kPerTile;
    const int64_t tail = (a.padded - head * 4 * kS) / 8;
    if (rounds > 0 && head < s.head_units && 8 * ((tail + cus - 1) / cus) + kS <= 4 * kS) s.head_units = head;
  }
  const bool tile = !amax_pass && s.unit_shift == 7 && staged_lds_bytes(a.k, true) <= kLdsLimit;
  const size_t lds = staged_lds_bytes(a.k, tile);
  const int64_t units =
      s.unit_shift == 7 ? s.head_units + (a.padded - s.head_units * 4 * kS) / 8 : a.padded >> s.unit_shift;
  const int64_t grid = units < dev.cu_count ? units : dev.cu_count;
  const dim3 g((uint32_t)grid), b(kStagedWaves * kWave);
  if (amax_pass) {
    hipLaunchKernelGGL((rms_adaln_staged<CPL, false, false, true>), g, b, lds, stream, s, a.frame_idx);
  } else if (tile) {
    if (a.y_out) hipLaunchKernelGGL((rms_adaln_staged<CPL, true, true, false>), g, b, lds, stream, s, a.frame_idx);
    else hipLaunchKernelGGL((rms_adaln_staged<CPL, false, true, false>), g, b, lds, stream, s, a.frame_idx);
  } else {
    if (a.y_out) hipLaunchKernelGGL((rms_adaln_staged<CPL, true, false, false>), g, b, lds, stream, s, a.frame_idx);
    else hipLaunchKernelGGL((rms_adaln_staged<CPL, false, false, false>), g, b, lds, stream, s, a.frame_idx);
  }
  return hipGetLastError();
}

template <int CPL, bool Y, bool TILE, bool AMAX>
hipError_t allow_lds_one() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&rms_adaln_staged<CPL, Y, TILE, AMAX>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
}

template <int CPL>
hipError_t allow_lds() {
  hipError_t e = allow_lds_one<CPL, false, false, false>();
  if (e == hipSuccess) e = allow_lds_one<CPL, true, false, false>();
  if (e == hipSuccess) e = allow_lds_one<CPL, false, true, false>();
  if (e == hipSuccess) e = allow_lds_one<CPL, true, true, false>();
  if (e == hipSuccess) e = allow_lds_one<CPL, false, false, true>();
  return e;
}

// One launch of the producer (amax_pass: the amax pass of a per-call scale instead).
hipError_t launch_rms(const RmsArgs& a, bool amax_pass, const DeviceInfo& dev, hipStream_t stream) {
  switch (a.k / 512) {
    case 1: return launch_staged<1>(a, amax_pass, dev, stream);
    case 2: return launch_staged<2>(a, amax_pass, dev, stream);
    case 3: return launch_staged<3>(a, amax_pass, dev, stream);
    case 4: return launch_staged<4>(a, amax_pass, dev, stream);
    case 5: return launch_staged<5>(a, amax_pass, dev, stream);
    case 6: return launch_staged<6>(a, amax_pass, dev, stream);
    case 7: return launch_staged<7>(a, amax_pass, dev, stream);
    case 8: return launch_staged<8>(a, amax_pass, dev, stream);
    case 9: return launch_staged<9>(a, amax_pass, dev, stream);
    case 10: return launch_staged<10>(a, amax_pass, dev, stream);
    case 11: return launch_staged<11>(a, amax_pass, dev, stream);
    case 12: return launch_staged<12>(a, amax_pass, dev, stream);
    case 13: return launch_staged<13>(a, amax_pass, dev, stream);
    case 14: return launch_staged<14>(a, amax_pass, dev, stream);
    case 15: return launch_staged<15>(a, amax_pass, dev, stream);
    case 16: return launch_staged<16>(a, amax_pass, dev, stream);
    default: break;
  }
  const int64_t blocks = (a.padded + 3) / 4;
  if (amax_pass) hipLaunchKernelGGL(rms_adaln_general<true>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(rms_adaln_general<false>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Device scratch of the allocation-free per-call entry point: element 0 is the word its amax
// pass folds max |y| into (zeroed by a fill kernel first), which the producer then reads.
// Every call needs that one word, whatever its m and k, so no input size can exceed it.  Each
// device holds its own copy until the process ends; calls that overlap on one device race on
// it.  Host code never uses the symbol itself (on the host it is only a stand-in): it uses
// the device address looked up once per device below.
constexpr int kScratchFloats = 64;   // 256 bytes
static __device__ __align__(256) float scratch[kScratchFloats];

static float* g_scratch_dev[kMaxDeviceSlots] = {};   // per device: the address of scratch

hipError_t prepare_rms_adaln(int device) {
  if (device < 0 || device >= kMaxDeviceSlots) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_dev[device] = static_cast<float*>(ptr);
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

float* rms_adaln_scratch(int device) {
  return (device >= 0 && device < kMaxDeviceSlots) ? g_scratch_dev[device] : nullptr;
}

hipError_t launch_rms_adaln(const RmsLaunch& p, const DeviceInfo& dev, hipStream_t stream) {
  RmsArgs a;
  a.x = static_cast<const uint4*>(p.x);
  a.w = static_cast<const uint16_t*>(p.weight);
  a.shift = static_cast<const uint16_t*>(p.shift);
  a.scale = static_cast<const uint16_t*>(p.scale);
  a.frame_stride = p.frame_stride;
  a.num_frames = p.num_frames;
  a.frame_idx = p.frame_idx;
  a.eps = p.eps;
  a.m = p.m;
  a.k = p.k;
  a.padded = (p.m + 127) / 128 * 128;
  a.global_amax = p.global_amax;
  a.codes = static_cast<uint32_t*>(p.codes);
  a.scales = static_cast<uint8_t*>(p.scales);
  a.rstd_out = p.rstd_out;
  a.y_out = static_cast<uint4*>(p.y_out);
  a.status = p.status_word;
  a.amax_dev = p.amax_dev;
  a.amax_out = nullptr;
  a.unit_shift = 7;
  if (p.amax_dev) {
    // per-call scale: zero the amax, fold max |y| into it, then quantize with it
    RmsArgs pass = a;
    pass.amax_dev = nullptr;
    pass.amax_out = p.amax_dev;
    hipError_t e = launch_zero_amax(pass.amax_out, stream);
    if (e == hipSuccess) e = launch_rms(pass, true, dev, stream);
    if (e != hipSuccess) return e;
  }
  return launch_rms(a, false, dev, stream);
}

}  // namespace nvfp4act
