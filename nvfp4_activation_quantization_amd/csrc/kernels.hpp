// kernels.hpp -- host-side launchers of the NVFP4 producer kernels (internal to
// libnvfp4act.so; the public interface is include/nvfp4act.h).  Arguments have been
// validated by the caller; each launcher only sizes the grid and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4act {

struct DeviceInfo {
  int cu_count;
};

// amax_dev: null for a static global_amax, else the device float an amax pass wrote (the
// global scale is then computed on the device from it).
hipError_t launch_quantize(const void* x, int64_t m, int64_t k, float global_amax, const float* amax_dev,
                           void* codes, void* scales, hipStream_t stream);

// *amax = 0, then max |x| over the m x k tensor folded into it.
hipError_t launch_zero_amax(float* amax, hipStream_t stream);
hipError_t launch_amax_x(const void* x, int64_t m, int64_t k, float* amax, const DeviceInfo& dev,
                         hipStream_t stream);

// The arguments of one rms_adaln_nvfp4 call (see include/nvfp4act.h).  amax_dev: null for
// the static global_amax; else the device float that receives max |y| of this call (an
// amax pass runs first and the quantizer takes its global scale from it).
struct RmsLaunch {
  const void* x;
  const void* weight;
  const void* shift;
  const void* scale;
  int64_t frame_stride, num_frames;
  const int32_t* frame_idx;
  float eps;
  int64_t m, k;
  float global_amax;
  float* amax_dev;
  void* codes;
  void* scales;
  float* rstd_out;
  void* y_out;
  uint32_t* status_word;
};

hipError_t launch_rms_adaln(const RmsLaunch& p, const DeviceInfo& dev, hipStream_t stream);

// The arguments of one SwiGLU call.  Value-first or two-pointer form (paired == false):
// row r of the values at up + r*ld and of the gates at gate + r*ld (bf16 elements);
// bias_up / bias_gate: null, or the f-entry bf16 biases of the value and gate columns.
// Paired form: row r of the projection at up + r*ld, the value of output column j at 2j and
// its gate at 2j + 1; gate and bias_gate unused; bias_up: null or one 2f-entry paired bias
// row.  amax_dev: as for RmsLaunch (null: static global_amax; else the per-call amax of y).
struct SwigluLaunch {
  const void* up;
  const void* gate;
  const void* bias_up;
  const void* bias_gate;
  bool paired;
  int64_t ld, m, f;
  float global_amax;
  float* amax_dev;
  void* codes;
  void* scales;
  void* y_out;
};

hipError_t launch_swiglu(const SwigluLaunch& p, const DeviceInfo& dev, hipStream_t stream);

// The arguments of one residual_rms_nvfp4 or residual_rms_adaln_nvfp4 call (see
// include/nvfp4act.h).  o null: no branch (h is only read); bias null: no bias.  mod: the
// adaLN form (gate rows multiply the branch; weight, shift, mod_scale and the frame index
// replace gamma; scale unused); strides in elements.  amax_dev: as for RmsLaunch.
constexpr int64_t kMaxResidualK = 8192;   // the row is held in registers

struct ResidualLaunch {
  float* h;
  const void* o;
  const void* bias;
  const float* scale;
  const float* gamma;
  float eps;
  int64_t m, k;
  float global_amax;
  float* amax_dev;
  void* codes;
  void* scales;
  float* rstd_out;
  void* y_out;
  bool mod;
  const void* gate;
  int64_t gate_stride;
  const void* weight;
  const void* shift;
  const void* mod_scale;
  int64_t frame_stride, num_frames;
  const int32_t* frame_idx;
  uint32_t* status_word;
};

hipError_t launch_residual_rms(const ResidualLaunch& p, hipStream_t stream);

// The arguments of one rms_silu_nvfp4 call (see include/nvfp4act.h): x [rows, c] fp16
// channels-last, gamma [c] fp16; codes [rows, c/2], scales [rows, c/16] (plain order).
struct RmsSiluLaunch {
  const void* x;
  const void* gamma;
  float eps;
  int64_t rows, c;
  float global_amax;
  float* amax_dev;
  void* codes;
  void* scales;
  float* rstd_out;
  void* y_out;
};

hipError_t launch_rms_silu(const RmsSiluLaunch& p, const DeviceInfo& dev, hipStream_t stream);

// The arguments of one ln_adaln_fp8 call (see include/nvfp4act.h): x [m, k] fp16, scale and
// shift [k] fp32; codes [m, k] E4M3 bytes.  scale_dev: null for the static act_scale; else
// the device float that receives this call's scale max|y| / 448 (an amax pass runs first).
struct LnFp8Launch {
  const void* x;
  const float* scale;
  const float* shift;
  float eps;
  int64_t m, k;
  float act_scale;
  float* scale_dev;
  void* codes;
  float* mean_out;
  float* rstd_out;
  float* y_out;
};

constexpr int64_t kMaxLnK = 8192;   // the row is held in registers

hipError_t launch_ln_fp8(const LnFp8Launch& p, const DeviceInfo& dev, hipStream_t stream);

// Per-device, once: allow the LDS sizes the kernels use.
// Devices the library keeps per-device state for (device ordinals 0 .. kMaxDeviceSlots - 1).
constexpr int kMaxDeviceSlots = 64;
// Once per device, with that device current: kernel attributes, and the device address of the
// scratch word of rms_adaln_nvfp4_dynamic_noalloc.
hipError_t prepare_rms_adaln(int device);
// That address (null before prepare_rms_adaln ran for the device).
float* rms_adaln_scratch(int device);
hipError_t prepare_swiglu();
hipError_t prepare_residual_rms();
hipError_t prepare_rms_silu();
hipError_t prepare_ln_fp8();


}  // namespace nvfp4act
