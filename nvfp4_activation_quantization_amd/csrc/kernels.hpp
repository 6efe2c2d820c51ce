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

hipError_t launch_quantize(const void* x, int64_t m, int64_t k, float global_amax, void* codes,
                           void* scales, hipStream_t stream);

hipError_t launch_rms_adaln(const void* x, const void* weight, const void* shift, const void* scale,
                            int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                            float eps, int64_t m, int64_t k, float global_amax, void* codes,
                            void* scales, float* rstd_out, void* y_out, uint32_t* status_word,
                            const DeviceInfo& dev, hipStream_t stream);

hipError_t launch_swiglu(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f,
                         float global_amax, void* codes, void* scales, void* y_out,
                         const DeviceInfo& dev, hipStream_t stream);

// Per-device, once: allow the LDS sizes the kernels use.
hipError_t prepare_rms_adaln();
hipError_t prepare_swiglu();

// Build the SiLU table of the current device and wait for it; *ambiguous receives the
// number of entries whose rounding fp64 could not decide (0 expected).
hipError_t build_silu_table(unsigned int* ambiguous);

}  // namespace nvfp4act
