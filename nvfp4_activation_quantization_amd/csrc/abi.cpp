// abi.cpp -- the C ABI of libnvfp4act.so (declared in include/nvfp4act.h): host-side
// argument checks, per-device set-up and status reporting.  No compute happens here; each
// entry point validates, then enqueues its kernel on the caller's stream.
//
// The status-code convention (int return, nonzero on failure, stream last) follows the
// C-ABI launchers of the FastVideo branch compare (launch_quant_probe / launch_gemm_swiglu,
// with h3_swiglu_gemm_binding.py raising on a nonzero code).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "nvfp4act.h"
#include "kernels.hpp"

namespace {

using nvfp4act::DeviceInfo;

constexpr int kMaxDevices = nvfp4act::kMaxDeviceSlots;

struct DeviceState {
  bool probed = false;
  bool usable = false;
  DeviceInfo info{0};
};

std::mutex g_mutex;
DeviceState g_dev[kMaxDevices];
thread_local int t_last_hip_error = 0;

int fail_hip(hipError_t e) {
  t_last_hip_error = (int)e;
  return NVFP4ACT_ERR_LAUNCH;
}

// Probe the current device once: gfx950, CU count, LDS attributes of the kernels.
int current_device(const DeviceInfo** info, int* device_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return NVFP4ACT_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  DeviceState& st = g_dev[dev];
  if (!st.probed) {
    st.probed = true;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return NVFP4ACT_ERR_DEVICE;
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return NVFP4ACT_ERR_DEVICE;
    st.info.cu_count = prop.multiProcessorCount;
    hipError_t e = nvfp4act::prepare_rms_adaln(dev);
    if (e == hipSuccess) e = nvfp4act::prepare_swiglu();
    if (e == hipSuccess) e = nvfp4act::prepare_residual_rms();
    if (e == hipSuccess) e = nvfp4act::prepare_rms_silu();
    if (e == hipSuccess) e = nvfp4act::prepare_ln_fp8();
    if (e != hipSuccess) {
      st.probed = false;
      return fail_hip(e);
    }
    st.usable = true;
  }
  if (!st.usable) return NVFP4ACT_ERR_DEVICE;
  *info = &st.info;
  if (device_out) *device_out = dev;
  return NVFP4ACT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_amax(float global_amax) {
  if (!std::isfinite(global_amax) || !(global_amax > 0.0f)) return NVFP4ACT_ERR_VALUE;
  if (!std::isfinite(2688.0f / global_amax)) return NVFP4ACT_ERR_VALUE;
  return NVFP4ACT_OK;
}

}  // namespace

extern "C" {

int64_t nvfp4act_padded_rows(int64_t m) { return m <= 0 ? 0 : (m + 127) / 128 * 128; }

int64_t nvfp4act_codes_bytes(int64_t m, int64_t k) { return m * k / 2; }

int64_t nvfp4act_scales_bytes(int64_t m, int64_t k) { return nvfp4act_padded_rows(m) * k / 16; }

float nvfp4act_global_scale(float global_amax) { return 2688.0f / global_amax; }

const char* nvfp4act_status_string(int status) {
  switch (status) {
    case NVFP4ACT_OK: return "ok";
    case NVFP4ACT_ERR_NULL: return "a required pointer is NULL";
    case NVFP4ACT_ERR_SHAPE: return "bad shape (m < 0, or k / f / ld / num_frames / frame_stride invalid)";
    case NVFP4ACT_ERR_ALIGN: return "pointer, row stride or frame stride not 16-byte aligned";
    case NVFP4ACT_ERR_VALUE: return "global_amax or eps out of range";
    case NVFP4ACT_ERR_DEVICE: return "no usable gfx950 device is current";
    case NVFP4ACT_ERR_LAUNCH: return "a HIP call failed (see nvfp4act_last_hip_error)";
    case NVFP4ACT_ERR_TABLE: return "the SiLU table could not be built exactly (no longer returned: the tables are fixed when the library is built)";
    default: return "unknown status";
  }
}

int nvfp4act_last_hip_error(void) { return t_last_hip_error; }

// The build passes the sha256 of the sources it compiled (csrc/* and include/nvfp4act.h).
#ifndef NVFP4ACT_SOURCE_DIGEST
#define NVFP4ACT_SOURCE_DIGEST "unknown"
#endif
const char* nvfp4act_source_digest(void) { return NVFP4ACT_SOURCE_DIGEST; }

int nvfp4act_init(void) {
  const DeviceInfo* info = nullptr;
  return current_device(&info, nullptr);
}

}  // extern "C"

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The checks and launches shared by the static (amax_dev == nullptr) and per-call
// (amax_dev: the device float receiving the call's amax) forms of each entry point.
int quantize_call(const void* x, int64_t m, int64_t k, float global_amax, float* amax_dev, void* codes,
                  void* scales, void* stream) {
  if (m < 0 || k <= 0 || k % 64 != 0) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!x || !codes || !scales) return NVFP4ACT_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return NVFP4ACT_ERR_ALIGN;
  if (!amax_dev) {
    int st = check_amax(global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (amax_dev) {
    e = nvfp4act::launch_zero_amax(amax_dev, s);
    if (e == hipSuccess) e = nvfp4act::launch_amax_x(x, m, k, amax_dev, *info, s);
  }
  if (e == hipSuccess) e = nvfp4act::launch_quantize(x, m, k, global_amax, amax_dev, codes, scales, s);
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

int rms_adaln_call(const void* x, const void* weight, const void* shift, const void* scale, int64_t frame_stride,
                   int64_t num_frames, const int32_t* frame_idx, float eps, int64_t m, int64_t k,
                   float global_amax, float* amax_dev, void* codes, void* scales, float* rstd_out, void* y_out,
                   uint32_t* status_word, void* stream) {
  if (m < 0 || k <= 0 || k % 512 != 0 || num_frames < 1 || frame_stride < k) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!x || !weight || !shift || !scale || !frame_idx || !codes || !scales) return NVFP4ACT_ERR_NULL;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(shift) || !aligned16(scale) ||
      !aligned16(codes) || !aligned16(scales) || (frame_stride * 2) % 16 != 0 ||
      (rstd_out && !aligned4(rstd_out)) || (y_out && !aligned16(y_out)) || !aligned4(frame_idx) ||
      (status_word && !aligned4(status_word)))
    return NVFP4ACT_ERR_ALIGN;
  if (!amax_dev) {
    int st = check_amax(global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  if (!std::isfinite(eps) || eps < 0.0f) return NVFP4ACT_ERR_VALUE;
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  nvfp4act::RmsLaunch p;
  p.x = x;
  p.weight = weight;
  p.shift = shift;
  p.scale = scale;
  p.frame_stride = frame_stride;
  p.num_frames = num_frames;
  p.frame_idx = frame_idx;
  p.eps = eps;
  p.m = m;
  p.k = k;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.rstd_out = rstd_out;
  p.y_out = y_out;
  p.status_word = status_word;
  hipError_t e = nvfp4act::launch_rms_adaln(p, *info, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

int swiglu_launch(const nvfp4act::SwigluLaunch& p, void* stream) {
  if (!p.amax_dev) {
    int st = check_amax(p.global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  hipError_t e = nvfp4act::launch_swiglu(p, *info, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

int swiglu_call(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f, float global_amax,
                float* amax_dev, void* codes, void* scales, void* y_out, void* stream) {
  if (m < 0 || f <= 0 || f % 64 != 0 || ld < f) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!up || !gate || !codes || !scales) return NVFP4ACT_ERR_NULL;
  if (!aligned16(up) || !aligned16(gate) || !aligned16(codes) || !aligned16(scales) ||
      (ld * 2) % 16 != 0 || (y_out && !aligned16(y_out)))
    return NVFP4ACT_ERR_ALIGN;
  nvfp4act::SwigluLaunch p{};
  p.up = up;
  p.gate = gate;
  p.paired = false;
  p.ld = ld;
  p.m = m;
  p.f = f;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.y_out = y_out;
  return swiglu_launch(p, stream);
}

bool packed_shape_ok(int interleaved, int64_t ld, int64_t m, int64_t f) {
  return m >= 0 && f > 0 && f % 64 == 0 && ld >= 2 * f && (interleaved == 0 || interleaved == 1);
}

int swiglu_packed_call(const void* proj, const void* bias, int interleaved, int64_t ld, int64_t m, int64_t f,
                       float global_amax, float* amax_dev, void* codes, void* scales, void* y_out, void* stream) {
  if (!packed_shape_ok(interleaved, ld, m, f)) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!proj || !codes || !scales) return NVFP4ACT_ERR_NULL;
  if (!aligned16(proj) || !aligned16(codes) || !aligned16(scales) || (ld * 2) % 16 != 0 ||
      (bias && !aligned16(bias)) || (y_out && !aligned16(y_out)))
    return NVFP4ACT_ERR_ALIGN;
  const uint16_t* o = static_cast<const uint16_t*>(proj);
  const uint16_t* b = static_cast<const uint16_t*>(bias);
  nvfp4act::SwigluLaunch p{};
  p.up = proj;
  p.paired = interleaved == 1;
  p.gate = p.paired ? nullptr : o + f;                 // value-first: gate half f columns on
  p.bias_up = bias;
  p.bias_gate = (b && !p.paired) ? b + f : nullptr;
  p.ld = ld;
  p.m = m;
  p.f = f;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.y_out = y_out;
  return swiglu_launch(p, stream);
}

int residual_rms_call(float* h, const void* o, const void* bias, const float* scale, const float* gamma, float eps,
                      int64_t m, int64_t k, float global_amax, float* amax_dev, void* codes, void* scales,
                      float* rstd_out, void* y_out, void* stream) {
  if (m < 0 || k <= 0 || k % 512 != 0 || k > nvfp4act::kMaxResidualK) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!h || !gamma || !codes || !scales || (o && !scale)) return NVFP4ACT_ERR_NULL;
  if (!aligned16(h) || !aligned16(gamma) || !aligned16(codes) || !aligned16(scales) || (o && !aligned16(o)) ||
      (o && !aligned16(scale)) || (o && bias && !aligned16(bias)) || (y_out && !aligned16(y_out)) ||
      (rstd_out && !aligned4(rstd_out)))
    return NVFP4ACT_ERR_ALIGN;
  if (!std::isfinite(eps) || eps < 0.0f) return NVFP4ACT_ERR_VALUE;
  if (!amax_dev) {
    int st = check_amax(global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  nvfp4act::ResidualLaunch p{};
  p.h = h;
  p.o = o;
  p.bias = o ? bias : nullptr;
  p.scale = o ? scale : nullptr;
  p.gamma = gamma;
  p.eps = eps;
  p.m = m;
  p.k = k;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.rstd_out = rstd_out;
  p.y_out = y_out;
  hipError_t e = nvfp4act::launch_residual_rms(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

// The adaLN form: the gate table multiplies the branch; RMSNorm weight and the next block's
// (shift, scale) rows replace gamma.
struct FoldTables {
  const void* gate;
  int64_t gate_stride;
  const void* weight;
  const void* shift;
  const void* scale;
  int64_t frame_stride, num_frames;
  const int32_t* frame_idx;
  uint32_t* status_word;
};

int residual_adaln_shape(int64_t m, int64_t k, const void* o, const FoldTables& f) {
  if (m < 0 || k <= 0 || k % 512 != 0 || k > nvfp4act::kMaxResidualK || f.num_frames < 1 || f.frame_stride < k ||
      (o && f.gate_stride < k))
    return NVFP4ACT_ERR_SHAPE;
  return NVFP4ACT_OK;
}

int residual_adaln_call(float* h, const void* o, const void* bias, const FoldTables& f, float eps, int64_t m,
                        int64_t k, float global_amax, float* amax_dev, void* codes, void* scales, float* rstd_out,
                        void* y_out, void* stream) {
  int st = residual_adaln_shape(m, k, o, f);
  if (st != NVFP4ACT_OK) return st;
  if (m == 0) return NVFP4ACT_OK;
  if (!h || !f.weight || !f.shift || !f.scale || !f.frame_idx || !codes || !scales || (o && !f.gate))
    return NVFP4ACT_ERR_NULL;
  if (!aligned16(h) || !aligned16(f.weight) || !aligned16(f.shift) || !aligned16(f.scale) || !aligned16(codes) ||
      !aligned16(scales) || (o && !aligned16(o)) || (o && !aligned16(f.gate)) || (o && bias && !aligned16(bias)) ||
      (y_out && !aligned16(y_out)) || (rstd_out && !aligned4(rstd_out)) || !aligned4(f.frame_idx) ||
      (f.status_word && !aligned4(f.status_word)) || (f.frame_stride * 2) % 16 != 0 ||
      (o && (f.gate_stride * 2) % 16 != 0))
    return NVFP4ACT_ERR_ALIGN;
  if (!std::isfinite(eps) || eps < 0.0f) return NVFP4ACT_ERR_VALUE;
  if (!amax_dev) {
    st = check_amax(global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  const DeviceInfo* info = nullptr;
  st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  nvfp4act::ResidualLaunch p{};
  p.h = h;
  p.o = o;
  p.bias = o ? bias : nullptr;
  p.eps = eps;
  p.m = m;
  p.k = k;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.rstd_out = rstd_out;
  p.y_out = y_out;
  p.mod = true;
  p.gate = o ? f.gate : nullptr;
  p.gate_stride = f.gate_stride;
  p.weight = f.weight;
  p.shift = f.shift;
  p.mod_scale = f.scale;
  p.frame_stride = f.frame_stride;
  p.num_frames = f.num_frames;
  p.frame_idx = f.frame_idx;
  p.status_word = f.status_word;
  hipError_t e = nvfp4act::launch_residual_rms(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

int rms_silu_call(const void* x, const void* gamma, float eps, int64_t rows, int64_t c, float global_amax,
                  float* amax_dev, void* codes, void* scales, float* rstd_out, void* y_out, void* stream) {
  if (rows < 0 || c < 16 || c > 512 || c % 16 != 0) return NVFP4ACT_ERR_SHAPE;
  if (rows == 0) return NVFP4ACT_OK;
  if (!x || !gamma || !codes || !scales) return NVFP4ACT_ERR_NULL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned4(codes) || (y_out && !aligned16(y_out)) ||
      (rstd_out && !aligned4(rstd_out)))
    return NVFP4ACT_ERR_ALIGN;
  if (!std::isfinite(eps) || eps < 0.0f) return NVFP4ACT_ERR_VALUE;
  if (!amax_dev) {
    int st = check_amax(global_amax);
    if (st != NVFP4ACT_OK) return st;
  }
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  nvfp4act::RmsSiluLaunch p{};
  p.x = x;
  p.gamma = gamma;
  p.eps = eps;
  p.rows = rows;
  p.c = c;
  p.global_amax = global_amax;
  p.amax_dev = amax_dev;
  p.codes = codes;
  p.scales = scales;
  p.rstd_out = rstd_out;
  p.y_out = y_out;
  hipError_t e = nvfp4act::launch_rms_silu(p, *info, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

bool ln_shape_ok(int64_t m, int64_t k) { return m >= 0 && k >= 512 && k % 512 == 0 && k <= nvfp4act::kMaxLnK; }

int ln_fp8_call(const void* x, const float* scale, const float* shift, float eps, int64_t m, int64_t k,
                float act_scale, float* scale_dev, void* codes, float* mean_out, float* rstd_out, float* y_out,
                void* stream) {
  if (!ln_shape_ok(m, k)) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  if (!x || !scale || !shift || !codes) return NVFP4ACT_ERR_NULL;
  if (!aligned16(x) || !aligned16(scale) || !aligned16(shift) || (reinterpret_cast<uintptr_t>(codes) & 7u) ||
      (y_out && !aligned16(y_out)) || (mean_out && !aligned4(mean_out)) || (rstd_out && !aligned4(rstd_out)))
    return NVFP4ACT_ERR_ALIGN;
  if (!std::isfinite(eps) || eps < 0.0f) return NVFP4ACT_ERR_VALUE;
  if (!scale_dev && (!std::isfinite(act_scale) || !(act_scale > 0.0f) || !std::isfinite(1.0f / act_scale)))
    return NVFP4ACT_ERR_VALUE;
  const DeviceInfo* info = nullptr;
  int st = current_device(&info, nullptr);
  if (st != NVFP4ACT_OK) return st;
  nvfp4act::LnFp8Launch p{};
  p.x = x;
  p.scale = scale;
  p.shift = shift;
  p.eps = eps;
  p.m = m;
  p.k = k;
  p.act_scale = act_scale;
  p.scale_dev = scale_dev;
  p.codes = codes;
  p.mean_out = mean_out;
  p.rstd_out = rstd_out;
  p.y_out = y_out;
  hipError_t e = nvfp4act::launch_ln_fp8(p, *info, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4ACT_OK : fail_hip(e);
}

// The per-call forms need the amax destination: one 4-byte aligned float (m == 0 aside).
int check_amax_out(int64_t m, const float* amax_out) {
  if (m == 0) return NVFP4ACT_OK;
  if (!amax_out) return NVFP4ACT_ERR_NULL;
  if (!aligned4(amax_out)) return NVFP4ACT_ERR_ALIGN;
  return NVFP4ACT_OK;
}

}  // namespace

extern "C" {

int nvfp4_quantize(const void* x, int64_t m, int64_t k, float global_amax, void* codes, void* scales,
                   void* stream) {
  return quantize_call(x, m, k, global_amax, nullptr, codes, scales, stream);
}

int nvfp4_quantize_dynamic(const void* x, int64_t m, int64_t k, float* amax_out, void* codes, void* scales,
                           void* stream) {
  if (m < 0 || k <= 0 || k % 64 != 0) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return quantize_call(x, m, k, 0.0f, amax_out, codes, scales, stream);
}

int rms_adaln_nvfp4(const void* x, const void* weight, const void* shift, const void* scale,
                    int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx, float eps,
                    int64_t m, int64_t k, float global_amax, void* codes, void* scales, float* rstd_out,
                    void* y_out, uint32_t* status_word, void* stream) {
  return rms_adaln_call(x, weight, shift, scale, frame_stride, num_frames, frame_idx, eps, m, k, global_amax,
                        nullptr, codes, scales, rstd_out, y_out, status_word, stream);
}

int rms_adaln_nvfp4_dynamic(const void* x, const void* weight, const void* shift, const void* scale,
                            int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx, float eps,
                            int64_t m, int64_t k, float* amax_out, void* codes, void* scales, float* rstd_out,
                            void* y_out, uint32_t* status_word, void* stream) {
  if (m < 0 || k <= 0 || k % 512 != 0 || num_frames < 1 || frame_stride < k) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return rms_adaln_call(x, weight, shift, scale, frame_stride, num_frames, frame_idx, eps, m, k, 0.0f, amax_out,
                        codes, scales, rstd_out, y_out, status_word, stream);
}

int rms_adaln_nvfp4_dynamic_noalloc(const void* x, const void* weight, const void* shift, const void* scale,
                                    int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx, float eps,
                                    int64_t m, int64_t k, void* codes, void* scales, float* rstd_out, void* y_out,
                                    uint32_t* status_word, void* stream) {
  if (m < 0 || k <= 0 || k % 512 != 0 || num_frames < 1 || frame_stride < k) return NVFP4ACT_ERR_SHAPE;
  if (m == 0) return NVFP4ACT_OK;
  const DeviceInfo* info = nullptr;
  int dev = -1;
  int st = current_device(&info, &dev);
  if (st != NVFP4ACT_OK) return st;
  float* amax_dev = nvfp4act::rms_adaln_scratch(dev);   // one word of the library's device scratch
  if (!amax_dev) return NVFP4ACT_ERR_DEVICE;
  return rms_adaln_call(x, weight, shift, scale, frame_stride, num_frames, frame_idx, eps, m, k, 0.0f, amax_dev,
                        codes, scales, rstd_out, y_out, status_word, stream);
}

int swiglu_nvfp4(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f, float global_amax,
                 void* codes, void* scales, void* y_out, void* stream) {
  return swiglu_call(up, gate, ld, m, f, global_amax, nullptr, codes, scales, y_out, stream);
}

int swiglu_nvfp4_dynamic(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f, float* amax_out,
                         void* codes, void* scales, void* y_out, void* stream) {
  if (m < 0 || f <= 0 || f % 64 != 0 || ld < f) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return swiglu_call(up, gate, ld, m, f, 0.0f, amax_out, codes, scales, y_out, stream);
}

int swiglu_packed_nvfp4(const void* proj, const void* bias, int interleaved, int64_t ld, int64_t m, int64_t f,
                        float global_amax, void* codes, void* scales, void* y_out, void* stream) {
  return swiglu_packed_call(proj, bias, interleaved, ld, m, f, global_amax, nullptr, codes, scales, y_out, stream);
}

int swiglu_packed_nvfp4_dynamic(const void* proj, const void* bias, int interleaved, int64_t ld, int64_t m,
                                int64_t f, float* amax_out, void* codes, void* scales, void* y_out, void* stream) {
  if (!packed_shape_ok(interleaved, ld, m, f)) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return swiglu_packed_call(proj, bias, interleaved, ld, m, f, 0.0f, amax_out, codes, scales, y_out, stream);
}

int residual_rms_nvfp4(float* h, const void* o, const void* bias, const float* scale, const float* gamma, float eps,
                      int64_t m, int64_t k, float global_amax, void* codes, void* scales, float* rstd_out,
                      void* y_out, void* stream) {
  return residual_rms_call(h, o, bias, scale, gamma, eps, m, k, global_amax, nullptr, codes, scales, rstd_out, y_out,
                           stream);
}

int residual_rms_nvfp4_dynamic(float* h, const void* o, const void* bias, const float* scale, const float* gamma,
                              float eps, int64_t m, int64_t k, float* amax_out, void* codes, void* scales,
                              float* rstd_out, void* y_out, void* stream) {
  if (m < 0 || k <= 0 || k % 512 != 0 || k > nvfp4act::kMaxResidualK) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return residual_rms_call(h, o, bias, scale, gamma, eps, m, k, 0.0f, amax_out, codes, scales, rstd_out, y_out,
                           stream);
}

int residual_rms_adaln_nvfp4(float* h, const void* o, const void* bias, const void* gate, int64_t gate_stride,
                             const void* weight, const void* shift, const void* scale, int64_t frame_stride,
                             int64_t num_frames, const int32_t* frame_idx, float eps, int64_t m, int64_t k,
                             float global_amax, void* codes, void* scales, float* rstd_out, void* y_out,
                             uint32_t* status_word, void* stream) {
  const FoldTables f{gate, gate_stride, weight, shift, scale, frame_stride, num_frames, frame_idx, status_word};
  return residual_adaln_call(h, o, bias, f, eps, m, k, global_amax, nullptr, codes, scales, rstd_out, y_out, stream);
}

int residual_rms_adaln_nvfp4_dynamic(float* h, const void* o, const void* bias, const void* gate,
                                     int64_t gate_stride, const void* weight, const void* shift, const void* scale,
                                     int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx, float eps,
                                     int64_t m, int64_t k, float* amax_out, void* codes, void* scales,
                                     float* rstd_out, void* y_out, uint32_t* status_word, void* stream) {
  const FoldTables f{gate, gate_stride, weight, shift, scale, frame_stride, num_frames, frame_idx, status_word};
  int st = residual_adaln_shape(m, k, o, f);
  if (st != NVFP4ACT_OK) return st;
  st = check_amax_out(m, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return residual_adaln_call(h, o, bias, f, eps, m, k, 0.0f, amax_out, codes, scales, rstd_out, y_out, stream);
}

int rms_silu_nvfp4(const void* x, const void* gamma, float eps, int64_t rows, int64_t c, float global_amax,
                   void* codes, void* scales, float* rstd_out, void* y_out, void* stream) {
  return rms_silu_call(x, gamma, eps, rows, c, global_amax, nullptr, codes, scales, rstd_out, y_out, stream);
}

int rms_silu_nvfp4_dynamic(const void* x, const void* gamma, float eps, int64_t rows, int64_t c, float* amax_out,
                           void* codes, void* scales, float* rstd_out, void* y_out, void* stream) {
  if (rows < 0 || c < 16 || c > 512 || c % 16 != 0) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(rows, amax_out);
  if (st != NVFP4ACT_OK) return st;
  return rms_silu_call(x, gamma, eps, rows, c, 0.0f, amax_out, codes, scales, rstd_out, y_out, stream);
}

int ln_adaln_fp8(const void* x, const float* scale, const float* shift, float eps, int64_t m, int64_t k,
                 float act_scale, void* codes, float* mean_out, float* rstd_out, float* y_out, void* stream) {
  return ln_fp8_call(x, scale, shift, eps, m, k, act_scale, nullptr, codes, mean_out, rstd_out, y_out, stream);
}

int ln_adaln_fp8_dynamic(const void* x, const float* scale, const float* shift, float eps, int64_t m, int64_t k,
                         float* act_scale_out, void* codes, float* mean_out, float* rstd_out, float* y_out,
                         void* stream) {
  if (!ln_shape_ok(m, k)) return NVFP4ACT_ERR_SHAPE;
  int st = check_amax_out(m, act_scale_out);
  if (st != NVFP4ACT_OK) return st;
  return ln_fp8_call(x, scale, shift, eps, m, k, 0.0f, act_scale_out, codes, mean_out, rstd_out, y_out, stream);
}

}  // extern "C"
