/*
 * nvfp4act.h -- C ABI of libnvfp4act.so: producer-fused NVFP4 activation
 * quantization for AMD Instinct MI355X (gfx950).
 *
 * Three producers, each fused with the same NVFP4 block quantizer:
 *   rms_adaln_nvfp4  RMSNorm (fp32 statistic) + adaLN modulation -> NVFP4
 *   swiglu_nvfp4     SiLU(gate) * up                              -> NVFP4
 *                    (swiglu_packed_nvfp4: packed projection, bias before
 *                    SiLU, value-first or paired columns)
 *   nvfp4_quantize   identity (attention-output quantize)         -> NVFP4
 * and a fourth that folds a residual add into the norm:
 *   residual_rms_nvfp4  h += bf16(o + bias) * scale (fp32, in place);
 *                       RMSNorm with an fp32 weight               -> NVFP4
 *   residual_rms_adaln_nvfp4  h += bf16(o + bias) * gate[t] (fp32, in place);
 *                       RMSNorm + adaLN of the next block         -> NVFP4
 * and, for fp16 channels-last (VAE) activations:
 *   rms_silu_nvfp4   RMSNorm over channels + SiLU                  -> NVFP4
 *
 * Sources: TensorRT-LLM PR #21483 "Fuse the MiniMax-H3 NVFP4 activation
 * quantize into the AdaLN, SwiGLU and attention-output producers" (Summary);
 * FastVideo API page "fastvideo.models.vaes.minimax_h3_nvfp4_fused" (module
 * summary, new_quantized, quantize, swiglu_quantize); FastVideo branch compare
 * "regen2k-nvfp4-decoder..fasth3-spark-exact-perf", minimax_h3_swiglu_quant.cuh
 * (scale_fp8, scale_float, fp4_pair, quant_probe, launch_quant_probe) and
 * h3_swiglu_gemm_binding.py (int status, nonzero -> error); FastVideo commit
 * log "vae-parallel-decode" (int64 indexing past 2^31 elements, frame-index
 * bounds contract).
 *
 * The NVFP4 format written by every entry point
 * ---------------------------------------------
 * Input rows of k bf16 values are cut into 16-element blocks.  With the
 * global scale gsf = 2688 / global_amax (2688 = 448 * 6, IEEE fp32):
 *   block scale   s   = E4M3(gsf * (max|y| * fp32(1/6))), round to nearest
 *                       even, saturating at 448 (code 0x7E); OCP E4M3 codes
 *   element code  q_i = E2M1(y_i * inv), inv = (s != 0) ? gsf / dec(s) : 0,
 *                       round to nearest even, saturating at 6; bit 3 = sign
 *                       of the product (so -0 encodes as 0x8)
 * codes  [m, k/2] bytes, row-major; byte j of a row holds columns 2j (low
 *        nibble) and 2j+1 (high nibble).
 * scales [pad(m), k/16] bytes, pad(m) = ceil(m/128)*128, in the 128x4
 *        swizzled layout: the scale of (row r, block b) is at byte
 *        ((r/128)*(k/64) + b/4)*512 + (r%32)*16 + ((r/32)%4)*4 + b%4.
 *        The bytes of rows m .. pad(m)-1 are written as 0.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All data pointers are device pointers (HIP device memory visible to the
 *   current device).  bf16 data is passed as raw 16-bit patterns.
 * - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *   void*, NULL = the default stream), allocates nothing and never waits for
 *   the device.  The first call on a device probes it once (its properties and
 *   kernel attributes; no device work, no stream use).  The SiLU tables of the
 *   swiglu_* and rms_silu_* calls are constants generated when the library is
 *   built, so those calls may be captured into a HIP graph from the first one.
 * - Ownership: the caller allocates and frees every buffer.  Inputs must stay
 *   valid and unmodified, and outputs untouched, until the stream work is done.
 *   The library writes only codes, scales and the non-NULL side outputs.
 * - Errors: arguments are checked on the host before anything is launched; on
 *   an error nothing is written and a nonzero status is returned (see
 *   NVFP4ACT_* below).  m == 0 (with valid k) is a no-op that returns 0 before
 *   any other check, so empty tensors may pass NULL pointers.  Faults inside a kernel
 *   surface at the caller's next synchronisation.
 * - Inputs are finite bf16.  Non-finite inputs are outside the contract.
 * - Calls are stateless and thread-safe; sizes are int64 and all device
 *   indexing is 64-bit (tensors past 2^31 elements are supported).
 */
#ifndef NVFP4ACT_H
#define NVFP4ACT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define NVFP4ACT_OK            0
#define NVFP4ACT_ERR_NULL      1  /* a required pointer is NULL                         */
#define NVFP4ACT_ERR_SHAPE     2  /* m < 0, bad k / f / ld / num_frames / frame_stride   */
#define NVFP4ACT_ERR_ALIGN     3  /* a pointer, row stride or frame stride not 16-byte aligned */
#define NVFP4ACT_ERR_VALUE     4  /* global_amax not finite or too small; eps not finite or < 0 */
#define NVFP4ACT_ERR_DEVICE    5  /* no usable gfx950 device is current                  */
#define NVFP4ACT_ERR_LAUNCH    6  /* a HIP call failed; see nvfp4act_last_hip_error()   */
#define NVFP4ACT_ERR_TABLE     7  /* reserved: no longer returned (SiLU tables are built in) */

/* ceil(m / 128) * 128: rows of the swizzled scale buffer */
int64_t nvfp4act_padded_rows(int64_t m);
/* m * k / 2: bytes of the packed codes */
int64_t nvfp4act_codes_bytes(int64_t m, int64_t k);
/* padded_rows(m) * k / 16: bytes of the swizzled scales */
int64_t nvfp4act_scales_bytes(int64_t m, int64_t k);
/* 2688.0f / global_amax (IEEE fp32), the global scale the kernels use */
float nvfp4act_global_scale(float global_amax);
/* static text for a status code */
const char* nvfp4act_status_string(int status);
/* HIP error code behind the last NVFP4ACT_ERR_LAUNCH of the calling thread */
int nvfp4act_last_hip_error(void);
/* Hex sha256 of the sources the library was built from (the files of csrc/ and
   this header, in name order, each preceded by its file name), so that a
   caller can check that a binary matches the sources beside it.  Static text. */
const char* nvfp4act_source_digest(void);

/* Probe the current device (gfx950, CU count, kernel attributes, the device
   address of the library's scratch).  Idempotent and optional: every entry
   point does it on its first call on a device.  Returns a status. */
int nvfp4act_init(void);

/* Standalone NVFP4 quantize of a bf16 tensor (the attention-output quantize).
   FastVideo API page, quantize; TensorRT-LLM PR #21483, attention-output
   quantize commit.
     x       [m, k] bf16, row-major, contiguous, 16-byte aligned
     m       rows, >= 0
     k       columns, a positive multiple of 64
     global_amax  static per-tensor amax (> 0, finite, 2688/global_amax finite)
     codes   [m, k/2] bytes (16-byte aligned)
     scales  [pad(m), k/16] bytes (16-byte aligned)
   Returns a status. */
int nvfp4_quantize(const void* x, int64_t m, int64_t k, float global_amax,
                   void* codes, void* scales, void* stream);

/* Fused RMSNorm + adaLN modulation -> NVFP4 (the AdaLN RMSNorm + modulation
   producer of TensorRT-LLM PR #21483; every bf16 rounding of the op-by-op
   eager path kept, FastVideo API page summary).  Per row r with t = frame_idx[r]:
     rstd = 1 / sqrt(sum(x^2) / k + eps)   fp32, fixed reduction tree:
            8 interleaved accumulators per lane over 8-element chunks
            L, L+64, ... (fused multiply-add), folded pairwise, then a
            butterfly over the 64 lanes at distances 1, 2, 4, ..., 32
     y    = bf16(bf16(bf16(bf16(x*rstd) * w) * bf16(1 + scale[t])) + shift[t])
   then the NVFP4 quantizer above.
     x            [m, k] bf16 (16-byte aligned rows)
     weight       [k] bf16 RMSNorm weight
     shift, scale modulation rows: frame t's rows start at shift + t*frame_stride
                  and scale + t*frame_stride elements (for a [T, 2, k] table of
                  (shift, scale): shift = table, scale = table + k, frame_stride = 2k)
     frame_stride elements between frames (>= k; frame_stride*2 a multiple of 16)
     num_frames   T >= 1
     frame_idx    [m] int32 frame of each row; must lie in [0, T).  A row with an
                  index outside that range is written as all-zero codes and
                  scale bytes (and a zero y_out row) and bit 0 of *status_word is
                  set; nothing waits for the check (FastVideo commit log,
                  modulation bounds contract).
     eps          >= 0 and finite
     m, k         m >= 0; k a positive multiple of 512
     global_amax  as for nvfp4_quantize
     codes, scales  outputs as for nvfp4_quantize
     rstd_out     [m] fp32, nullable: the row statistic
     y_out        [m, k] bf16, nullable: the pre-quantization activation
     status_word  one uint32 in device memory, nullable; bits are only ever set
                  (OR), so the caller clears it
   Returns a status. */
int rms_adaln_nvfp4(const void* x, const void* weight, const void* shift, const void* scale,
                    int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                    float eps, int64_t m, int64_t k, float global_amax,
                    void* codes, void* scales, float* rstd_out, void* y_out,
                    uint32_t* status_word, void* stream);

/* SwiGLU -> NVFP4 (FastVideo API page, swiglu_quantize; TensorRT-LLM PR
   #21483, SiLU-and-mul producer):
     y = bf16(S[gate] * up),  S[g] = bf16(g * sigmoid(g)) correctly rounded
   then the NVFP4 quantizer above.
     up, gate  row i at up + i*ld, gate + i*ld elements, f values each (for a
               value-first [m, 2f] projection: gate = up + f, ld = 2f)
     ld        row stride in elements (>= f; ld*2 a multiple of 16)
     m, f      m >= 0; f a positive multiple of 64
     global_amax, codes, scales  as for nvfp4_quantize (k = f)
     y_out     [m, f] bf16, nullable
   Returns a status. */
int swiglu_nvfp4(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f,
                 float global_amax, void* codes, void* scales, void* y_out, void* stream);

/* SwiGLU -> NVFP4 of a packed [m, 2f] projection with an optional bias added
   before SiLU (FastVideo API page, swiglu_quantize: the projection arrives
   value half first and without its bias; FastVideo branch compare,
   minimax_h3_swiglu_quant.cuh, quant_probe: the paired layout).  For output
   column j of row i (row i of the projection at proj + i*ld elements):
     interleaved = 0   value at column j,    gate at column f + j
     interleaved = 1   value at column 2j,   gate at column 2j + 1
   With a bias, value and gate first become bf16(value + bias[vc]) and
   bf16(gate + bias[gc]) (fp32 sum, round to nearest even), vc and gc being the
   columns just named; then y = bf16(S[gate] * value) and the quantizer.
     proj         bf16, 16-byte aligned
     bias         nullable; 2f bf16 values in the projection's column order
                  (one projection row), 16-byte aligned
     interleaved  0 or 1 (otherwise status 2)
     ld           row stride in elements (>= 2f; ld*2 a multiple of 16)
     m, f, global_amax, codes, scales, y_out  as for swiglu_nvfp4
   A biased value or gate that overflows bf16 is outside the contract, like a
   non-finite input.  Returns a status. */
int swiglu_packed_nvfp4(const void* proj, const void* bias, int interleaved, int64_t ld, int64_t m,
                        int64_t f, float global_amax, void* codes, void* scales, void* y_out,
                        void* stream);

/* fp32 residual stream + RMSNorm (fp32 weight) -> NVFP4 (FastVideo API page,
   residual_norm_quantize: a block's branch output is added to the fp32
   residual stream in place, and the next norm's quantized activation is
   produced in the same pass).  Per row, element d:
     t    = bf16(o[d] + bias[d])            (t = o[d] without a bias)
     h[d] = h[d] + t * scale[d]             fp32, the product rounded before the
                                            add; written back into h
     rstd = 1 / sqrt(sum(h^2) / k + eps)    fp32, fixed reduction tree:
            4 accumulators per lane over the 4-element quads L, L+64, ...
            (fused multiply-add), folded as (a0 + a1) + (a2 + a3), then the
            butterfly of rms_adaln_nvfp4 over the 64 lanes
     y[d] = bf16((h[d] * rstd) * gamma[d])
   then the NVFP4 quantizer above.
     h         [m, k] fp32, row-major, contiguous, 16-byte aligned; updated in
               place when o is given, only read otherwise
     o         [m, k] bf16 (contiguous, 16-byte aligned), nullable: no residual
     bias      [k] bf16, nullable (ignored without o)
     scale     [k] fp32, required with o (ignored without)
     gamma     [k] fp32 RMSNorm weight
     eps       >= 0 and finite
     m, k      m >= 0; k a positive multiple of 512, at most 8192 (a row is
               held in registers)
     global_amax, codes, scales  as for nvfp4_quantize
     rstd_out  [m] fp32, nullable
     y_out     [m, k] bf16, nullable: the pre-quantization activation
   Every pointer argument is 16-byte aligned (rstd_out 4-byte).  Returns a
   status. */
int residual_rms_nvfp4(float* h, const void* o, const void* bias, const float* scale,
                       const float* gamma, float eps, int64_t m, int64_t k, float global_amax,
                       void* codes, void* scales, float* rstd_out, void* y_out, void* stream);

/* The gated MLP residual of a DiT block carried out by the next block's RMSNorm
   + adaLN producer, over an fp32 residual stream (TensorRT-LLM PR #21483,
   Summary: the next block's normalization performs the MLP branch's residual
   add, taking the gate from the current block's AdaLN table and the shift and
   scale from its own; FastVideo API page, residual_norm_quantize: the fp32
   stream updated in place).  Per row r with t = frame_idx[r], element d:
     u    = bf16(o[d] + bias[d])               (u = o[d] without a bias)
     h[d] = h[d] + u * gate_t[d]               fp32, the product rounded, then
                                               the add; written back into h
     rstd = the fp32 statistic of residual_rms_nvfp4 over the updated row
     y    = bf16(bf16(bf16(bf16(h*rstd) * w) * bf16(1 + scale_t)) + shift_t)
   then the NVFP4 quantizer above.
     h            [m, k] fp32 (as for residual_rms_nvfp4)
     o, bias      the branch and its bias, as for residual_rms_nvfp4 (o
                  nullable: no residual add)
     gate         the folding block's gate rows: row t at gate + t*gate_stride
                  bf16 elements (required with o)
     gate_stride  >= k, gate_stride*2 a multiple of 16 (checked only with o)
     weight       [k] bf16 RMSNorm weight
     shift, scale the next block's modulation rows, laid out as for
                  rms_adaln_nvfp4 (frame_stride, num_frames)
     frame_idx    [m] int32, in [0, num_frames).  A row outside that range keeps
                  its h (no residual add), is written as zero codes, zero scale
                  bytes and a zero y_out row, and sets bit 0 of *status_word;
                  its rstd_out is the statistic of the unchanged row
     eps, m, k, global_amax, codes, scales, rstd_out, y_out  as for
                  residual_rms_nvfp4; status_word as for rms_adaln_nvfp4
   Returns a status. */
int residual_rms_adaln_nvfp4(float* h, const void* o, const void* bias, const void* gate,
                             int64_t gate_stride, const void* weight, const void* shift,
                             const void* scale, int64_t frame_stride, int64_t num_frames,
                             const int32_t* frame_idx, float eps, int64_t m, int64_t k,
                             float global_amax, void* codes, void* scales, float* rstd_out,
                             void* y_out, uint32_t* status_word, void* stream);

/* Channels-last RMSNorm + SiLU -> NVFP4 of fp16 activations (FlashRT PR #142,
   fp16_quant_nvfp4_ndhwc: the fused RMS_norm + SiLU + NVFP4 quantize of the
   VAE's channels-last tensors, per-16-channel UE4M3 scales; fp32 statistics
   with an fp16 affine as in its RMSNorm+RoPE kernel).  Per row (one voxel's c
   channels):
     rstd = 1 / sqrt(sum(x^2) / c + eps)   fp32; the tree of rms_adaln_nvfp4
            with one 8-element chunk per lane over S lanes, S the smallest
            power of two >= c/8 (lanes past c/8 hold 0), butterfly 1 .. S/2
     a    = fp16(fp16(x * rstd) * gamma)
     y    = fp16(a * sigmoid(a)) correctly rounded
   then the NVFP4 quantizer above, with the scale bytes in plain row order.
     x         [rows, c] fp16, row-major (channels-last), 16-byte aligned
     gamma     [c] fp16, 16-byte aligned
     eps       >= 0 and finite
     rows, c   rows >= 0; c a multiple of 16 in [16, 512]
     global_amax  as for nvfp4_quantize
     codes     [rows, c/2] bytes (4-byte aligned)
     scales    [rows, c/16] bytes: the E4M3 scale of block b of row r at
               r*(c/16) + b (no swizzle, no padding rows)
     rstd_out  [rows] fp32, nullable
     y_out     [rows, c] fp16, nullable: the pre-quantization activation
   Returns a status. */
int rms_silu_nvfp4(const void* x, const void* gamma, float eps, int64_t rows, int64_t c,
                   float global_amax, void* codes, void* scales, float* rstd_out, void* y_out,
                   void* stream);

/* LayerNorm (fp32 statistics) + adaLN -> per-tensor FP8 E4M3 (FlashRT PR #142,
   commit notes on fp16_ada_layernorm_quant_fp8: one pass, fp32 LayerNorm
   statistics, adaLN modulation, one FP8 scale shared by the three projections
   that read the result; it also feeds the FFN's first projection).  Per row of
   k elements:
     mean = sum(x) / k              fp32; the tree of rms_adaln_nvfp4 (lane L
                                    owns the 8-element chunks L + 64 j, eight
                                    accumulators, pairwise lane fold, butterfly)
     var  = sum((x - mean)^2) / k   the same tree, fused multiply-adds
     rstd = 1 / sqrt(var + eps)
     y    = (((x - mean) * rstd) * (1 + scale)) + shift   fp32, each op rounded
     code = E4M3(y * (1 / act_scale)), nearest-even, saturating at +-448, the
            sign kept (a negative zero or a negative value that rounds to zero
            gives 0x80)
     x         [m, k] fp16, row-major, 16-byte aligned
     scale, shift  [k] fp32 each (the call's adaLN modulation row), 16-byte
               aligned
     eps       >= 0 and finite
     m, k      m >= 0; k a multiple of 512 in [512, 8192]
     act_scale the static per-tensor scale: finite, > 0, with 1 / act_scale
               finite
     codes     [m, k] bytes (8-byte aligned)
     mean_out, rstd_out  [m] fp32 each, nullable
     y_out     [m, k] fp32, nullable (16-byte aligned): the pre-quantization y
   Returns a status. */
int ln_adaln_fp8(const void* x, const float* scale, const float* shift, float eps, int64_t m,
                 int64_t k, float act_scale, void* codes, float* mean_out, float* rstd_out,
                 float* y_out, void* stream);

/* The per-call form of ln_adaln_fp8 (FlashRT PR #142: 2-pass device-side amax
   then quantize, no host sync): *act_scale_out = 0, an amax pass folds max |y|
   over all rows into it, a one-thread kernel turns it into act_scale =
   amax / 448, then ln_adaln_fp8 runs with 1 / act_scale taken on the device
   (0 when act_scale is 0 or its reciprocal overflows: every code a signed
   zero).  act_scale_out: one float in device memory (4-byte aligned, required
   unless m == 0; not written when m == 0); it holds the call's scale afterwards
   (the dequantization factor of the codes).  Calls that share it and overlap
   on the device race on it. */
int ln_adaln_fp8_dynamic(const void* x, const float* scale, const float* shift, float eps,
                         int64_t m, int64_t k, float* act_scale_out, void* codes, float* mean_out,
                         float* rstd_out, float* y_out, void* stream);

/* Per-call (dynamic) global amax
   ------------------------------
   The *_dynamic forms take the global amax from the tensor itself instead of
   a static calibration (FlashRT PR #142: NVFP4 W4A4 with a dynamic per-call
   activation scale, a device-side amax pass then the quantize, no host sync;
   FastVideo API page, NVFP4DecoderLinear act_scale="dynamic", per-call
   abs-max).  Each call enqueues three kernels on `stream`: *amax_out = 0; an
   amax pass that folds max |y| over all rows into *amax_out (y = the producer's
   pre-quantization activation; rows with an out-of-range frame index count as
   y = 0); the producer with the global scale computed on the device:
     gsf = 2688 / *amax_out   if that is positive and finite,
     gsf = 0                  otherwise (an all-zero tensor, or an amax so
                              small that 2688 / amax overflows): every block
                              scale is 0 and every code a signed zero.
   The maximum is exact and order-free, so results do not depend on the launch.
   amax_out is one float in device memory (4-byte aligned, required unless
   m == 0; not written when m == 0).  The other arguments, outputs and status
   codes are those of the static form; the producer's work is done twice (once
   for the amax, once to quantize).  Calls that share one amax_out and overlap
   on the device race on it. */
int nvfp4_quantize_dynamic(const void* x, int64_t m, int64_t k, float* amax_out,
                           void* codes, void* scales, void* stream);

int rms_adaln_nvfp4_dynamic(const void* x, const void* weight, const void* shift, const void* scale,
                            int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                            float eps, int64_t m, int64_t k, float* amax_out,
                            void* codes, void* scales, float* rstd_out, void* y_out,
                            uint32_t* status_word, void* stream);

/* rms_adaln_nvfp4_dynamic without the amax_out argument, for callers that
   cannot allocate device memory (code under HIP graph capture, tight serving
   loops, harnesses that forbid hipMalloc): the call's amax word lives in a
   256-byte scratch array that the library holds in device memory for each
   device, from the first call on that device until the process ends.  The
   call itself allocates nothing (no hipMalloc, hipFree or allocating library
   routine); it enqueues the same three kernels as rms_adaln_nvfp4_dynamic (a
   fill kernel zeroes the word, the amax pass, the producer) on `stream`.
   Every call needs exactly one word of that scratch whatever m and k are, so
   no input size exceeds it.  All calls on one device share the word: calls
   that overlap on the device (different streams, or host threads without
   ordering) race on it and may quantize with each other's amax; serialize
   them.  The amax itself is not returned.  Arguments, outputs and status
   codes are those of rms_adaln_nvfp4_dynamic. */
int rms_adaln_nvfp4_dynamic_noalloc(const void* x, const void* weight, const void* shift,
                                    const void* scale, int64_t frame_stride, int64_t num_frames,
                                    const int32_t* frame_idx, float eps, int64_t m, int64_t k,
                                    void* codes, void* scales, float* rstd_out, void* y_out,
                                    uint32_t* status_word, void* stream);

int swiglu_nvfp4_dynamic(const void* up, const void* gate, int64_t ld, int64_t m, int64_t f,
                         float* amax_out, void* codes, void* scales, void* y_out, void* stream);

int swiglu_packed_nvfp4_dynamic(const void* proj, const void* bias, int interleaved, int64_t ld,
                                int64_t m, int64_t f, float* amax_out, void* codes, void* scales,
                                void* y_out, void* stream);

/* The amax pass reads h and o without writing anything; the second pass
   updates h as the static form does. */
int residual_rms_nvfp4_dynamic(float* h, const void* o, const void* bias, const float* scale,
                               const float* gamma, float eps, int64_t m, int64_t k,
                               float* amax_out, void* codes, void* scales, float* rstd_out,
                               void* y_out, void* stream);

int residual_rms_adaln_nvfp4_dynamic(float* h, const void* o, const void* bias, const void* gate,
                                     int64_t gate_stride, const void* weight, const void* shift,
                                     const void* scale, int64_t frame_stride, int64_t num_frames,
                                     const int32_t* frame_idx, float eps, int64_t m, int64_t k,
                                     float* amax_out, void* codes, void* scales, float* rstd_out,
                                     void* y_out, uint32_t* status_word, void* stream);

int rms_silu_nvfp4_dynamic(const void* x, const void* gamma, float eps, int64_t rows, int64_t c,
                           float* amax_out, void* codes, void* scales, float* rstd_out, void* y_out,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4ACT_H */
