/*
 * nvfp4_oracle.c -- plain, slow, single-threaded CPU oracle for producer-fused
 * NVFP4 activation quantization (RMSNorm + adaLN, SwiGLU and standalone
 * producers, each followed by the NVFP4 block quantizer).
 *
 * TEST INFRASTRUCTURE ONLY.  This file defines what the GPU library must
 * compute, bit for bit.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the HIP library and must never be called from it.
 *
 * Sources (the pages this follows; no code is taken from them):
 *   [H3-API]  FastVideo API page "fastvideo.models.vaes.minimax_h3_nvfp4_fused":
 *             module summary (every bf16 rounding of the eager path is kept,
 *             E4M3 block scales, 128x4 swizzle, zeroed padding rows),
 *             new_quantized (buffer shapes), quantize, swiglu_quantize.
 *   [TRT]     TensorRT-LLM PR #21483 "Fuse the MiniMax-H3 NVFP4 activation
 *             quantize into the AdaLN, SwiGLU and attention-output producers",
 *             Summary (AdaLN RMSNorm + modulation and SiLU-and-mul producers
 *             emit packed E2M1 codes and swizzled E4M3 scales; static scales).
 *   [PROBE]   FastVideo branch compare "regen2k-nvfp4-decoder..fasth3-spark-
 *             exact-perf", file minimax_h3_swiglu_quant.cuh: scale_fp8,
 *             scale_float, fp4_pair and the quant_probe kernel (block amax over
 *             16 lanes, scale = gsf * amax / 6 rounded to E4M3 with saturation,
 *             per-element multiply by the inverse scale, E2M1 pair packing,
 *             swizzled scale index, padding rows).
 *   [INT64]   FastVideo commit log, branch vae-parallel-decode: the int64
 *             indexing fix at 2^31 elements and the frame-index bounds
 *             contract of the modulation wrappers.
 *   [FlashRT] FlashRT PR #142 (MiniMax-Remover): fp16_ada_layernorm_quant_fp8
 *             (one-pass fp32-stat LayerNorm + adaLN + per-tensor FP8 E4M3
 *             with one scale shared by Q/K/V); fp16_quant_nvfp4_ndhwc, the
 *             fused RMS_norm + SiLU + NVFP4 quantize of channels-last VAE
 *             activations, per-16-channel UE4M3 scales; the RMSNorm+RoPE
 *             kernel's fp32 statistics with an fp16 affine.
 *   [H3-API residual_norm_quantize]  the fp32 residual stream: in-place
 *             h += bf16(o + bias) * scale, then NVFP4 of bf16(rms_norm(h,
 *             gamma, eps)) with fp32 gamma; hidden size a multiple of 512.
 *
 * Readings taken where the pages are silent:
 *   - global scale gsf = 2688 / global_amax (448 * 6), IEEE fp32 division;
 *   - 1/6 is the correctly rounded fp32 constant, not an approximate rcp;
 *   - inverse scale = gsf / dec(s) (IEEE), and 0 when the scale code is 0;
 *   - RMSNorm statistic: the fixed reduction tree of rms_rstd() below;
 *   - RMSNorm output is rounded to bf16 before the weight multiply;
 *   - SiLU is tabulated as the correctly rounded bf16 of g*sigmoid(g);
 *   - fp32 residual stream: the quad tree of rms_sum_f32() below; the product
 *     t * scale is rounded before the add (no fused multiply-add); the norm
 *     is (h * rstd) * gamma in fp32, rounded to bf16 once.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (SSE float, no x87
 * for the fp32 chain).  Every entry point clears FTZ/DAZ and selects
 * round-to-nearest in MXCSR for its duration, so denormals are IEEE.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------- */
/* floating-point environment                                                */
/* ------------------------------------------------------------------------- */

static unsigned int enter_ieee(void) {
    unsigned int saved = _mm_getcsr();
    /* clear FTZ (bit 15), DAZ (bit 6) and rounding control (bits 13-14 -> RN),
       mask all exceptions (bits 7-12) */
    unsigned int csr = (saved & ~(0x8000u | 0x0040u | 0x6000u)) | 0x1F80u;
    _mm_setcsr(csr);
    return saved;
}

static void leave_ieee(unsigned int saved) { _mm_setcsr(saved); }

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ------------------------------------------------------------------------- */
/* bf16 (round to nearest, ties to even; no flush to zero)                   */
/* ------------------------------------------------------------------------- */

/* The bf16 value nearest to f: of the two bf16 neighbours of f (f with its low
   16 bits cleared, and the next bf16 away from zero) take the nearer; on a tie
   take the one whose last kept bit is 0.  Overflow past the largest finite
   bf16 rounds to infinity as IEEE rounding does.  NaN -> canonical 0x7FC0. */
static uint16_t bf16_round(float f) {
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return 0x7FC0u;
    uint32_t toward_zero = u >> 16;          /* truncated magnitude, sign kept */
    uint32_t dropped = u & 0xFFFFu;          /* the discarded 16 bits          */
    int round_up;
    if (dropped > 0x8000u) round_up = 1;
    else if (dropped < 0x8000u) round_up = 0;
    else round_up = (int)(toward_zero & 1u); /* exact tie: go to even          */
    return (uint16_t)(toward_zero + (uint32_t)round_up);
}

static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16 -> fp32: the value after one kept bf16 rounding */
static float rb(float f) { return bf16_to_f32(bf16_round(f)); }

/* ------------------------------------------------------------------------- */
/* fp16 (IEEE binary16: 5 exponent bits, bias 15, 10 mantissa bits)          */
/* ------------------------------------------------------------------------- */

/* Exact value of an fp16 pattern as fp32 (every fp16 value is an fp32 value). */
static float f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    if (e == 0x1Fu) return f32_from_bits(sign | 0x7F800000u | (m << 13));   /* inf, NaN */
    double v = (e == 0) ? ldexp((double)m, -24) : ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
    float f = (float)v;                       /* exact */
    return (sign ? -f : f);
}

/* The fp16 value nearest to f, ties to the even pattern; magnitudes from the
   midpoint 65520 up round to infinity; subnormals kept (quantum 2^-24);
   NaN -> 0x7E00.  Works on the exact fp32 value in double precision. */
static uint16_t f16_round(float f) {
    if (isnan(f)) return 0x7E00u;
    uint16_t sign = signbit(f) ? 0x8000u : 0;
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    int e2;
    frexp(a, &e2);                            /* a = fr * 2^e2, fr in [0.5, 1) */
    int E = e2 - 1;                           /* 2^E <= a < 2^(E+1) */
    int qexp = (E < -14) ? -24 : E - 10;      /* fp16 quantum exponent */
    double n = ldexp(a, -qexp);               /* exact */
    double fl = floor(n), frac = n - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) == 1.0)) fl += 1.0;
    if (fl == 0.0) return sign;               /* below half the smallest subnormal */
    double v = ldexp(fl, qexp);               /* the rounded magnitude (< 65520: finite) */
    /* encode */
    int ev;
    frexp(v, &ev);
    int Ev = ev - 1;
    uint16_t bits;
    if (Ev < -14) bits = (uint16_t)ldexp(v, 24);                       /* subnormal (or 2^-14) */
    else bits = (uint16_t)(((Ev + 15) << 10) | ((uint32_t)(ldexp(v, -Ev) * 1024.0) - 1024u));
    return (uint16_t)(sign | bits);
}

/* fp32 -> fp16 -> fp32: the value after one kept fp16 rounding */
static float rh(float f) { return f16_to_f32(f16_round(f)); }

/* ------------------------------------------------------------------------- */
/* E4M3 (OCP FN: bias 7, 3 mantissa bits, max finite 448 = code 0x7E)       */
/* ------------------------------------------------------------------------- */

/* Value of a non-negative E4M3 code 0..126 (0x7F is NaN and never produced):
   exponent field 0 is subnormal m * 2^-9, otherwise 2^(e-7) * (1 + m/8). */
static double e4m3_value(uint8_t code) {
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* The values of codes 0..126 (e4m3_value), filled once when the library is
   loaded so that the encoder's search reads a table. */
static double e4m3_values[127];

__attribute__((constructor)) static void fill_e4m3_values(void) {
    for (int c = 0; c < 127; ++c) e4m3_values[c] = e4m3_value((uint8_t)c);
}

/* Round a non-negative fp32 to the nearest finite E4M3 value, ties to the
   even code, saturating (everything at or above 448, +inf included, maps to
   448).  The finite codes 0..126 are increasing in value, so the encoder
   finds the bracketing pair and compares x with their exact midpoint. */
static uint8_t e4m3_encode(float x) {
    double v = (double)x;                    /* exact */
    if (!(v > 0.0)) return 0;                /* +0, -0 (and NaN: out of contract) */
    if (v >= 448.0) return 0x7E;
    int lo = 0, hi = 126;                    /* invariant: value(lo) <= v < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_values[mid] <= v) lo = mid; else hi = mid;
    }
    double a = e4m3_values[lo], b = e4m3_values[hi];
    double midpoint = 0.5 * (a + b);         /* exact: few significant bits */
    if (v < midpoint) return (uint8_t)lo;
    if (v > midpoint) return (uint8_t)hi;
    return (uint8_t)((lo % 2 == 0) ? lo : hi);
}

/* ------------------------------------------------------------------------- */
/* E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; bit 3 sign)   */
/* ------------------------------------------------------------------------- */

static double e2m1_value(uint8_t code) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest E2M1 magnitude to |v| with ties to the even code, saturating at 6
   (so +-inf -> 6); the sign bit is the sign of v, so -0 and small negatives
   encode as 0x8.  NaN is outside the contract (encoded as 0x7 | sign). */
static uint8_t e2m1_encode(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (isnan(v)) return (uint8_t)(sign | 7);
    if (a >= 6.0) return (uint8_t)(sign | 7);
    int lo = 0;
    while (lo < 7 && e2m1_value((uint8_t)(lo + 1)) <= a) lo++;
    int hi = lo + 1;                         /* value(lo) <= a < value(hi) */
    double midpoint = 0.5 * (e2m1_value((uint8_t)lo) + e2m1_value((uint8_t)hi));
    int code;
    if (a < midpoint) code = lo;
    else if (a > midpoint) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------- */
/* swizzled scale layout                                                     */
/* ------------------------------------------------------------------------- */

/* Byte offset of the scale of 16-element block b of row r in a scale buffer
   for rows of k elements ([PROBE] quant_probe index): 128-row x 4-block tiles
   of 512 bytes, tiles ordered row-tile-major; inside a tile the byte for
   (r, b) sits at (r % 32) * 16 + ((r / 32) % 4) * 4 + b % 4. */
static int64_t scale_offset(int64_t r, int64_t b, int64_t k) {
    int64_t tiles_per_row_tile = k / 64;
    return ((r / 128) * tiles_per_row_tile + b / 4) * 512
         + (r % 32) * 16 + ((r / 32) % 4) * 4 + (b % 4);
}

static int64_t padded_rows(int64_t m) { return (m + 127) / 128 * 128; }

/* ------------------------------------------------------------------------- */
/* the NVFP4 block quantizer                                                 */
/* ------------------------------------------------------------------------- */

static const uint32_t RCP6_BITS = 0x3E2AAAABu;   /* fp32 nearest to 1/6 */

static float global_scale(float global_amax) { return 2688.0f / global_amax; }

/* Global scale of a per-call (dynamic) amax, measured on the tensor itself
   ([FlashRT] "dynamic per-call activation" scale, device-side amax then
   quantize; [H3-API] NVFP4DecoderLinear act_scale="dynamic", per-call
   abs-max).  The pages give the scale only for a positive amax.  Reading: the
   same 2688 / amax when that is positive and finite; otherwise (an all-zero
   tensor, or an amax so small that 2688 / amax overflows) the scale is 0, so
   every block scale is E4M3 0 and every element code is a signed zero. */
static float dynamic_global_scale(float amax) {
    if (!(amax > 0.0f)) return 0.0f;
    float g = 2688.0f / amax;
    return isfinite(g) ? g : 0.0f;
}

/* Quantize one row of bf16 values y[0..k) ([PROBE] quant_probe):
   for every 16-element block, amax = max |y|; sf = gsf * (amax * (1/6));
   s = E4M3(sf); inv = s ? gsf / dec(s) : 0; code_i = E2M1(y_i * inv).
   Codes are packed with the even column in the low nibble. */
static void quantize_row(const float* y, int64_t k, float gsf,
                         uint8_t* codes_row, uint8_t* scale_bytes) {
    const float rcp6 = f32_from_bits(RCP6_BITS);
    for (int64_t b = 0; b < k / 16; ++b) {
        const float* blk = y + 16 * b;
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) {
            float a = fabsf(blk[i]);
            if (a > amax) amax = a;
        }
        float sf = gsf * (amax * rcp6);
        uint8_t s = e4m3_encode(sf);
        float inv = (s != 0) ? gsf / (float)e4m3_value(s) : 0.0f;
        for (int i = 0; i < 16; i += 2) {
            uint8_t lo = e2m1_encode(blk[i] * inv);
            uint8_t hi = e2m1_encode(blk[i + 1] * inv);
            codes_row[8 * b + i / 2] = (uint8_t)(lo | (hi << 4));
        }
        scale_bytes[b] = s;
    }
}

/* Write a row's linear scale bytes into the swizzled buffer. */
static void place_scales(const uint8_t* scale_bytes, int64_t r, int64_t k, uint8_t* scales) {
    for (int64_t b = 0; b < k / 16; ++b) scales[scale_offset(r, b, k)] = scale_bytes[b];
}

/* ------------------------------------------------------------------------- */
/* RMSNorm statistic: fixed reduction tree (requires k % 512 == 0)           */
/* ------------------------------------------------------------------------- */

/* The row is cut into k/8 chunks of 8 elements.  Lane L (0..63) owns chunks
   L, L+64, L+128, ...; it keeps 8 accumulators, one per position inside a
   chunk, and for its chunks in increasing order adds each square with one
   fused multiply-add.  It then folds its accumulators as
   ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7)).  The 64 lane sums are combined by a
   butterfly: at distance s = 1, 2, 4, 8, 16, 32 every lane adds the value of
   lane L xor s.  ms = sum / k and rstd = 1 / sqrt(ms + eps), IEEE fp32. */
static float rms_rstd(const uint16_t* x, int64_t k, float eps) {
    float lane[64];
    const int64_t chunks = k / 8;
    for (int L = 0; L < 64; ++L) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int64_t c = L; c < chunks; c += 64) {
            for (int e = 0; e < 8; ++e) {
                float v = bf16_to_f32(x[8 * c + e]);
                a[e] = fmaf(v, v, a[e]);
            }
        }
        lane[L] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
    for (int s = 1; s < 64; s *= 2) {
        float next[64];
        for (int L = 0; L < 64; ++L) next[L] = lane[L] + lane[L ^ s];
        memcpy(lane, next, sizeof lane);
    }
    float ms = lane[0] / (float)k;
    return 1.0f / sqrtf(ms + eps);
}

/* ------------------------------------------------------------------------- */
/* exported entry points                                                     */
/* ------------------------------------------------------------------------- */

#define EXPORT __attribute__((visibility("default")))

EXPORT void orc_bf16_round(const float* in, uint16_t* out, int64_t n) {
    unsigned int s = enter_ieee();
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(in[i]);
    leave_ieee(s);
}

EXPORT void orc_e4m3_encode(const float* in, uint8_t* out, int64_t n) {
    unsigned int s = enter_ieee();
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(in[i]);
    leave_ieee(s);
}

EXPORT double orc_e4m3_value(uint8_t code) { return e4m3_value(code); }

EXPORT void orc_e2m1_encode(const float* in, uint8_t* out, int64_t n) {
    unsigned int s = enter_ieee();
    for (int64_t i = 0; i < n; ++i) out[i] = e2m1_encode(in[i]);
    leave_ieee(s);
}

EXPORT double orc_e2m1_value(uint8_t code) { return e2m1_value(code); }

EXPORT int64_t orc_scale_offset(int64_t r, int64_t b, int64_t k) { return scale_offset(r, b, k); }

EXPORT int64_t orc_padded_rows(int64_t m) { return padded_rows(m); }

EXPORT float orc_global_scale(float global_amax) {
    unsigned int s = enter_ieee();
    float g = global_scale(global_amax);
    leave_ieee(s);
    return g;
}

EXPORT float orc_dynamic_global_scale(float amax) {
    unsigned int s = enter_ieee();
    float g = dynamic_global_scale(amax);
    leave_ieee(s);
    return g;
}

/* max |x| over n bf16 values, as fp32 (exact: a maximum of exact values). */
EXPORT float orc_max_abs_bf16(const uint16_t* x, int64_t n) {
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(bf16_to_f32(x[i]));
        if (a > m) m = a;
    }
    return m;
}

EXPORT float orc_rms_rstd(const uint16_t* x, int64_t k, float eps) {
    unsigned int s = enter_ieee();
    float r = rms_rstd(x, k, eps);
    leave_ieee(s);
    return r;
}

/* Quantize n rows given as bf16 patterns (row i is y + i*k).
   codes: [n, k/2]; scale_bytes: [n, k/16] in plain row order. */
EXPORT void orc_quantize_rows(const uint16_t* y, int64_t n, int64_t k, float global_amax,
                              uint8_t* codes, uint8_t* scale_bytes) {
    unsigned int s = enter_ieee();
    float gsf = global_scale(global_amax);
    float* row = (float*)malloc(sizeof(float) * (size_t)k);
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < k; ++i) row[i] = bf16_to_f32(y[r * k + i]);
        quantize_row(row, k, gsf, codes + r * (k / 2), scale_bytes + r * (k / 16));
    }
    free(row);
    leave_ieee(s);
}

/* Standalone quantize of x [m, k] ([H3-API] quantize; [TRT] attention-output
   quantize).  scales is the swizzled [pad(m), k/16] buffer; padding rows are
   written as zero. */
EXPORT void orc_nvfp4_quantize_gsf(const uint16_t* x, int64_t m, int64_t k, float gsf,
                                   uint8_t* codes, uint8_t* scales) {
    unsigned int s = enter_ieee();
    memset(scales, 0, (size_t)(padded_rows(m) * (k / 16)));
    float* row = (float*)malloc(sizeof(float) * (size_t)k);
    uint8_t* sb = (uint8_t*)malloc((size_t)(k / 16));
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t i = 0; i < k; ++i) row[i] = bf16_to_f32(x[r * k + i]);
        quantize_row(row, k, gsf, codes + r * (k / 2), sb);
        place_scales(sb, r, k, scales);
    }
    free(sb);
    free(row);
    leave_ieee(s);
}

EXPORT void orc_nvfp4_quantize(const uint16_t* x, int64_t m, int64_t k, float global_amax,
                               uint8_t* codes, uint8_t* scales) {
    unsigned int s = enter_ieee();
    float gsf = global_scale(global_amax);
    leave_ieee(s);
    orc_nvfp4_quantize_gsf(x, m, k, gsf, codes, scales);
}

/* RMSNorm + adaLN modulation of one row ([TRT] AdaLN RMSNorm + modulation;
   [H3-API] every bf16 rounding kept):
     n   = bf16(x * rstd)          (x: bf16 input, rstd: fp32 statistic)
     nw  = bf16(n * w)
     opl = bf16(1 + scale[t])
     mm  = bf16(nw * opl)
     y   = bf16(mm + shift[t])
   y_row receives the bf16 values as fp32. */
static void rms_adaln_row(const uint16_t* x, const uint16_t* w, const uint16_t* shift_t,
                          const uint16_t* scale_t, int64_t k, float rstd, float* y_row) {
    for (int64_t i = 0; i < k; ++i) {
        float n = rb(bf16_to_f32(x[i]) * rstd);
        float nw = rb(n * bf16_to_f32(w[i]));
        float opl = rb(1.0f + bf16_to_f32(scale_t[i]));
        float mm = rb(nw * opl);
        y_row[i] = rb(mm + bf16_to_f32(shift_t[i]));
    }
}

/* Fused RMSNorm + adaLN -> NVFP4 over rows.
   x: [n, k] bf16 rows (row i is x + i*k), row_ids[i] = the row's index r in the
   full tensor (used only to place scale bytes; pass NULL for r = i).
   frame_idx[i]: the row's frame; table row t of shift / scale is at
   shift + t*frame_stride, scale + t*frame_stride.
   An index outside [0, num_frames) gives all-zero codes and scale bytes, a
   zero y row, and sets bit 0 of *status ([INT64] bounds contract).
   Outputs (any may be NULL except codes):
     codes [n, k/2]; scale_bytes [n, k/16] plain order (or NULL);
     scales: swizzled buffer addressed by row_ids (or NULL);
     rstd [n]; y [n, k] bf16 patterns. */
EXPORT void orc_rms_adaln_rows_gsf(const uint16_t* x, int64_t n, int64_t k, const int64_t* row_ids,
                                   const uint16_t* w, const uint16_t* shift, const uint16_t* scale,
                                   int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                                   float eps, float gsf, uint8_t* codes, uint8_t* scale_bytes,
                                   uint8_t* scales, float* rstd_out, uint16_t* y_out, uint32_t* status) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)k);
    uint8_t* sb = (uint8_t*)malloc((size_t)(k / 16));
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* xr = x + i * k;
        int64_t r = row_ids ? row_ids[i] : i;
        int32_t t = frame_idx[i];
        float rstd = rms_rstd(xr, k, eps);
        if (rstd_out) rstd_out[i] = rstd;
        if (t < 0 || (int64_t)t >= num_frames) {
            memset(codes + i * (k / 2), 0, (size_t)(k / 2));
            memset(sb, 0, (size_t)(k / 16));
            for (int64_t j = 0; j < k; ++j) y[j] = 0.0f;
            if (status) *status |= 1u;
        } else {
            rms_adaln_row(xr, w, shift + (int64_t)t * frame_stride, scale + (int64_t)t * frame_stride,
                          k, rstd, y);
            quantize_row(y, k, gsf, codes + i * (k / 2), sb);
        }
        if (scale_bytes) memcpy(scale_bytes + i * (k / 16), sb, (size_t)(k / 16));
        if (scales) place_scales(sb, r, k, scales);
        if (y_out)
            for (int64_t j = 0; j < k; ++j) y_out[i * k + j] = bf16_round(y[j]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}

/* The same with the global scale of a static amax (2688 / global_amax). */
EXPORT void orc_rms_adaln_rows(const uint16_t* x, int64_t n, int64_t k, const int64_t* row_ids,
                               const uint16_t* w, const uint16_t* shift, const uint16_t* scale,
                               int64_t frame_stride, int64_t num_frames, const int32_t* frame_idx,
                               float eps, float global_amax, uint8_t* codes, uint8_t* scale_bytes,
                               uint8_t* scales, float* rstd_out, uint16_t* y_out, uint32_t* status) {
    unsigned int s = enter_ieee();
    float gsf = global_scale(global_amax);
    leave_ieee(s);
    orc_rms_adaln_rows_gsf(x, n, k, row_ids, w, shift, scale, frame_stride, num_frames, frame_idx, eps, gsf,
                           codes, scale_bytes, scales, rstd_out, y_out, status);
}

/* ------------------------------------------------------------------------- */
/* fp32 residual stream + RMSNorm -> NVFP4                                   */
/* ------------------------------------------------------------------------- */

/* Sum of h^2 over an fp32 row in a fixed tree (the fp32 counterpart of
   rms_rstd's; [H3-API] module summary: the statistic follows a fixed
   reduction order with 4-wide vectors and sequential fused multiply-adds per
   thread, whose order this tree fixes for 64 lanes).  Requires k % 256 == 0.
   The row is cut into quads of 4 consecutive elements; lane L in [0, 64) owns
   quads L, L + 64, L + 128, ... and keeps four accumulators a_e (e = position
   in the quad) starting at +0, updated for its quads in ascending order with
   a_e = fma(v, v, a_e).  Its lane value is (a0 + a1) + (a2 + a3).  The 64
   lane values are combined by the same butterfly as rms_rstd's. */
static float rms_sum_f32(const float* h, int64_t k) {
    float lane[64];
    const int64_t quads = k / 4;
    for (int L = 0; L < 64; ++L) {
        float a[4] = {0, 0, 0, 0};
        for (int64_t q = L; q < quads; q += 64)
            for (int e = 0; e < 4; ++e) a[e] = fmaf(h[4 * q + e], h[4 * q + e], a[e]);
        lane[L] = (a[0] + a[1]) + (a[2] + a[3]);
    }
    for (int s = 1; s < 64; s *= 2) {
        float next[64];
        for (int L = 0; L < 64; ++L) next[L] = lane[L] + lane[L ^ s];
        memcpy(lane, next, sizeof lane);
    }
    return lane[0];
}

EXPORT float orc_rms_sum_f32(const float* h, int64_t k) {
    unsigned int s = enter_ieee();
    float r = rms_sum_f32(h, k);
    leave_ieee(s);
    return r;
}

/* rstd of an fp32 row: 1 / sqrt(sum / k + eps), IEEE fp32. */
static float rms_rstd_f32(const float* h, int64_t k, float eps) {
    float ms = rms_sum_f32(h, k) / (float)k;
    return 1.0f / sqrtf(ms + eps);
}

EXPORT float orc_rms_rstd_f32(const float* h, int64_t k, float eps) {
    unsigned int s = enter_ieee();
    float r = rms_rstd_f32(h, k, eps);
    leave_ieee(s);
    return r;
}

/* Residual add into an fp32 stream, then RMSNorm with an fp32 weight, then
   the NVFP4 quantizer, over rows ([H3-API] residual_norm_quantize).
   h: [n, k] fp32 rows, updated in place when o is given.  For element d of a
   row, with o given:
     t    = bf16(o[d] + bias[d])        (t = o[d] when bias is NULL)
     h[d] = h[d] + fp32(t * scale[d])   (the product rounded, then the add)
   and in every case, on the (updated) row:
     rstd = 1 / sqrt(sum(h^2) / k + eps)   (rms_sum_f32's tree)
     y[d] = bf16((h[d] * rstd) * gamma[d])
   then the block quantizer.  o: [n, k] bf16 or NULL (no residual: h is only
   read); bias: [k] bf16 or NULL; scale, gamma: [k] fp32.  row_ids, codes,
   scale_bytes, scales, rstd_out, y_out as in orc_rms_adaln_rows_gsf. */
EXPORT void orc_residual_rms_rows_gsf(float* h, const uint16_t* o, const uint16_t* bias,
                                      const float* scale, const float* gamma, float eps, int64_t n,
                                      int64_t k, const int64_t* row_ids, float gsf, uint8_t* codes,
                                      uint8_t* scale_bytes, uint8_t* scales, float* rstd_out,
                                      uint16_t* y_out) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)k);
    uint8_t* sb = (uint8_t*)malloc((size_t)(k / 16));
    for (int64_t i = 0; i < n; ++i) {
        float* hr = h + i * k;
        int64_t r = row_ids ? row_ids[i] : i;
        if (o) {
            for (int64_t d = 0; d < k; ++d) {
                uint16_t t = o[i * k + d];
                if (bias) t = bf16_round(bf16_to_f32(t) + bf16_to_f32(bias[d]));
                float prod = bf16_to_f32(t) * scale[d];
                hr[d] = hr[d] + prod;
            }
        }
        float rstd = rms_rstd_f32(hr, k, eps);
        if (rstd_out) rstd_out[i] = rstd;
        for (int64_t d = 0; d < k; ++d) {
            float nrm = hr[d] * rstd;
            y[d] = rb(nrm * gamma[d]);
        }
        quantize_row(y, k, gsf, codes + i * (k / 2), sb);
        if (scale_bytes) memcpy(scale_bytes + i * (k / 16), sb, (size_t)(k / 16));
        if (scales) place_scales(sb, r, k, scales);
        if (y_out)
            for (int64_t d = 0; d < k; ++d) y_out[i * k + d] = bf16_round(y[d]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}

/* The residual add of a DiT block's gated MLP branch carried out by the next
   block's RMSNorm + adaLN producer ([TRT] Summary: the next block's
   normalization performs the MLP branch's residual add, with the gate from the
   current block's AdaLN table and shift and scale from its own),
   over an fp32 residual stream as in orc_residual_rms_rows_gsf.  Row i with
   t = frame_idx[i] in [0, num_frames), element d:
     u    = bf16(o[d] + bias[d])            (u = o[d] when bias is NULL)
     h[d] = h[d] + u * gate_t[d]            fp32: the product rounded, then the add
   with gate_t the row t of the block's own table (gate + t*gate_stride, bf16);
   then on the updated row, with the statistic of rms_sum_f32's tree:
     rstd = 1 / sqrt(sum(h^2) / k + eps)
     n    = bf16(h * rstd)
     nw   = bf16(n * w)
     opl  = bf16(1 + scale_t)
     mm   = bf16(nw * opl)
     y    = bf16(mm + shift_t)
   (shift_t, scale_t: row t of the next block's table, at shift + t*frame_stride,
   scale + t*frame_stride) and the block quantizer.  A row whose index lies
   outside [0, num_frames) is left unchanged in h, gets all-zero codes and
   scale bytes and a zero y row, its rstd is that of the unchanged row, and bit
   0 of *status is set ([INT64] bounds contract).  o may be NULL (no residual
   add); bias may be NULL.  Outputs as in orc_rms_adaln_rows_gsf. */
EXPORT void orc_residual_rms_adaln_rows_gsf(float* h, const uint16_t* o, const uint16_t* bias,
                                            const uint16_t* gate, int64_t gate_stride, const uint16_t* w,
                                            const uint16_t* shift, const uint16_t* scale,
                                            int64_t frame_stride, int64_t num_frames,
                                            const int32_t* frame_idx, float eps, int64_t n, int64_t k,
                                            const int64_t* row_ids, float gsf, uint8_t* codes,
                                            uint8_t* scale_bytes, uint8_t* scales, float* rstd_out,
                                            uint16_t* y_out, uint32_t* status) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)k);
    uint8_t* sb = (uint8_t*)malloc((size_t)(k / 16));
    for (int64_t i = 0; i < n; ++i) {
        float* hr = h + i * k;
        int64_t r = row_ids ? row_ids[i] : i;
        int32_t t = frame_idx[i];
        int ok = t >= 0 && (int64_t)t < num_frames;
        if (ok && o) {
            const uint16_t* gt = gate + (int64_t)t * gate_stride;
            for (int64_t d = 0; d < k; ++d) {
                uint16_t u = o[i * k + d];
                if (bias) u = bf16_round(bf16_to_f32(u) + bf16_to_f32(bias[d]));
                float prod = bf16_to_f32(u) * bf16_to_f32(gt[d]);
                hr[d] = hr[d] + prod;
            }
        }
        float rstd = rms_rstd_f32(hr, k, eps);
        if (rstd_out) rstd_out[i] = rstd;
        if (!ok) {
            memset(codes + i * (k / 2), 0, (size_t)(k / 2));
            memset(sb, 0, (size_t)(k / 16));
            for (int64_t d = 0; d < k; ++d) y[d] = 0.0f;
            if (status) *status |= 1u;
        } else {
            const uint16_t* sh = shift + (int64_t)t * frame_stride;
            const uint16_t* sc = scale + (int64_t)t * frame_stride;
            for (int64_t d = 0; d < k; ++d) {
                float nn = rb(hr[d] * rstd);
                float nw = rb(nn * bf16_to_f32(w[d]));
                float opl = rb(1.0f + bf16_to_f32(sc[d]));
                float mm = rb(nw * opl);
                y[d] = rb(mm + bf16_to_f32(sh[d]));
            }
            quantize_row(y, k, gsf, codes + i * (k / 2), sb);
        }
        if (scale_bytes) memcpy(scale_bytes + i * (k / 16), sb, (size_t)(k / 16));
        if (scales) place_scales(sb, r, k, scales);
        if (y_out)
            for (int64_t d = 0; d < k; ++d) y_out[i * k + d] = bf16_round(y[d]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}

/* ------------------------------------------------------------------------- */
/* channels-last RMSNorm + SiLU -> NVFP4 (fp16)                              */
/* ------------------------------------------------------------------------- */

/* RMS statistic of one channels-last row of c fp16 values (c % 16 == 0,
   c <= 512), the fixed tree of rms_rstd with one 8-element chunk per lane
   over S slots, S = the smallest power of two >= c/8: slot L < c/8 holds the
   lane value ((q0+q1)+(q2+q3))+((q4+q5)+(q6+q7)) of chunk L (q_e = x_e^2,
   exact in fp32), the other slots hold +0, and a butterfly over the S slots
   at distances 1, 2, ..., S/2 combines them into the sum (rms_sum_f16row);
   rstd = 1 / sqrt(sum / c + eps). */
static float rms_sum_f16row(const uint16_t* x, int64_t c) {
    float slot[64];
    int chunks = (int)(c / 8), S = 1;
    while (S < chunks) S *= 2;
    for (int L = 0; L < S; ++L) {
        if (L >= chunks) { slot[L] = 0.0f; continue; }
        float q[8];
        for (int e = 0; e < 8; ++e) {
            float v = f16_to_f32(x[8 * L + e]);
            q[e] = v * v;
        }
        slot[L] = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
    }
    for (int d = 1; d < S; d *= 2) {
        float next[64];
        for (int L = 0; L < S; ++L) next[L] = slot[L] + slot[L ^ d];
        memcpy(slot, next, sizeof(float) * (size_t)S);
    }
    return slot[0];
}

static float rms_rstd_f16row(const uint16_t* x, int64_t c, float eps) {
    return 1.0f / sqrtf(rms_sum_f16row(x, c) / (float)c + eps);
}

EXPORT float orc_rms_sum_f16row(const uint16_t* x, int64_t c) {
    unsigned int s = enter_ieee();
    float r = rms_sum_f16row(x, c);
    leave_ieee(s);
    return r;
}

EXPORT float orc_rms_rstd_f16row(const uint16_t* x, int64_t c, float eps) {
    unsigned int s = enter_ieee();
    float r = rms_rstd_f16row(x, c, eps);
    leave_ieee(s);
    return r;
}

/* RMSNorm (fp32 statistic, fp16 affine) + SiLU -> NVFP4 over channels-last
   rows ([FlashRT] fp16_quant_nvfp4_ndhwc, the fused RMS_norm + SiLU + NVFP4
   variant; the RMSNorm+RoPE kernel's "fp32 stats + fp16 affine").  Row i of
   x [n, c] fp16 (one voxel's channels):
     rstd = rms_rstd_f16row(row)
     nn   = fp16(x * rstd)
     a    = fp16(nn * gamma)               gamma: [c] fp16
     y    = S16[a]                         S16: the fp16 SiLU table
   then the block quantizer over the c channels.  Scale bytes are written in
   plain row order, [n, c/16] (channels-last operand, no GEMM swizzle).
   rstd_out [n], y_out [n, c] fp16, scale_bytes: nullable. */
EXPORT void orc_rms_silu_rows_gsf(const uint16_t* x, const uint16_t* gamma, float eps, int64_t n,
                                  int64_t c, const uint16_t* table, float gsf, uint8_t* codes,
                                  uint8_t* scale_bytes, float* rstd_out, uint16_t* y_out) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)c);
    uint8_t* sb = (uint8_t*)malloc((size_t)(c / 16));
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* xr = x + i * c;
        float rstd = rms_rstd_f16row(xr, c, eps);
        if (rstd_out) rstd_out[i] = rstd;
        for (int64_t d = 0; d < c; ++d) {
            float nn = rh(f16_to_f32(xr[d]) * rstd);
            uint16_t a = f16_round(nn * f16_to_f32(gamma[d]));
            y[d] = f16_to_f32(table[a]);
        }
        quantize_row(y, c, gsf, codes + i * (c / 2), sb);
        if (scale_bytes) memcpy(scale_bytes + i * (c / 16), sb, (size_t)(c / 16));
        if (y_out)
            for (int64_t d = 0; d < c; ++d) y_out[i * c + d] = f16_round(y[d]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}

/* ------------------------------------------------------------------------- */
/* LayerNorm + adaLN -> per-tensor FP8 E4M3 (fp16 input)                     */
/* ------------------------------------------------------------------------- */

/* The fixed tree of rms_rstd over the values v[0..k) of an fp32 row
   (k % 512 == 0): lane L owns chunks L + 64j, 8 accumulators a_e over its
   chunks in ascending order, updated by add(a_e, v) (SUM) or by
   fma(v, v, a_e) (SQUARES); lane value ((a0+a1)+(a2+a3))+((a4+a5)+(a6+a7));
   butterfly over the 64 lanes. */
static float tree_sum_f32(const float* v, int64_t k, int squares) {
    float lane[64];
    const int64_t chunks = k / 8;
    for (int L = 0; L < 64; ++L) {
        float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int64_t c = L; c < chunks; c += 64)
            for (int e = 0; e < 8; ++e) {
                float x = v[8 * c + e];
                a[e] = squares ? fmaf(x, x, a[e]) : a[e] + x;
            }
        lane[L] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
    for (int s = 1; s < 64; s *= 2) {
        float next[64];
        for (int L = 0; L < 64; ++L) next[L] = lane[L] + lane[L ^ s];
        memcpy(lane, next, sizeof lane);
    }
    return lane[0];
}

EXPORT float orc_tree_sum_f32(const float* v, int64_t k, int squares) {
    unsigned int s = enter_ieee();
    float r = tree_sum_f32(v, k, squares);
    leave_ieee(s);
    return r;
}

/* Signed E4M3 (OCP FN) code of an fp32 value: sign bit 7 (-0 -> 0x80), the
   magnitude nearest-even and saturating at 448 (e4m3_encode). */
static uint8_t e4m3_encode_signed(float v) {
    uint8_t sign = signbit(v) ? 0x80u : 0;
    return (uint8_t)(sign | e4m3_encode(fabsf(v)));
}

EXPORT void orc_e4m3_encode_signed(const float* in, uint8_t* out, int64_t n) {
    unsigned int s = enter_ieee();
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode_signed(in[i]);
    leave_ieee(s);
}

/* LayerNorm with fp32 statistics + adaLN modulation, quantized per tensor to
   FP8 E4M3 ([FlashRT] fp16_ada_layernorm_quant_fp8: one pass, fp32 statistics,
   one shared FP8 scale for the three projections that read the result).
   Row i of x [n, k] fp16 (k % 512 == 0), fp32 vectors scale, shift [k]:
     mean = tree_sum(x) / k
     d    = x - mean
     var  = tree_sum_of_squares(d) / k          (fma accumulation)
     rstd = 1 / sqrt(var + eps)
     y    = ((d * rstd) * (1 + scale)) + shift  fp32, each operation rounded
     q    = E4M3(y * inv_scale)                 inv_scale = 1 / act_scale (fp32)
   codes [n, k] (one byte each); mean_out, rstd_out [n], y_out [n, k] fp32:
   nullable. */
EXPORT void orc_ln_adaln_fp8_rows(const uint16_t* x, const float* scale, const float* shift, float eps,
                                  int64_t n, int64_t k, float inv_scale, uint8_t* codes,
                                  float* mean_out, float* rstd_out, float* y_out) {
    unsigned int s = enter_ieee();
    float* v = (float*)malloc(sizeof(float) * (size_t)k);
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* xr = x + i * k;
        for (int64_t d = 0; d < k; ++d) v[d] = f16_to_f32(xr[d]);
        float mean = tree_sum_f32(v, k, 0) / (float)k;
        for (int64_t d = 0; d < k; ++d) v[d] = v[d] - mean;
        float var = tree_sum_f32(v, k, 1) / (float)k;
        float rstd = 1.0f / sqrtf(var + eps);
        if (mean_out) mean_out[i] = mean;
        if (rstd_out) rstd_out[i] = rstd;
        for (int64_t d = 0; d < k; ++d) {
            float xh = v[d] * rstd;
            float opl = 1.0f + scale[d];
            float m = xh * opl;
            float y = m + shift[d];
            if (y_out) y_out[i * k + d] = y;
            codes[i * k + d] = e4m3_encode_signed(y * inv_scale);
        }
    }
    free(v);
    leave_ieee(s);
}

/* The quantizer's inverse scale of a per-tensor scale: 1 / act_scale (fp32). */
EXPORT float orc_fp8_inverse_scale(float act_scale) {
    unsigned int s = enter_ieee();
    float r = 1.0f / act_scale;
    leave_ieee(s);
    return r;
}

/* The per-call scale of the FP8 producer: act_scale = amax / 448 (fp32), 0 when
   amax is 0; the inverse scale is then 1 / act_scale, or 0 when act_scale is 0
   or the reciprocal overflows (every code a signed zero). */
EXPORT float orc_fp8_dynamic_scale(float amax) {
    unsigned int s = enter_ieee();
    float r = amax / 448.0f;
    leave_ieee(s);
    return r;
}

EXPORT float orc_fp8_dynamic_inverse(float act_scale) {
    unsigned int s = enter_ieee();
    float r = 0.0f;
    if (act_scale > 0.0f) {
        r = 1.0f / act_scale;
        if (isinf(r)) r = 0.0f;
    }
    leave_ieee(s);
    return r;
}

/* ------------------------------------------------------------------------- */
/* SiLU table and the SwiGLU producer                                        */
/* ------------------------------------------------------------------------- */

/* Round the real number hi + lo (|lo| far below half a bf16 ulp of hi) to the
   nearest bf16, ties to even.  lo only decides the direction when hi lies
   exactly on a rounding midpoint.  Values so close to a midpoint that the long
   double evaluation cannot decide them are counted in *ambiguous.
   bf16 has the fp32 exponent range: quantum 2^(E-7) for 2^E <= |v| < 2^(E+1),
   E >= -126, and the subnormal quantum 2^-133 below 2^-126. */
static uint16_t ld_to_bf16(long double hi, long double lo, int* ambiguous) {
    uint16_t sign = signbit(hi) ? 0x8000u : 0;
    long double a = fabsl(hi);
    if (a == 0.0L) return sign;
    int e2;
    frexpl(a, &e2);                         /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                         /* 2^E <= a < 2^(E+1)          */
    int qexp = (E < -126) ? -133 : E - 7;
    long double n = ldexpl(a, -qexp);       /* exact power-of-two scaling  */
    long double fl = floorl(n);
    long double frac = n - fl;
    int up;
    if (frac == 0.5L && lo != 0.0L) {
        up = (signbit(lo) == signbit(hi));  /* lo pushes the magnitude up or down */
    } else {
        if (fabsl(frac - 0.5L) < 0x1p-40L) (*ambiguous)++;
        up = frac > 0.5L || (frac == 0.5L && fmodl(fl, 2.0L) == 1.0L);
    }
    long double r = up ? fl + 1.0L : fl;
    float value = (float)ldexpl(r, qexp);   /* <= 9 significant bits: exact, or inf */
    return (uint16_t)(sign | (bits_from_f32(value) >> 16));
}

/* S[g] = bf16(g * sigmoid(g)) = bf16(g / (1 + e^-g)) for every bf16 pattern g,
   evaluated in x87 long double and rounded once ([H3-API] swiglu_quantize's
   SiLU table).  For |g| < 2^-30 the value is written as g/2 + (g/2) tanh(g/2):
   there e^-g rounds to 1 and g/2 can sit exactly on a bf16 midpoint (odd
   subnormal multiples), which the tanh term, always of the sign of g^2 > 0,
   decides.  -inf -> -0, +inf -> +inf, NaN -> 0x7FC0.  Returns the number of
   entries too close to a midpoint to be decided (expected 0). */
EXPORT int orc_silu_table(uint16_t* table) {
    unsigned int s = enter_ieee();
    int ambiguous = 0;
    for (uint32_t g = 0; g < 65536u; ++g) {
        uint32_t exp_field = (g >> 7) & 0xFFu;
        uint32_t mant = g & 0x7Fu;
        if (exp_field == 0xFFu) {
            if (mant != 0) table[g] = 0x7FC0u;
            else table[g] = (g & 0x8000u) ? 0x8000u : 0x7F80u;
            continue;
        }
        long double x = (long double)bf16_to_f32((uint16_t)g);
        long double hi, lo;
        if (fabsl(x) < 0x1p-30L) {
            hi = x / 2.0L;
            lo = hi * tanhl(hi);
        } else {
            hi = x / (1.0L + expl(-x));
            lo = 0.0L;
        }
        table[g] = ld_to_bf16(hi, lo, &ambiguous);
    }
    leave_ieee(s);
    return ambiguous;
}

/* Round the real hi + lo to the nearest fp16, ties to even (as ld_to_bf16,
   with fp16's quantum: 2^(E-10) for 2^E <= |v| < 2^(E+1), E >= -14, and the
   subnormal quantum 2^-24; from 65520 up: infinity). */
static uint16_t ld_to_f16(long double hi, long double lo, int* ambiguous) {
    uint16_t sign = signbit(hi) ? 0x8000u : 0;
    long double a = fabsl(hi);
    if (a == 0.0L) return sign;
    if (a >= 65520.0L) return (uint16_t)(sign | 0x7C00u);   /* no value sits near 65520 */
    int e2;
    frexpl(a, &e2);
    int E = e2 - 1;
    int qexp = (E < -14) ? -24 : E - 10;
    long double n = ldexpl(a, -qexp);
    long double fl = floorl(n);
    long double frac = n - fl;
    int up;
    if (frac == 0.5L && lo != 0.0L) {
        up = (signbit(lo) == signbit(hi));
    } else {
        if (fabsl(frac - 0.5L) < 0x1p-40L) (*ambiguous)++;
        up = frac > 0.5L || (frac == 0.5L && fmodl(fl, 2.0L) == 1.0L);
    }
    long double r = up ? fl + 1.0L : fl;
    return (uint16_t)(sign | f16_round((float)ldexpl(r, qexp)));   /* exact: <= 11 bits */
}

/* S16[g] = fp16(g * sigmoid(g)) for every fp16 pattern g, as orc_silu_table
   does for bf16 (long double, one rounding; |g| < 2^-30 through the tanh
   form).  -inf -> -0, +inf -> +inf, NaN -> 0x7E00.  Returns the number of
   entries too close to a midpoint to decide (expected 0). */
EXPORT int orc_silu_table_f16(uint16_t* table) {
    unsigned int s = enter_ieee();
    int ambiguous = 0;
    for (uint32_t g = 0; g < 65536u; ++g) {
        uint32_t exp_field = (g >> 10) & 0x1Fu;
        uint32_t mant = g & 0x3FFu;
        if (exp_field == 0x1Fu) {
            if (mant != 0) table[g] = 0x7E00u;
            else table[g] = (g & 0x8000u) ? 0x8000u : 0x7C00u;
            continue;
        }
        long double x = (long double)f16_to_f32((uint16_t)g);
        long double hi, lo;
        if (fabsl(x) < 0x1p-30L) {
            hi = x / 2.0L;
            lo = hi * tanhl(hi);
        } else {
            hi = x / (1.0L + expl(-x));
            lo = 0.0L;
        }
        table[g] = ld_to_f16(hi, lo, &ambiguous);
    }
    leave_ieee(s);
    return ambiguous;
}

EXPORT void orc_f16_round(const float* in, uint16_t* out, int64_t n) {
    unsigned int s = enter_ieee();
    for (int64_t i = 0; i < n; ++i) out[i] = f16_round(in[i]);
    leave_ieee(s);
}

/* SwiGLU -> NVFP4 over rows ([H3-API] swiglu_quantize; [TRT] SiLU-and-mul
   producer):  y = bf16(S[gate] * up), then the block quantizer.
   up / gate rows are ld elements apart (row i at up + i*ld, gate + i*ld);
   f output columns.  table: the 65536-entry SiLU table from orc_silu_table.
   row_ids / scales / scale_bytes / y_out as in orc_rms_adaln_rows. */
EXPORT void orc_swiglu_rows_gsf(const uint16_t* up, const uint16_t* gate, int64_t ld, int64_t n,
                                int64_t f, const int64_t* row_ids, const uint16_t* table,
                                float gsf, uint8_t* codes, uint8_t* scale_bytes,
                                uint8_t* scales, uint16_t* y_out) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)f);
    uint8_t* sb = (uint8_t*)malloc((size_t)(f / 16));
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = row_ids ? row_ids[i] : i;
        for (int64_t j = 0; j < f; ++j) {
            float silu = bf16_to_f32(table[gate[i * ld + j]]);
            y[j] = rb(silu * bf16_to_f32(up[i * ld + j]));
        }
        quantize_row(y, f, gsf, codes + i * (f / 2), sb);
        if (scale_bytes) memcpy(scale_bytes + i * (f / 16), sb, (size_t)(f / 16));
        if (scales) place_scales(sb, r, f, scales);
        if (y_out)
            for (int64_t j = 0; j < f; ++j) y_out[i * f + j] = bf16_round(y[j]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}

/* The same with the global scale of a static amax (2688 / global_amax). */
EXPORT void orc_swiglu_rows(const uint16_t* up, const uint16_t* gate, int64_t ld, int64_t n,
                            int64_t f, const int64_t* row_ids, const uint16_t* table,
                            float global_amax, uint8_t* codes, uint8_t* scale_bytes,
                            uint8_t* scales, uint16_t* y_out) {
    unsigned int s = enter_ieee();
    float gsf = global_scale(global_amax);
    leave_ieee(s);
    orc_swiglu_rows_gsf(up, gate, ld, n, f, row_ids, table, gsf, codes, scale_bytes, scales, y_out);
}

/* SwiGLU -> NVFP4 of a packed projection with an optional bias ([H3-API]
   swiglu_quantize: o [M, 2F] holds the value half first and arrives without
   its bias;
   [branch compare] quant_probe: the paired layout with the value of output
   column j at projection column 2j and its gate at 2j + 1).  Row i of the
   projection starts at proj + i*ld.  For output column j:
     interleaved == 0:  value column j,      gate column F + j
     interleaved == 1:  value column 2j,     gate column 2j + 1
   bias (NULL: none) is one bf16 row of 2F entries in the projection's own
   column order.  The bias add is a bf16 tensor add: each of value and gate
   becomes bf16(o + bias) at its column (as residual_norm_quantize's bf16(o +
   bias) on the same page), and then y = bf16(S[gate] * value), the block
   quantizer and the layout as in orc_swiglu_rows_gsf. */
EXPORT void orc_swiglu_packed_rows_gsf(const uint16_t* proj, const uint16_t* bias, int interleaved,
                                       int64_t ld, int64_t n, int64_t f, const int64_t* row_ids,
                                       const uint16_t* table, float gsf, uint8_t* codes,
                                       uint8_t* scale_bytes, uint8_t* scales, uint16_t* y_out) {
    unsigned int s = enter_ieee();
    float* y = (float*)malloc(sizeof(float) * (size_t)f);
    uint8_t* sb = (uint8_t*)malloc((size_t)(f / 16));
    for (int64_t i = 0; i < n; ++i) {
        int64_t r = row_ids ? row_ids[i] : i;
        const uint16_t* row = proj + i * ld;
        for (int64_t j = 0; j < f; ++j) {
            int64_t vc = interleaved ? 2 * j : j;          /* value column */
            int64_t gc = interleaved ? 2 * j + 1 : f + j;  /* gate column  */
            uint16_t v = row[vc], g = row[gc];
            if (bias) {
                v = bf16_round(bf16_to_f32(v) + bf16_to_f32(bias[vc]));
                g = bf16_round(bf16_to_f32(g) + bf16_to_f32(bias[gc]));
            }
            y[j] = rb(bf16_to_f32(table[g]) * bf16_to_f32(v));
        }
        quantize_row(y, f, gsf, codes + i * (f / 2), sb);
        if (scale_bytes) memcpy(scale_bytes + i * (f / 16), sb, (size_t)(f / 16));
        if (scales) place_scales(sb, r, f, scales);
        if (y_out)
            for (int64_t j = 0; j < f; ++j) y_out[i * f + j] = bf16_round(y[j]);
    }
    free(sb);
    free(y);
    leave_ieee(s);
}
