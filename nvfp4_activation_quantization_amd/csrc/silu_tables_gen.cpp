// silu_tables_gen.cpp -- build-time generator of the library's two SiLU tables (a host
// program run by build.py; not part of libnvfp4act.so).  For every 16-bit pattern g:
//   bf16 table: S[g] = bf16(g * sigmoid(g)) of the bf16 value g   (the SwiGLU producer)
//   fp16 table: S[g] = fp16(g * sigmoid(g)) of the fp16 value g   (the VAE RMSNorm + SiLU)
// rounded to nearest, ties to even, from an fp64 evaluation: hi = x / (1 + exp(-x)); for
// |x| < 2^-30, where exp(-x) rounds to 1 and x/2 may sit exactly on a midpoint, hi = x/2
// and lo = (x/2)^2 (silu(x) = x/2 + (x/2) tanh(x/2), the second term ~ (x/2)^2 > 0 decides
// that tie).  A value within 2^-36 quanta of a midpoint is not decidable from fp64: the
// generator then stops with an error instead of guessing.  NaN -> the format's quiet NaN,
// +inf -> +inf, -inf -> -0 (the limit of x * sigmoid(x)).
//
// Usage: silu_tables_gen <bf16 output> <fp16 output>; each output is the comma-separated
// initializer of a 65,536-entry uint16_t array.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace {

int g_undecided = 0;

// Round hi + lo to a format with `mant` explicit mantissa bits and minimum normal exponent
// emin (quantum 2^(e - mant) for 2^e <= |v|, 2^(emin - mant) below 2^emin).
double round_nearest_even(double hi, double lo, int mant, int emin) {
  const double a = std::fabs(hi);
  if (a == 0.0) return hi;
  const int e = std::ilogb(a);
  const int qexp = (e < emin ? emin : e) - mant;
  const double n = std::ldexp(a, -qexp);   // exact: a power-of-two scaling
  const double fl = std::floor(n);
  const double frac = n - fl;
  bool up;
  if (frac == 0.5 && lo != 0.0) {
    up = (lo > 0.0) == (hi > 0.0);
  } else {
    if (std::fabs(frac - 0.5) < 0x1p-36) ++g_undecided;
    up = frac > 0.5 || (frac == 0.5 && std::fmod(fl, 2.0) == 1.0);
  }
  const double mag = std::ldexp(up ? fl + 1.0 : fl, qexp);
  return std::signbit(hi) ? -mag : mag;
}

void silu_parts(double x, double* hi, double* lo) {
  if (std::fabs(x) < 0x1p-30) {
    *hi = 0.5 * x;
    *lo = *hi * *hi;
  } else {
    *hi = x / (1.0 + std::exp(-x));
    *lo = 0.0;
  }
}

uint16_t bf16_entry(uint32_t g) {
  const uint32_t ex = (g >> 7) & 0xFFu, mant = g & 0x7Fu;
  if (ex == 0xFFu) return mant ? 0x7FC0u : ((g & 0x8000u) ? 0x8000u : 0x7F80u);
  uint32_t bits = g << 16;
  float xf;
  std::memcpy(&xf, &bits, 4);
  double hi, lo;
  silu_parts((double)xf, &hi, &lo);
  const double r = round_nearest_even(hi, lo, 7, -126);   // at most 8 significant bits
  const float rf = (float)r;                                // exact
  if (rf == 0.0f) return std::signbit(rf) ? 0x8000u : 0u;
  std::memcpy(&bits, &rf, 4);
  return (uint16_t)(bits >> 16);
}

uint16_t f16_entry(uint32_t g) {
  const uint32_t ex = (g >> 10) & 0x1Fu, mant = g & 0x3FFu;
  if (ex == 0x1Fu) return mant ? 0x7E00u : ((g & 0x8000u) ? 0x8000u : 0x7C00u);
  // fp16 value: (-1)^s * 2^(ex-15) * (1 + mant/1024), or 2^-14 * mant/1024 for ex == 0
  const double mag = ex ? std::ldexp(1.0 + mant / 1024.0, (int)ex - 15) : std::ldexp(mant / 1024.0, -14);
  const double x = (g & 0x8000u) ? -mag : mag;
  double hi, lo;
  silu_parts(x, &hi, &lo);
  const double r = round_nearest_even(hi, lo, 10, -14);
  const uint16_t sign = std::signbit(r) ? 0x8000u : 0u;
  const double a = std::fabs(r);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return sign | 0x7C00u;                  // rounds to infinity
  const int e = std::ilogb(a);
  if (e < -14) return sign | (uint16_t)std::ldexp(a, 24);   // subnormal: a multiple of 2^-24
  const double frac = std::ldexp(a, -e) - 1.0;               // in [0, 1), a multiple of 2^-10
  if (e > 15) return sign | 0x7C00u;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)std::ldexp(frac, 10);
}

bool write_table(const char* path, uint16_t (*entry)(uint32_t)) {
  FILE* f = std::fopen(path, "w");
  if (!f) return false;
  for (uint32_t g = 0; g < 65536u; ++g) std::fprintf(f, "0x%04x,%s", entry(g), (g % 12 == 11) ? "\n" : "");
  std::fprintf(f, "\n");
  return std::fclose(f) == 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <bf16 table out> <fp16 table out>\n", argv[0]);
    return 2;
  }
  if (!write_table(argv[1], bf16_entry) || !write_table(argv[2], f16_entry)) {
    std::fprintf(stderr, "silu_tables_gen: cannot write the tables\n");
    return 1;
  }
  if (g_undecided != 0) {
    std::fprintf(stderr, "silu_tables_gen: %d entries lie too close to a rounding midpoint for fp64\n", g_undecided);
    return 1;
  }
  return 0;
}
