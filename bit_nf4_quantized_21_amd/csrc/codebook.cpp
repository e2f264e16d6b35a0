// Host-side construction of the 4-bit decode tables: the NF4 codebook and
// the two 4-bit types the pages compare NF4 with (news write-up, innovations
// list: NF4 gives better results than 4-bit integers and 4-bit floats).
//
// NF4 is the 4-bit data type that is information-theoretically optimal for
// normally distributed weights ("QLoRA: Efficient Finetuning of Quantized
// LLMs", Abstract item (a)): its 16 values are quantiles of the standard
// normal distribution, normalised to [-1, 1] with an exact zero.  The pages
// do not spell out the construction; the library takes 8 positive quantiles
// at probabilities p_max - j (p_max - 1/2)/8 (j = 0..7), 7 negative ones at
// p_max - j (p_max - 1/2)/7 (j = 0..6) mirrored, and 0, with
// p_max = 1 - (1/30 + 1/32)/2, divides by the quantile at p_max and rounds
// the sorted values to fp32.
//
// The inverse normal CDF here is this library's own: a rational first guess
// refined by Halley steps on erfc from the C library, accurate to about one
// fp64 ulp.
#include <algorithm>
#include <cmath>
#include <utility>

#include "codebook.hpp"

namespace qlora {

static double rational_guess(double p) {
  // P. J. Acklam's piecewise rational approximation of the normal quantile
  // (relative error about 1e-9); the Halley steps below make it exact to
  // fp64 rounding.
  static const double a[6] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                              1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[5] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                              6.680131188771972e+01, -1.328068155288572e+01};
  static const double c[6] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                              -2.549732539343734e+00, 4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[4] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                              3.754408661907416e+00};
  const double plow = 0.02425, phigh = 1.0 - plow;
  if (p < plow) {
    double q = std::sqrt(-2.0 * std::log(p));
    return (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  if (p > phigh) {
    double q = std::sqrt(-2.0 * std::log(1.0 - p));
    return -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
           ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1.0);
  }
  double q = p - 0.5, r = q * q;
  return (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
         (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1.0);
}

double normal_quantile(double p) {
  double x = rational_guess(p);
  const double sqrt2 = 1.4142135623730950488, sqrt2pi = 2.5066282746310005024;
  for (int it = 0; it < 3; ++it) {
    // Phi(x) - p with Phi(x) = erfc(-x/sqrt2)/2; Halley step.
    double e = 0.5 * std::erfc(-x / sqrt2) - p;
    double u = e * sqrt2pi * std::exp(0.5 * x * x);
    x = x - u / (1.0 + 0.5 * x * u);
  }
  return x;
}

void build_codebook(float out[16]) {
  const double pmax = 1.0 - (1.0 / 30.0 + 1.0 / 32.0) / 2.0;
  const double step_pos = (pmax - 0.5) / 8.0;
  const double step_neg = (pmax - 0.5) / 7.0;
  const double top = normal_quantile(pmax);
  double v[16];
  int n = 0;
  for (int j = 0; j < 8; ++j) v[n++] = normal_quantile(pmax - j * step_pos) / top;
  for (int j = 0; j < 7; ++j) v[n++] = -normal_quantile(pmax - j * step_neg) / top;
  v[n++] = 0.0;
  std::sort(v, v + 16);
  for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
}

// Int4: code = k mod 16 (4-bit two's complement), value k / 7 rounded to
// fp32, k = -7..7 (symmetric absmax scaling; code 8, k = -8, is never
// produced and decodes to -8/7).  FP4: OCP E2M1, code = sign << 3 |
// exponent << 1 | mantissa with exponent bias 1 (subnormal when the exponent
// field is 0), magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 divided by 6 so that
// the largest is 1, rounded to fp32 (code 8, -0, is never produced).
void build_type_table(int qtype, float out[16]) {
  if (qtype == kQNF4) {
    build_codebook(out);
    return;
  }
  for (int c = 0; c < 16; ++c) {
    if (qtype == kQINT4) {
      const int k = c < 8 ? c : c - 16;
      out[c] = (float)(k / 7.0);
    } else {
      const int e = (c >> 1) & 3, m = c & 1;
      const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
      const float v = (float)(mag / 6.0);
      out[c] = (c & 8) ? -v : v;
    }
  }
}

void build_type_levels(int qtype, const float table[16], TypeLevels* out) {
  int n = 0;
  for (int c = 0; c < 16; ++c) {
    if (qtype != kQNF4 && c == 8) continue;  // never produced
    out->level[n] = table[c];
    out->code[n] = (uint32_t)c;
    ++n;
  }
  // insertion sort by value (16 entries)
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && out->level[j - 1] > out->level[j]; --j) {
      std::swap(out->level[j - 1], out->level[j]);
      std::swap(out->code[j - 1], out->code[j]);
    }
  out->n = n;
  out->zero_code = 0;
  for (int i = 0; i < n; ++i)
    if (out->level[i] == 0.0f) {
      out->zero_code = out->code[i];
      break;
    }
}

}  // namespace qlora
