/*
 * Oracle: container rounding (BF16, FP8-e4m3, INT8), the FP8/INT8 route
 * pre-cast and the reported metrics.  TEST INFRASTRUCTURE ONLY (see epo.h).
 *
 * Passages followed:
 *  - EntroPack paper, section 3.1 and Figure 2(b): decoding ends with row
 *    rescaling and dtype conversion; the abstract and appendix A.6: BF16,
 *    FP16, FP8 and INT8 containers with the storage rate independent of the
 *    numeric precision.
 *  - Appendix B.1: weights are first converted to row-scaled FP8 or INT8, then
 *    compressed, and reconstructed in that format.  The per-row scale is not
 *    printed; this oracle uses max|W_r| / 448 (FP8-e4m3 largest finite value)
 *    and max|W_r| / 127 (INT8, symmetric).
 *  - EntroPackPreQuants model card: bpp = 8 * sum(storage bytes) / sum(numel);
 *    weight error = sqrt(sum ||Wq - W||^2) / sqrt(sum ||W||^2).
 *
 * Rounding (readings where the pages are silent): BF16 = round-to-nearest-even
 * of the fp32 value; FP8 = OCP e4m3fn (bias 7, no infinities, largest finite
 * 448, subnormals kept), value clamped to [-448, 448] then rounded to nearest
 * even; INT8 = round half to even, then clamp to [-128, 127].  Signed zeros
 * keep their sign in BF16 and FP8.
 */
#include <math.h>
#include <string.h>

#include "epo.h"

static double rint_even(double x) {
  double f = floor(x);
  double d = x - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

uint16_t epo_f32_to_bf16(float y) {
  uint32_t u;
  memcpy(&u, &y, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  /* keep the upper 16 bits, rounding the dropped 16 bits to nearest, ties to even */
  uint32_t lower = u & 0xFFFFu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
  return (uint16_t)upper;
}

/* Value of an e4m3fn code (used by the FP8 route and by tests). */
double epo_fp8e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);                 /* subnormal: m * 2^-9 */
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

uint8_t epo_f32_to_fp8e4m3(float yf) {
  double y = (double)yf;
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs(y);
  if (a > 448.0) a = 448.0;
  /* quantum of the binade that a falls in (subnormal quantum below 2^-6) */
  double q;
  if (a >= ldexp(1.0, -6)) {
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) -> floor(log2 a) = e - 1 */
    q = ldexp(1.0, (e - 1) - 3);
  } else {
    q = ldexp(1.0, -9);
  }
  double r = rint_even(a / q) * q;   /* exact: a / q is a scaling by a power of two */
  if (r > 448.0) r = 448.0;          /* cannot happen after the clamp; kept for clarity */
  if (r == 0.0) return sign;
  int e;
  frexp(r, &e);
  int ex = e - 1;                    /* r in [2^ex, 2^(ex+1)) */
  uint8_t code;
  if (ex >= -6) {
    int mant = (int)((r / ldexp(1.0, ex) - 1.0) * 8.0);
    code = (uint8_t)(((ex + 7) << 3) | mant);
  } else {
    code = (uint8_t)(r / ldexp(1.0, -9));   /* subnormal: exponent field 0 */
  }
  return (uint8_t)(sign | code);
}

/* IEEE binary16, round to nearest even: the value is rounded at the quantum of
 * its binade (2^(e-10); subnormal quantum 2^-24 below 2^-14); a result of 2^16
 * or more overflows to infinity (largest finite 65504). */
uint16_t epo_f32_to_f16(float yf) {
  double y = (double)yf;
  uint16_t sign = signbit(y) ? 0x8000u : 0u;
  if (isnan(y)) return (uint16_t)(sign | 0x7E00u);
  double a = fabs(y);
  if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
  double q;
  if (a >= ldexp(1.0, -14)) {
    int e;
    frexp(a, &e);                       /* floor(log2 a) = e - 1 */
    q = ldexp(1.0, (e - 1) - 10);
  } else {
    q = ldexp(1.0, -24);
  }
  double r = rint_even(a / q) * q;
  if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u);
  if (r == 0.0) return sign;
  int e;
  frexp(r, &e);
  int E = e - 1;                        /* r = 1.m * 2^E after rounding */
  if (E < -14) return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
  uint16_t m = (uint16_t)((r / ldexp(1.0, E) - 1.0) * 1024.0);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | m);
}

void epo_f32_to_f16_batch(const float* y, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = epo_f32_to_f16(y[i]);
}

int8_t epo_f32_to_int8(float yf) {
  double r = rint_even((double)yf);
  if (r > 127.0) r = 127.0;
  if (r < -128.0) r = -128.0;
  return (int8_t)r;
}

/* UINT8 container (paper, appendix A.6: unsigned integer dtypes carry an
 * offset): the integer nearest y (ties to even) moved up by 128, then clamped
 * to the unsigned byte range [0, 255]. */
uint8_t epo_f32_to_uint8(float yf) {
  double u = rint_even((double)yf) + 128.0;
  if (u > 255.0) u = 255.0;
  if (u < 0.0) u = 0.0;
  return (uint8_t)u;
}

void epo_f32_to_uint8_batch(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = epo_f32_to_uint8(y[i]);
}

void epo_f32_to_bf16_batch(const float* y, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = epo_f32_to_bf16(y[i]);
}
void epo_f32_to_fp8e4m3_batch(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = epo_f32_to_fp8e4m3(y[i]);
}
void epo_f32_to_int8_batch(const float* y, int64_t n, int8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = epo_f32_to_int8(y[i]);
}

/* Row-scaled FP8 / INT8 pre-cast.  Wq receives the values of the codes (what
 * EntroPack then compresses), qscale the per-row scale (fp32). */
void epo_route_precast(const float* W, int64_t rows, int64_t cols, int route, float* Wq,
                       float* qscale) {
  for (int64_t r = 0; r < rows; ++r) {
    float amax = 0.0f;
    for (int64_t c = 0; c < cols; ++c) {
      float a = fabsf(W[r * cols + c]);
      if (a > amax) amax = a;
    }
    float q = (route == EPO_ROUTE_FP8) ? amax / 448.0f : amax / 127.0f;
    qscale[r] = q;
    for (int64_t c = 0; c < cols; ++c) {
      float v;
      if (q == 0.0f) {
        v = 0.0f;
      } else {
        float y = W[r * cols + c] / q;
        if (route == EPO_ROUTE_FP8) {
          v = (float)epo_fp8e4m3_value(epo_f32_to_fp8e4m3(y));
        } else {
          double t = rint_even((double)y);
          if (t > 127.0) t = 127.0;
          if (t < -127.0) t = -127.0;
          v = (float)t;
        }
      }
      Wq[r * cols + c] = v;
    }
  }
}

double epo_bpp(const uint64_t* stored_bytes, const uint64_t* numel, int n) {
  double b = 0.0, e = 0.0;
  for (int i = 0; i < n; ++i) {
    b += (double)stored_bytes[i];
    e += (double)numel[i];
  }
  return e > 0.0 ? 8.0 * b / e : 0.0;
}

double epo_rel_l2(const float* Wq, const float* W, int64_t n) {
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double d = (double)Wq[i] - (double)W[i];
    num += d * d;
    den += (double)W[i] * (double)W[i];
  }
  return den > 0.0 ? sqrt(num) / sqrt(den) : 0.0;
}
