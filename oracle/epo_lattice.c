/*
 * Oracle: row normalisation, nearest E8 point and the invertible integer
 * fields.  TEST INFRASTRUCTURE ONLY (see epo.h).
 *
 * Passages followed:
 *  - EntroPack paper, section 1 and section 3.2 ("Row-normalized lattice
 *    representation"): rows are normalised, blocks of eight normalised weights
 *    are quantised onto E8 and represented as invertible integer fields.  The
 *    normalising statistic is not printed; this oracle uses the row RMS.
 *  - Conway & Sloane (1982), "Fast quantizing and decoding algorithms for
 *    lattice quantizers and codes" (reference 7 of the paper): the nearest
 *    point of D_n rounds every coordinate and, if the coordinate sum is odd,
 *    re-rounds the coordinate with the largest rounding error the other way;
 *    E8 = D8 u (D8 + 1/2) takes the nearer of the two coset answers.
 *  - Paper, appendix A.3 (entropy-model ablation): the coded fields are
 *    (c, z1..z7, m); m replaces z8 by exploiting the even-sum constraint
 *    ("parity reduction").  The equation itself is not printed; this oracle
 *    uses m = floor(z8 / 2), the one-bit reduction that z8's parity (fixed by
 *    z1..z7) makes invertible.
 */
#include <math.h>
#include <string.h>

#include "epo.h"

/* Round to the nearest integer, ties to even.  Written out instead of relying
 * on the floating-point environment. */
static double round_half_even(double x) {
  double f = floor(x);
  double d = x - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  /* exact tie */
  return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

void epo_round_half_even(const double* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_half_even(x[i]);
}

/* Nearest point of D8 = {y in Z^8 : sum y even} (Conway & Sloane).
 * Ties in the rounding go to even; ties in "largest rounding error" go to the
 * lowest coordinate index. */
void epo_d8_nearest(const double v[8], double y[8]) {
  int64_t sum = 0;
  int worst = 0;
  double worst_err = -1.0;
  for (int i = 0; i < 8; ++i) {
    y[i] = round_half_even(v[i]);
    sum += (int64_t)y[i];
    double err = fabs(v[i] - y[i]);
    if (err > worst_err) {
      worst_err = err;
      worst = i;
    }
  }
  if (sum % 2 != 0) y[worst] += (v[worst] >= y[worst]) ? 1.0 : -1.0;
}

/* Nearest point of E8 = D8 u (D8 + 1/2).  Returns the coset bit c (0: integer
 * coordinates, 1: half-integer coordinates).  Distance ties go to coset 0. */
int epo_e8_nearest(const double v[8], double x[8]) {
  double y0[8], w[8], y1[8];
  epo_d8_nearest(v, y0);
  for (int i = 0; i < 8; ++i) w[i] = v[i] - 0.5;
  epo_d8_nearest(w, y1);
  for (int i = 0; i < 8; ++i) y1[i] += 0.5;
  double d0 = 0.0, d1 = 0.0;
  for (int i = 0; i < 8; ++i) {
    d0 += (v[i] - y0[i]) * (v[i] - y0[i]);
    d1 += (v[i] - y1[i]) * (v[i] - y1[i]);
  }
  if (d0 <= d1) {
    memcpy(x, y0, sizeof(y0));
    return 0;
  }
  memcpy(x, y1, sizeof(y1));
  return 1;
}

void epo_e8_nearest_batch(const double* v, int64_t nvec, double* x, int32_t* coset) {
  for (int64_t g = 0; g < nvec; ++g) {
    int c = epo_e8_nearest(v + 8 * g, x + 8 * g);
    if (coset) coset[g] = c;
  }
}

/* E8 point -> fields (c, z1..z7, m).  z = x - c/2 lies in D8. */
void epo_point_to_fields(const double x[8], int32_t fields[9]) {
  /* the point is in the half-integer coset iff its first coordinate is not an integer */
  int c = (floor(x[0]) != x[0]) ? 1 : 0;
  int32_t z[8];
  for (int i = 0; i < 8; ++i) z[i] = (int32_t)(x[i] - 0.5 * c);
  fields[0] = c;
  for (int i = 0; i < 7; ++i) fields[1 + i] = z[i];
  /* m = floor(z8 / 2) */
  fields[8] = (int32_t)floor((double)z[7] / 2.0);
}

/* Inverse: z8 = 2m + parity(z1 + ... + z7), x = z + c/2. */
void epo_fields_to_point(const int32_t fields[9], double x[8]) {
  int c = fields[0];
  int64_t s7 = 0;
  for (int i = 0; i < 7; ++i) s7 += fields[1 + i];
  int64_t parity = ((s7 % 2) + 2) % 2;
  int64_t z8 = 2 * (int64_t)fields[8] + parity;
  for (int i = 0; i < 7; ++i) x[i] = (double)fields[1 + i] + 0.5 * c;
  x[7] = (double)z8 + 0.5 * c;
}

void epo_point_to_fields_batch(const double* x, int64_t nvec, int32_t* fields) {
  for (int64_t g = 0; g < nvec; ++g) epo_point_to_fields(x + 8 * g, fields + 9 * g);
}

void epo_fields_to_point_batch(const int32_t* fields, int64_t nvec, double* x) {
  for (int64_t g = 0; g < nvec; ++g) epo_fields_to_point(fields + 9 * g, x + 8 * g);
}

/* Row statistic: n_r = sqrt(mean_c W[r,c]^2), accumulated in fp64 in column order. */
void epo_row_rms(const float* W, int64_t rows, int64_t cols, double* norms) {
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c) {
      double w = (double)W[r * cols + c];
      acc += w * w;
    }
    norms[r] = sqrt(acc / (double)cols);
  }
}
