/*
 * Oracle: tensor-level encoder (scale search, full quantisation, alphabet
 * escalation, row refit, tables, tiles), stored-size accounting and the
 * tensor decoder.  TEST INFRASTRUCTURE ONLY (see epo.h).
 *
 * Passages followed:
 *  - EntroPack paper, section 3.1 (pipeline), section 3.4 "Geometric search"
 *    (bisection of the geometric midpoint of a scale bracket; a rate above the
 *    target replaces lo, otherwise hi; b is raised when an alphabet exceeds
 *    2^b, and the scale is coarsened at the highest precision).
 *  - Appendix C.1: twelve bisection steps on [1e-3, 8], about 2^18 sampled
 *    eight-dimensional vectors taken as complete rows with a shape-dependent
 *    seed; b starts at 11 for targets up to 7 bpp and at 12 above; b rises to
 *    at most 15; then s <- 1.05 s A_max / 2^b until the alphabets fit.
 *  - Appendix C.3 "Tile layout and storage" and Table 5: V = max(32, floor(S/9))
 *    vectors per tile, S = 32768 (2 bpp), 16384 (4), 8192 (7), 4096 (8);
 *    4J + 4 = 132 bytes of tile metadata per tile plus one final offset.
 *  - Section 3.6 "Stored representation": payload words, offsets, terminal
 *    states, tables with alphabet offsets, row reconstruction scales and the
 *    tensor layout make up the stored bytes.
 *  - Section 3.5 heading "Row-scale refit": one fitted FP32 reconstruction
 *    scale per row (section 3.1).  The formula is not printed; this oracle
 *    uses the least-squares scale <W_r, sX_r> / <sX_r, sX_r>.
 *
 * Readings where the pages are silent (listed in the design notes):
 *  - Rate estimate: bits = sum over sampled symbols of -log2(f/M) with the
 *    sample's own normalised tables, scaled to the tensor's vector count, plus
 *    the exact side-information bytes; an unnormalisable sample scores +inf.
 *  - Targets 3, 5, 6 bpp use the tile size of the largest listed target below.
 *  - The row sample is a partial Fisher-Yates shuffle driven by SplitMix64
 *    (Steele, Lea & Flood, 2014) seeded with rows * 2^32 + cols, then sorted.
 *  - Container bytes: 32-byte header (rows, cols as i64; V, T, b as u32; s as
 *    f32), c-table 2 x u16, each coordinate table i32 min + u16 A + A x u16,
 *    FP32 row scales, FP32 route scales for the FP8/INT8 routes, 32 x u32
 *    states + u32 offset per tile, one final u32 offset, u16 payload words.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "epo.h"

/* internal entry points from epo_rans.c */
void* epo__tables_new(const uint16_t* const* freq, const uint32_t* alphabet, uint32_t b);
void  epo__tables_free(void* t);
int   epo__tile_encode(uint32_t n, const int32_t* sym, const void* tb, uint32_t* states,
                       uint16_t* words, uint32_t cap, uint32_t* nwords);
int   epo__tile_decode(uint32_t n, const uint32_t* states, const uint16_t* words,
                       uint32_t nwords, const void* tb, int32_t* sym);

struct epo_tensor {
  int64_t rows, cols;
  uint32_t V, T, b;
  float s;
  int route;
  double est_bpp;
  float* row_scales;
  float* route_scales;
  uint32_t* states;
  uint32_t* offsets;
  uint16_t* payload;
  uint64_t nwords;
  uint32_t alphabet[EPO_TABLES];
  int32_t minval[EPO_TABLES];
  uint32_t freq_base[EPO_TABLES];
  uint16_t* freqs;
  uint32_t nfreqs;
  int coding;
};

uint32_t epo_default_vectors_per_tile(double target_bpp) {
  uint32_t S;
  if (target_bpp >= 8.0) S = 4096;
  else if (target_bpp >= 7.0) S = 8192;
  else if (target_bpp >= 4.0) S = 16384;
  else S = 32768;
  uint32_t V = S / EPO_FIELDS;
  return V < 32 ? 32 : V;
}

uint32_t epo_default_prob_bits(double target_bpp) { return target_bpp <= 7.0 ? 11u : 12u; }

uint64_t epo_num_tiles(int64_t rows, int64_t cols, uint32_t V) {
  uint64_t nvec = (uint64_t)rows * (uint64_t)cols / 8u;
  return (nvec + V - 1) / V;
}

uint64_t epo_stored_bytes(int64_t rows, uint32_t T, uint64_t nwords,
                          const uint32_t alphabet[EPO_TABLES], int route) {
  uint64_t bytes = 32;                       /* header */
  bytes += 4;                                /* c-table: two u16 frequencies */
  for (int k = 1; k < EPO_TABLES; ++k) bytes += 4 + 2 + 2ull * alphabet[k];
  bytes += 4ull * (uint64_t)rows;            /* FP32 row reconstruction scales */
  if (route != EPO_ROUTE_DIRECT) bytes += 4ull * (uint64_t)rows;  /* route scales */
  bytes += 132ull * T + 4;                   /* tile metadata (4J + 4 per tile) + final offset */
  bytes += 2ull * nwords;                    /* payload */
  return bytes;
}

uint64_t epo_stored_bytes_coded(int64_t rows, uint32_t T, uint64_t nwords,
                                const uint32_t alphabet[EPO_TABLES], int route, int coding) {
  uint64_t bytes = epo_stored_bytes(rows, T, nwords, alphabet, route);
  if (coding == EPO_CODING_POOLED)   /* the coset-1 copies of the 8 tables are not stored */
    for (int f = 1; f < EPO_FIELDS; ++f) bytes -= 4 + 2 + 2ull * alphabet[epo_table_index(f, 1)];
  return bytes;
}

/* SplitMix64 (Steele, Lea & Flood 2014). */
static uint64_t splitmix64(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int cmp_i64(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x > y) - (x < y);
}

/* Complete rows covering about 2^18 vectors, chosen with a shape-dependent seed. */
void epo_sample_rows(int64_t rows, int64_t cols, int64_t* picked, int64_t* npicked) {
  int64_t per_row = cols / 8;
  int64_t want = per_row > 0 ? ((1ll << 18) + per_row - 1) / per_row : rows;
  if (want < 1) want = 1;
  if (want > rows) want = rows;
  int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (rows ? rows : 1));
  for (int64_t i = 0; i < rows; ++i) perm[i] = i;
  uint64_t st = ((uint64_t)rows << 32) + (uint64_t)cols;
  for (int64_t i = 0; i < want; ++i) {
    uint64_t j = (uint64_t)i + splitmix64(&st) % (uint64_t)(rows - i);
    int64_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
  qsort(perm, (size_t)want, sizeof(int64_t), cmp_i64);
  memcpy(picked, perm, sizeof(int64_t) * (size_t)want);
  *npicked = want;
  free(perm);
}

/* Quantise the listed rows at scale s into fields [nrows * cols/8][9]. */
static void quantize_rows(const float* W, int64_t cols, const double* norms,
                          const int64_t* row_idx, int64_t nrows, double s, int32_t* fields) {
  int64_t per_row = cols / 8;
  double v[8], x[8];
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = row_idx ? row_idx[i] : i;
    double n = norms[r];
    for (int64_t j = 0; j < per_row; ++j) {
      for (int q = 0; q < 8; ++q) {
        double u = n > 0.0 ? (double)W[r * cols + 8 * j + q] / n : 0.0;
        v[q] = u / s;
      }
      epo_e8_nearest(v, x);
      epo_point_to_fields(x, fields + 9 * (i * per_row + j));
    }
  }
}

/* min/max of every table over the given fields; has[k] = 0 if no symbol. */
static void table_ranges(const int32_t* fields, int64_t nvec, int32_t* minv, int32_t* maxv,
                         int* has) {
  for (int k = 0; k < EPO_TABLES; ++k) has[k] = 0, minv[k] = 0, maxv[k] = 0;
  /* the c-table always covers {0, 1} */
  has[0] = 1;
  minv[0] = 0;
  maxv[0] = 1;
  for (int64_t g = 0; g < nvec; ++g) {
    const int32_t* fl = fields + 9 * g;
    int c = fl[0];
    for (int f = 1; f < EPO_FIELDS; ++f) {
      int k = epo_table_index(f, c);
      int32_t val = fl[f];
      if (!has[k]) {
        has[k] = 1;
        minv[k] = maxv[k] = val;
      } else {
        if (val < minv[k]) minv[k] = val;
        if (val > maxv[k]) maxv[k] = val;
      }
    }
  }
}

/* counts[k][i] for value minv[k] + i */
static uint64_t** table_counts(const int32_t* fields, int64_t nvec, const int32_t* minv,
                               const uint32_t* A) {
  uint64_t** counts = (uint64_t**)malloc(sizeof(uint64_t*) * EPO_TABLES);
  for (int k = 0; k < EPO_TABLES; ++k) counts[k] = (uint64_t*)calloc(A[k] ? A[k] : 1, sizeof(uint64_t));
  for (int64_t g = 0; g < nvec; ++g) {
    const int32_t* fl = fields + 9 * g;
    int c = fl[0];
    counts[0][c] += 1;
    for (int f = 1; f < EPO_FIELDS; ++f) {
      int k = epo_table_index(f, c);
      counts[k][fl[f] - minv[k]] += 1;
    }
  }
  return counts;
}

static void free_counts(uint64_t** counts) {
  for (int k = 0; k < EPO_TABLES; ++k) free(counts[k]);
  free(counts);
}

static void alphabets_from_ranges(const int32_t* minv, const int32_t* maxv, const int* has,
                                  uint32_t* A) {
  for (int k = 0; k < EPO_TABLES; ++k)
    A[k] = has[k] ? (uint32_t)((int64_t)maxv[k] - (int64_t)minv[k] + 1) : 0u;
  A[0] = 2;
}

double epo_estimate_bpp(const float* W, int64_t rows, int64_t cols, const double* norms,
                        const int64_t* sample, int64_t nsample, double s, uint32_t b,
                        uint32_t V, int route) {
  int64_t per_row = cols / 8;
  int64_t nvec_s = nsample * per_row;
  if (nvec_s == 0) return 0.0;
  int32_t* fields = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)nvec_s);
  quantize_rows(W, cols, norms, sample, nsample, s, fields);
  int32_t minv[EPO_TABLES], maxv[EPO_TABLES];
  int has[EPO_TABLES];
  uint32_t A[EPO_TABLES];
  table_ranges(fields, nvec_s, minv, maxv, has);
  alphabets_from_ranges(minv, maxv, has, A);
  uint64_t** counts = table_counts(fields, nvec_s, minv, A);
  double bits = 0.0;
  int ok = 1;
  for (int k = 0; k < EPO_TABLES && ok; ++k) {
    if (A[k] == 0) continue;
    uint16_t* f = (uint16_t*)malloc(sizeof(uint16_t) * A[k]);
    if (epo_normalize_freqs(counts[k], A[k], b, f) != 0) {
      ok = 0;
    } else {
      for (uint32_t i = 0; i < A[k]; ++i)
        if (counts[k][i]) bits += (double)counts[k][i] * ((double)b - log2((double)f[i]));
    }
    free(f);
  }
  free_counts(counts);
  free(fields);
  if (!ok) return INFINITY;
  uint64_t nvec = (uint64_t)rows * (uint64_t)per_row;
  uint32_t T = (uint32_t)epo_num_tiles(rows, cols, V);
  double payload_bytes = bits * ((double)nvec / (double)nvec_s) / 8.0;
  double side = (double)epo_stored_bytes(rows, T, 0, A, route);
  return 8.0 * (payload_bytes + side) / ((double)rows * (double)cols);
}

static double scale_search(const float* W, int64_t rows, int64_t cols, const double* norms,
                           const int64_t* sample, int64_t nsample, double target, uint32_t b,
                           uint32_t V, int route) {
  double lo = 1e-3, hi = 8.0;
  for (int it = 0; it < 12; ++it) {
    double s = sqrt(lo * hi);
    double est = epo_estimate_bpp(W, rows, cols, norms, sample, nsample, s, b, V, route);
    if (est > target) lo = s;
    else hi = s;
  }
  return sqrt(lo * hi);
}

static uint32_t max_coord_alphabet(const int32_t* fields, int64_t nvec) {
  int32_t minv[EPO_TABLES], maxv[EPO_TABLES];
  int has[EPO_TABLES];
  uint32_t A[EPO_TABLES];
  table_ranges(fields, nvec, minv, maxv, has);
  alphabets_from_ranges(minv, maxv, has, A);
  uint32_t amax = 0;
  for (int k = 1; k < EPO_TABLES; ++k)
    if (A[k] > amax) amax = A[k];
  return amax;
}

/* Shared tail of the encoder: given the final fields at scale s and precision b,
 * fit row scales, build tables and encode tiles. */
static int finish_encode(const float* Wq, int64_t rows, int64_t cols, float s, uint32_t b,
                         uint32_t V, const int32_t* fields_in, int coding, epo_tensor* t) {
  int64_t per_row = cols / 8;
  int64_t nvec = rows * per_row;
  t->s = s;
  t->b = b;
  t->V = V;
  t->T = (uint32_t)epo_num_tiles(rows, cols, V);

  /* row refit: r = <W_r, s X_r> / <s X_r, s X_r> */
  t->row_scales = (float*)malloc(sizeof(float) * (rows ? rows : 1));
  double x[8];
  for (int64_t r = 0; r < rows; ++r) {
    double num = 0.0, den = 0.0;
    for (int64_t j = 0; j < per_row; ++j) {
      epo_fields_to_point(fields_in + 9 * (r * per_row + j), x);
      for (int q = 0; q < 8; ++q) {
        double sx = (double)s * x[q];
        num += (double)Wq[r * cols + 8 * j + q] * sx;
        den += sx * sx;
      }
    }
    t->row_scales[r] = den > 0.0 ? (float)(num / den) : 0.0f;
  }

  /* the coded fields: direct z8 replaces m by z8 = 2m + parity(z1..z7) */
  t->coding = coding;
  const int32_t* fields = fields_in;
  int32_t* zf = NULL;
  if (coding == EPO_CODING_DIRECT_Z8) {
    zf = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)(nvec ? nvec : 1));
    memcpy(zf, fields_in, sizeof(int32_t) * 9 * (size_t)nvec);
    for (int64_t g = 0; g < nvec; ++g) {
      double x[8];
      epo_fields_to_point(fields_in + 9 * g, x);
      zf[9 * g + 8] = (int32_t)(x[7] - 0.5 * fields_in[9 * g]);
    }
    fields = zf;
  }

  /* tables */
  int32_t maxv[EPO_TABLES];
  int has[EPO_TABLES];
  table_ranges(fields, nvec, t->minval, maxv, has);
  if (coding == EPO_CODING_POOLED) {
    /* one range per field over both cosets */
    for (int f = 1; f < EPO_FIELDS; ++f) {
      int k0 = epo_table_index(f, 0), k1 = epo_table_index(f, 1);
      if (has[k0] && has[k1]) {
        if (t->minval[k1] < t->minval[k0]) t->minval[k0] = t->minval[k1];
        if (maxv[k1] > maxv[k0]) maxv[k0] = maxv[k1];
      } else if (has[k1]) {
        t->minval[k0] = t->minval[k1];
        maxv[k0] = maxv[k1];
        has[k0] = 1;
      }
      t->minval[k1] = t->minval[k0];
      maxv[k1] = maxv[k0];
      has[k1] = has[k0];
    }
  }
  alphabets_from_ranges(t->minval, maxv, has, t->alphabet);
  for (int k = 0; k < EPO_TABLES; ++k)
    if (!has[k]) t->minval[k] = 0;
  t->minval[0] = 0;
  /* an ablation's alphabets (z8, or a pooled range) may outgrow 2^b */
  for (int k = 1; k < EPO_TABLES; ++k)
    if (t->alphabet[k] > (1u << b)) {
      free(zf);
      return -13;
    }
  uint64_t** counts = table_counts(fields, nvec, t->minval, t->alphabet);
  if (coding == EPO_CODING_POOLED) {
    /* pooled counts; the coset-1 slot shares the coset-0 table */
    for (int f = 1; f < EPO_FIELDS; ++f) {
      int k0 = epo_table_index(f, 0), k1 = epo_table_index(f, 1);
      for (uint32_t i = 0; i < t->alphabet[k0]; ++i) counts[k0][i] += counts[k1][i];
    }
  }
  uint32_t nf = 0;
  for (int k = 0; k < EPO_TABLES; ++k) {
    if (coding == EPO_CODING_POOLED && k > 0 && (k - 1) % 2 == 1) {
      t->freq_base[k] = t->freq_base[k - 1];
      continue;
    }
    t->freq_base[k] = nf;
    nf += t->alphabet[k];
  }
  t->nfreqs = nf;
  t->freqs = (uint16_t*)calloc(nf ? nf : 1, sizeof(uint16_t));
  int rc = 0;
  for (int k = 0; k < EPO_TABLES && rc == 0; ++k) {
    if (coding == EPO_CODING_POOLED && k > 0 && (k - 1) % 2 == 1) continue;
    if (t->alphabet[k]) rc = epo_normalize_freqs(counts[k], t->alphabet[k], b, t->freqs + t->freq_base[k]);
  }
  free_counts(counts);
  if (rc != 0) return -10;

  /* zero-based symbols */
  int32_t* sym = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)(nvec ? nvec : 1));
  for (int64_t g = 0; g < nvec; ++g) {
    const int32_t* fl = fields + 9 * g;
    int c = fl[0];
    sym[9 * g] = c;
    for (int f = 1; f < EPO_FIELDS; ++f) sym[9 * g + f] = fl[f] - t->minval[epo_table_index(f, c)];
  }

  /* tiles */
  const uint16_t* fptr[EPO_TABLES];
  for (int k = 0; k < EPO_TABLES; ++k) fptr[k] = t->freqs + t->freq_base[k];
  void* tb = epo__tables_new(fptr, t->alphabet, b);
  t->states = (uint32_t*)malloc(sizeof(uint32_t) * EPO_LANES * (t->T ? t->T : 1));
  t->offsets = (uint32_t*)malloc(sizeof(uint32_t) * (t->T + 1));
  uint64_t cap_total = 9ull * (uint64_t)nvec;
  t->payload = (uint16_t*)malloc(sizeof(uint16_t) * (cap_total ? cap_total : 1));
  uint64_t pos = 0;
  for (uint32_t ti = 0; ti < t->T && rc == 0; ++ti) {
    uint64_t first = (uint64_t)ti * V;
    uint32_t n = (uint32_t)((nvec - first) < V ? (nvec - first) : V);
    uint32_t nw = 0;
    t->offsets[ti] = (uint32_t)pos;
    rc = epo__tile_encode(n, sym + 9 * first, tb, t->states + EPO_LANES * ti,
                          t->payload + pos, 9u * n, &nw);
    pos += nw;
  }
  t->offsets[t->T] = (uint32_t)pos;
  t->nwords = pos;
  epo__tables_free(tb);
  free(sym);
  free(zf);
  return rc == 0 ? 0 : -11;
}

static epo_tensor* tensor_new(int64_t rows, int64_t cols, int route) {
  epo_tensor* t = (epo_tensor*)calloc(1, sizeof(epo_tensor));
  t->rows = rows;
  t->cols = cols;
  t->route = route;
  return t;
}

static float* prepare_input(const float* W, int64_t rows, int64_t cols, int route,
                            epo_tensor* t) {
  size_t n = (size_t)(rows * cols);
  float* Wq = (float*)malloc(sizeof(float) * (n ? n : 1));
  if (route == EPO_ROUTE_DIRECT) {
    memcpy(Wq, W, sizeof(float) * n);
  } else {
    t->route_scales = (float*)malloc(sizeof(float) * (rows ? rows : 1));
    epo_route_precast(W, rows, cols, route, Wq, t->route_scales);
  }
  return Wq;
}

/* Algorithm 1 with the precision escalation and coarsening of appendix C.1:
 * returns the final scale, raises *b as needed, leaves the full tensor's
 * fields at that scale in `fields` and the sampled rate estimate in *est. */
static float baseline_scale(const float* Wq, int64_t rows, int64_t cols, const double* norms,
                            double target_bpp, uint32_t V, int route, uint32_t* bp,
                            int32_t* fields, double* est) {
  int64_t* sample = (int64_t*)malloc(sizeof(int64_t) * (rows ? rows : 1));
  int64_t nsample = 0;
  epo_sample_rows(rows, cols, sample, &nsample);
  int64_t nvec = rows * (cols / 8);
  uint32_t b = *bp;
  float s = 1.0f;
  for (;;) {
    double sd = scale_search(Wq, rows, cols, norms, sample, nsample, target_bpp, b, V, route);
    *est = epo_estimate_bpp(Wq, rows, cols, norms, sample, nsample, sd, b, V, route);
    s = (float)sd;
    quantize_rows(Wq, cols, norms, NULL, rows, (double)s, fields);
    uint32_t amax = max_coord_alphabet(fields, nvec);
    if (amax <= (1u << b)) break;
    if (b < 15) {
      b += 1;
      continue;
    }
    while (amax > (1u << b)) {
      s = (float)(1.05 * (double)s * (double)amax / (double)(1u << b));
      quantize_rows(Wq, cols, norms, NULL, rows, (double)s, fields);
      amax = max_coord_alphabet(fields, nvec);
    }
    break;
  }
  free(sample);
  *bp = b;
  return s;
}

int epo_encode(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t V,
               uint32_t b0, int route, epo_tensor** out) {
  return epo_encode_coded(W, rows, cols, target_bpp, V, b0, route, EPO_CODING_STANDARD, out);
}

int epo_encode_coded(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t V,
                     uint32_t b0, int route, int coding, epo_tensor** out) {
  if (coding < EPO_CODING_STANDARD || coding > EPO_CODING_DIRECT_Z8) return -1;
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return -1;
  if (route < 0 || route > 2) return -1;
  if (V == 0) V = epo_default_vectors_per_tile(target_bpp);
  if (V < 32) return -1;
  uint32_t b = b0 ? b0 : epo_default_prob_bits(target_bpp);
  if (b < 9 || b > 15) return -1;
  if ((uint64_t)rows * (uint64_t)cols / 8u > 0xFFFFFFFFull) return -1;

  epo_tensor* t = tensor_new(rows, cols, route);
  float* Wq = prepare_input(W, rows, cols, route, t);
  double* norms = (double*)malloc(sizeof(double) * (rows ? rows : 1));
  epo_row_rms(Wq, rows, cols, norms);
  int64_t nvec = rows * (cols / 8);
  int32_t* fields = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)(nvec ? nvec : 1));
  float s = baseline_scale(Wq, rows, cols, norms, target_bpp, V, route, &b, fields, &t->est_bpp);
  int rc = finish_encode(Wq, rows, cols, s, b, V, fields, coding, t);
  free(fields);
  free(norms);
  free(Wq);
  if (rc != 0) {
    epo_tensor_free(t);
    return rc;
  }
  *out = t;
  return 0;
}

/* Encode at a given scale and precision (no search; used by tests that need a
 * particular alphabet or precision). */
int epo_encode_fixed_scale(const float* W, int64_t rows, int64_t cols, float s, uint32_t V,
                           uint32_t b, int route, epo_tensor** out) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || V < 32 || b < 9 || b > 15) return -1;
  if (!(s > 0.0f)) return -1;
  epo_tensor* t = tensor_new(rows, cols, route);
  float* Wq = prepare_input(W, rows, cols, route, t);
  double* norms = (double*)malloc(sizeof(double) * (rows ? rows : 1));
  epo_row_rms(Wq, rows, cols, norms);
  int64_t nvec = rows * (cols / 8);
  int32_t* fields = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)(nvec ? nvec : 1));
  quantize_rows(Wq, cols, norms, NULL, rows, (double)s, fields);
  int rc = 0;
  if (max_coord_alphabet(fields, nvec) > (1u << b)) rc = -12;
  if (rc == 0) rc = finish_encode(Wq, rows, cols, s, b, V, fields, EPO_CODING_STANDARD, t);
  free(fields);
  free(norms);
  free(Wq);
  if (rc != 0) {
    epo_tensor_free(t);
    return rc;
  }
  t->est_bpp = 0.0;
  *out = t;
  return 0;
}

void epo_tensor_free(epo_tensor* t) {
  if (!t) return;
  free(t->row_scales);
  free(t->route_scales);
  free(t->states);
  free(t->offsets);
  free(t->payload);
  free(t->freqs);
  free(t);
}

void epo_tensor_info(const epo_tensor* t, int64_t* rows, int64_t* cols, uint32_t* V,
                     uint32_t* T, uint32_t* b, float* s, uint64_t* nwords, uint32_t* nfreqs,
                     int* route, double* est_bpp) {
  *rows = t->rows;
  *cols = t->cols;
  *V = t->V;
  *T = t->T;
  *b = t->b;
  *s = t->s;
  *nwords = t->nwords;
  *nfreqs = t->nfreqs;
  *route = t->route;
  *est_bpp = t->est_bpp;
}

int epo_tensor_coding(const epo_tensor* t) { return t->coding; }

void epo_tensor_tables(const epo_tensor* t, uint32_t* alphabet, int32_t* minval,
                       uint32_t* freq_base) {
  memcpy(alphabet, t->alphabet, sizeof(t->alphabet));
  memcpy(minval, t->minval, sizeof(t->minval));
  memcpy(freq_base, t->freq_base, sizeof(t->freq_base));
}

void epo_tensor_copy(const epo_tensor* t, float* row_scales, float* route_scales,
                     uint32_t* states, uint32_t* offsets, uint16_t* payload, uint16_t* freqs) {
  if (row_scales) memcpy(row_scales, t->row_scales, sizeof(float) * (size_t)t->rows);
  if (route_scales && t->route_scales)
    memcpy(route_scales, t->route_scales, sizeof(float) * (size_t)t->rows);
  if (states) memcpy(states, t->states, sizeof(uint32_t) * EPO_LANES * t->T);
  if (offsets) memcpy(offsets, t->offsets, sizeof(uint32_t) * (t->T + 1));
  if (payload) memcpy(payload, t->payload, sizeof(uint16_t) * (size_t)t->nwords);
  if (freqs) memcpy(freqs, t->freqs, sizeof(uint16_t) * t->nfreqs);
}

/* Decode tiles [tile_begin, tile_end) of a tensor given as plain arrays. */
int epo_decode(int64_t rows, int64_t cols, uint32_t V, uint32_t T, uint32_t b, float s,
               const float* row_scales, const uint32_t* states, const uint32_t* offsets,
               const uint16_t* payload, const uint16_t* freqs, const uint32_t* freq_base,
               const uint32_t* alphabet, const int32_t* minval, int out_kind, void* out,
               int32_t* tile_status, uint32_t tile_begin, uint32_t tile_end) {
  return epo_decode_coded(rows, cols, V, T, b, s, row_scales, states, offsets, payload, freqs,
                          freq_base, alphabet, minval, EPO_CODING_STANDARD, out_kind, out,
                          tile_status, tile_begin, tile_end);
}

int epo_decode_coded(int64_t rows, int64_t cols, uint32_t V, uint32_t T, uint32_t b, float s,
                     const float* row_scales, const uint32_t* states, const uint32_t* offsets,
                     const uint16_t* payload, const uint16_t* freqs, const uint32_t* freq_base,
                     const uint32_t* alphabet, const int32_t* minval, int coding, int out_kind,
                     void* out, int32_t* tile_status, uint32_t tile_begin, uint32_t tile_end) {
  if (coding < EPO_CODING_STANDARD || coding > EPO_CODING_DIRECT_Z8) return -1;
  if (rows < 0 || cols <= 0 || cols % 8 != 0 || V < 32 || b < 9 || b > 15) return -1;
  if (T != epo_num_tiles(rows, cols, V)) return -1;
  if (tile_begin > tile_end || tile_end > T) return -1;
  if (alphabet[0] != 2) return -1;
  for (int k = 1; k < EPO_TABLES; ++k)
    if (alphabet[k] > (1u << b)) return -1;
  int64_t per_row = cols / 8;
  uint64_t nvec = (uint64_t)rows * (uint64_t)per_row;
  const uint16_t* fptr[EPO_TABLES];
  for (int k = 0; k < EPO_TABLES; ++k) fptr[k] = freqs + freq_base[k];
  void* tb = epo__tables_new(fptr, alphabet, b);
  int32_t* sym = (int32_t*)malloc(sizeof(int32_t) * 9 * V);
  for (uint32_t ti = tile_begin; ti < tile_end; ++ti) {
    uint64_t first = (uint64_t)ti * V;
    uint32_t n = (uint32_t)((nvec - first) < V ? (nvec - first) : V);
    uint32_t start = offsets[ti];
    uint32_t nw = offsets[ti + 1] >= start ? offsets[ti + 1] - start : 0;
    int rc = (offsets[ti + 1] >= start)
                 ? epo__tile_decode(n, states + EPO_LANES * ti, payload + start, nw, tb, sym)
                 : EPO_TILE_BAD_LENGTH;
    if (tile_status) tile_status[ti] = rc;
    if (rc != EPO_TILE_OK) continue;
    for (uint32_t v = 0; v < n; ++v) {
      uint64_t g = first + v;
      int32_t fl[9];
      int c = sym[9 * v];
      fl[0] = c;
      for (int f = 1; f < EPO_FIELDS; ++f)
        fl[f] = sym[9 * v + f] + minval[epo_table_index(f, c)];
      if (out_kind == EPO_OUT_FIELDS) {
        memcpy((int32_t*)out + 9 * g, fl, sizeof(fl));
        continue;
      }
      double x[8];
      if (coding == EPO_CODING_DIRECT_Z8) {
        /* the eighth field is z8 itself: x = z + c/2 for all eight coordinates */
        for (int i = 0; i < 8; ++i) x[i] = (double)fl[1 + i] + 0.5 * c;
      } else {
        epo_fields_to_point(fl, x);
      }
      uint64_t r = g / (uint64_t)per_row;
      float gs = s * row_scales[r];              /* fp32(s * r_row) */
      for (int q = 0; q < 8; ++q) {
        uint64_t o = 8 * g + (uint64_t)q;
        if (out_kind == EPO_OUT_LATTICE2X) {
          ((int32_t*)out)[o] = (int32_t)(2.0 * x[q]);
          continue;
        }
        float y = (float)x[q] * gs;              /* fp32(x * g) */
        switch (out_kind) {
          case EPO_OUT_BF16: ((uint16_t*)out)[o] = epo_f32_to_bf16(y); break;
          case EPO_OUT_FP8: ((uint8_t*)out)[o] = epo_f32_to_fp8e4m3(y); break;
          case EPO_OUT_INT8: ((int8_t*)out)[o] = epo_f32_to_int8(y); break;
          case EPO_OUT_UINT8: ((uint8_t*)out)[o] = epo_f32_to_uint8(y); break;
          case EPO_OUT_FP16: ((uint16_t*)out)[o] = epo_f32_to_f16(y); break;
          default: ((float*)out)[o] = y; break;
        }
      }
    }
  }
  free(sym);
  epo__tables_free(tb);
  return 0;
}

/* ------------------------------------------------------------------------
 * Per-row rate-distortion refinement (paper, section 3.5 "Per-row
 * rate-distortion refinement", appendix C.2 and appendix A.4).
 *
 * What the pages fix: each row chooses one of K quantisation resolutions
 * rho_k * s with rho_1 = 1 and ratios inside [0.70, 1.45], added by bisecting
 * the widest remaining interval in log scale, so the sets are nested; the
 * candidates' fields, fitted row scales and distortions are computed once;
 * each sweep updates the shared probability model from the selected fields
 * and then selects the rows' candidates through one common rate penalty; the
 * allocation keeps the single-scale baseline's storage.  Algorithm 2 itself
 * is not printed.  Readings (listed in the design notes):
 *  - The first interval bisected is the wider of [0.70, 1] and [1, 1.45] in
 *    log scale (ties: the lower one); the bounds are not candidates.
 *  - Distortion D_rk = sum over the row of (w - y)^2 in fp64, y being the
 *    decoded fp32 value fp32(x * fp32(s * r_rk)) with the candidate's
 *    least-squares row scale r_rk.
 *  - Rate R_rk = sum over the row's symbols of (b_m - log2 f) bits under the
 *    model's normalised tables (precision b_m = the smallest b' >= b that
 *    holds the model's alphabets), a symbol the model does not hold costing
 *    b_m bits; costs are kept in units of 2^-16 bit (rounded to nearest) so
 *    that totals are exact integers.
 *  - The budget is the baseline selection's total rate under the first
 *    sweep's model.  The penalty lambda is the smallest one (to a 60-step
 *    bisection) at which the rows' choices argmin_k D_rk + lambda R_rk (ties
 *    to the lower k) fit the budget; lambda = 0 if the least-distortion
 *    choices already fit.
 *  - Sweeps stop early if the selected fields need more than 15 bits of
 *    precision; the container keeps b if the final fields fit 2^b, raises it
 *    otherwise (at most 15), and falls back to the baseline fields if even
 *    that does not hold them.
 * ------------------------------------------------------------------------ */

void epo_rdo_ratios(uint32_t K, double* rho) {
  /* log-scale intervals, kept sorted by position */
  double lo[64], hi[64];
  int n = 2;
  lo[0] = log(0.70);
  hi[0] = 0.0;
  lo[1] = 0.0;
  hi[1] = log(1.45);
  if (K == 0) return;
  rho[0] = 1.0;
  for (uint32_t k = 1; k < K && n < 63; ++k) {
    int w = 0;
    for (int i = 1; i < n; ++i)
      if (hi[i] - lo[i] > hi[w] - lo[w]) w = i;
    double mid = 0.5 * (lo[w] + hi[w]);
    rho[k] = exp(mid);
    for (int i = n; i > w + 1; --i) lo[i] = lo[i - 1], hi[i] = hi[i - 1];
    lo[w + 1] = mid;
    hi[w + 1] = hi[w];
    hi[w] = mid;
    ++n;
  }
}

/* model cost tables: cost[base[k] + i] in 2^-16 bit for value minv[k] + i */
typedef struct {
  int32_t minv[EPO_TABLES];
  uint32_t A[EPO_TABLES];
  uint32_t base[EPO_TABLES];
  int64_t* cost;
  int64_t miss;          /* cost of a symbol the model does not hold */
} rdo_model;

static int rdo_model_build(const int32_t* fields, int64_t nvec, uint32_t b, rdo_model* m) {
  int32_t maxv[EPO_TABLES];
  int has[EPO_TABLES];
  table_ranges(fields, nvec, m->minv, maxv, has);
  alphabets_from_ranges(m->minv, maxv, has, m->A);
  uint32_t bm = b;
  for (int k = 1; k < EPO_TABLES; ++k)
    while (m->A[k] > (1u << bm) && bm < 15) ++bm;
  for (int k = 1; k < EPO_TABLES; ++k)
    if (m->A[k] > (1u << bm)) return -1;
  uint32_t tot = 0;
  for (int k = 0; k < EPO_TABLES; ++k) {
    m->base[k] = tot;
    tot += m->A[k];
  }
  m->cost = (int64_t*)malloc(sizeof(int64_t) * (tot ? tot : 1));
  m->miss = (int64_t)65536 * (int64_t)bm;
  uint64_t** counts = table_counts(fields, nvec, m->minv, m->A);
  int rc = 0;
  for (int k = 0; k < EPO_TABLES && rc == 0; ++k) {
    if (m->A[k] == 0) continue;
    uint16_t* f = (uint16_t*)malloc(sizeof(uint16_t) * m->A[k]);
    if (epo_normalize_freqs(counts[k], m->A[k], bm, f) != 0) {
      rc = -1;
    } else {
      for (uint32_t i = 0; i < m->A[k]; ++i)
        m->cost[m->base[k] + i] =
            f[i] ? llround(65536.0 * ((double)bm - log2((double)f[i]))) : m->miss;
    }
    free(f);
  }
  free_counts(counts);
  if (rc != 0) free(m->cost);
  return rc;
}

static int64_t rdo_row_rate(const int32_t* fl, int64_t per_row, const rdo_model* m) {
  int64_t r = 0;
  for (int64_t j = 0; j < per_row; ++j, fl += 9) {
    int c = fl[0];
    for (int f = 0; f < EPO_FIELDS; ++f) {
      int k = epo_table_index(f, c);
      int64_t i = (int64_t)fl[f] - (int64_t)m->minv[k];
      r += (i >= 0 && i < (int64_t)m->A[k]) ? m->cost[m->base[k] + i] : m->miss;
    }
  }
  return r;
}

/* rows' choices at penalty lam; returns their total rate */
static int64_t rdo_choose(const double* D, const int64_t* R, int64_t rows, uint32_t K, double lam,
                          int32_t* sel) {
  int64_t tot = 0;
  for (int64_t r = 0; r < rows; ++r) {
    uint32_t best = 0;
    double jb = D[r * K] + lam * ((double)R[r * K] / 65536.0);
    for (uint32_t k = 1; k < K; ++k) {
      double j = D[r * K + k] + lam * ((double)R[r * K + k] / 65536.0);
      if (j < jb) jb = j, best = k;
    }
    if (sel) sel[r] = (int32_t)best;
    tot += R[r * K + best];
  }
  return tot;
}

static double rdo_lambda(const double* D, const int64_t* R, int64_t rows, uint32_t K, int64_t budget) {
  if (rdo_choose(D, R, rows, K, 0.0, NULL) <= budget) return 0.0;
  double sd = 0.0, sr = 0.0;
  for (int64_t r = 0; r < rows; ++r) sd += D[r * K], sr += (double)R[r * K] / 65536.0;
  double hi = (sd > 0.0 && sr > 0.0) ? sd / sr : 1e-30;
  double lo = 0.0;
  int it = 0;
  while (rdo_choose(D, R, rows, K, hi, NULL) > budget && it < 200) {
    lo = hi;
    hi *= 2.0;
    ++it;
  }
  for (int i = 0; i < 60; ++i) {
    double mid = 0.5 * (lo + hi);
    if (rdo_choose(D, R, rows, K, mid, NULL) > budget) lo = mid;
    else hi = mid;
  }
  return hi;
}

/* Candidates' fields [K][nvec * 9], row scales [rows * K] and distortions. */
static void rdo_candidates(const float* Wq, int64_t rows, int64_t cols, const double* norms, float s,
                           uint32_t K, const double* rho, int32_t* cand, float* rsc, double* D) {
  int64_t per_row = cols / 8;
  int64_t nvec = rows * per_row;
  for (uint32_t k = 0; k < K; ++k) {
    int32_t* fk = cand + (size_t)k * 9 * (size_t)nvec;
    quantize_rows(Wq, cols, norms, NULL, rows, (double)s * rho[k], fk);
    for (int64_t r = 0; r < rows; ++r) {
      double num = 0.0, den = 0.0, x[8];
      for (int64_t j = 0; j < per_row; ++j) {
        epo_fields_to_point(fk + 9 * (r * per_row + j), x);
        for (int q = 0; q < 8; ++q) {
          double sx = (double)s * x[q];
          num += (double)Wq[r * cols + 8 * j + q] * sx;
          den += sx * sx;
        }
      }
      float rs = den > 0.0 ? (float)(num / den) : 0.0f;
      float gs = s * rs;
      double d = 0.0;
      for (int64_t j = 0; j < per_row; ++j) {
        epo_fields_to_point(fk + 9 * (r * per_row + j), x);
        for (int q = 0; q < 8; ++q) {
          float y = (float)x[q] * gs;
          double e = (double)Wq[r * cols + 8 * j + q] - (double)y;
          d += e * e;
        }
      }
      rsc[r * K + k] = rs;
      D[r * K + k] = d;
    }
  }
}

static void rdo_gather(const int32_t* cand, int64_t rows, int64_t per_row, const int32_t* sel,
                       int32_t* out) {
  int64_t nvec = rows * per_row;
  for (int64_t r = 0; r < rows; ++r)
    memcpy(out + 9 * r * per_row, cand + (size_t)sel[r] * 9 * (size_t)nvec + 9 * r * per_row,
           sizeof(int32_t) * 9 * (size_t)per_row);
}

/* The refinement proper.  trace (optional, first sweep only): D, R [rows*K],
 * row scales [rows*K], budget, lambda, selection [rows]. */
static int rdo_run(const float* Wq, int64_t rows, int64_t cols, const double* norms, float s,
                   uint32_t b, uint32_t K, uint32_t sweeps, int32_t* fields, double* tD,
                   int64_t* tR, float* tS, int64_t* tbudget, double* tlam, int32_t* tsel) {
  int64_t per_row = cols / 8;
  int64_t nvec = rows * per_row;
  double rho[64];
  epo_rdo_ratios(K, rho);
  int32_t* cand = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)K * (size_t)(nvec ? nvec : 1));
  float* rsc = (float*)malloc(sizeof(float) * (size_t)K * (size_t)(rows ? rows : 1));
  double* D = (double*)malloc(sizeof(double) * (size_t)K * (size_t)(rows ? rows : 1));
  int64_t* R = (int64_t*)malloc(sizeof(int64_t) * (size_t)K * (size_t)(rows ? rows : 1));
  int32_t* sel = (int32_t*)calloc((size_t)(rows ? rows : 1), sizeof(int32_t));
  rdo_candidates(Wq, rows, cols, norms, s, K, rho, cand, rsc, D);
  int64_t budget = -1;
  for (uint32_t sw = 0; sw < sweeps; ++sw) {
    rdo_gather(cand, rows, per_row, sel, fields);
    rdo_model m;
    if (rdo_model_build(fields, nvec, b, &m) != 0) break;
    for (int64_t r = 0; r < rows; ++r)
      for (uint32_t k = 0; k < K; ++k)
        R[r * K + k] = rdo_row_rate(cand + (size_t)k * 9 * (size_t)nvec + 9 * r * per_row, per_row, &m);
    free(m.cost);
    if (budget < 0) {
      budget = 0;
      for (int64_t r = 0; r < rows; ++r) budget += R[r * K + sel[r]];
    }
    double lam = rdo_lambda(D, R, rows, K, budget);
    rdo_choose(D, R, rows, K, lam, sel);
    if (sw == 0) {
      if (tD) memcpy(tD, D, sizeof(double) * (size_t)K * (size_t)rows);
      if (tR) memcpy(tR, R, sizeof(int64_t) * (size_t)K * (size_t)rows);
      if (tS) memcpy(tS, rsc, sizeof(float) * (size_t)K * (size_t)rows);
      if (tbudget) *tbudget = budget;
      if (tlam) *tlam = lam;
      if (tsel) memcpy(tsel, sel, sizeof(int32_t) * (size_t)rows);
    }
  }
  rdo_gather(cand, rows, per_row, sel, fields);
  free(sel);
  free(R);
  free(D);
  free(rsc);
  free(cand);
  return 0;
}

int epo_encode_rdo(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t V,
                   uint32_t b0, int route, uint32_t K, uint32_t sweeps, epo_tensor** out) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return -1;
  if (route < 0 || route > 2 || K < 1 || K > 32) return -1;
  if (V == 0) V = epo_default_vectors_per_tile(target_bpp);
  if (V < 32) return -1;
  uint32_t b = b0 ? b0 : epo_default_prob_bits(target_bpp);
  if (b < 9 || b > 15) return -1;
  if ((uint64_t)rows * (uint64_t)cols / 8u > 0xFFFFFFFFull) return -1;
  epo_tensor* t = tensor_new(rows, cols, route);
  float* Wq = prepare_input(W, rows, cols, route, t);
  double* norms = (double*)malloc(sizeof(double) * (rows ? rows : 1));
  epo_row_rms(Wq, rows, cols, norms);
  int64_t nvec = rows * (cols / 8);
  int32_t* base = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)(nvec ? nvec : 1));
  float s = baseline_scale(Wq, rows, cols, norms, target_bpp, V, route, &b, base, &t->est_bpp);
  int32_t* fields = base;
  int32_t* sel = NULL;
  if (K > 1 && sweeps > 0 && nvec > 0) {
    sel = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)nvec);
    rdo_run(Wq, rows, cols, norms, s, b, K, sweeps, sel, NULL, NULL, NULL, NULL, NULL, NULL);
    uint32_t amax = max_coord_alphabet(sel, nvec), bf = b;
    while (amax > (1u << bf) && bf < 15) ++bf;
    if (amax <= (1u << bf)) {
      fields = sel;
      b = bf;
    }
  }
  int rc = finish_encode(Wq, rows, cols, s, b, V, fields, EPO_CODING_STANDARD, t);
  free(sel);
  free(base);
  free(norms);
  free(Wq);
  if (rc != 0) {
    epo_tensor_free(t);
    return rc;
  }
  *out = t;
  return 0;
}

int epo_rdo_trace(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t V,
                  uint32_t b0, int route, uint32_t K, double* D, int64_t* R, float* row_scales,
                  int64_t* budget, double* lambda, int32_t* sel, float* s_out, uint32_t* b_out) {
  if (rows <= 0 || cols <= 0 || cols % 8 != 0 || K < 1 || K > 32) return -1;
  if (V == 0) V = epo_default_vectors_per_tile(target_bpp);
  uint32_t b = b0 ? b0 : epo_default_prob_bits(target_bpp);
  epo_tensor* t = tensor_new(rows, cols, route);
  float* Wq = prepare_input(W, rows, cols, route, t);
  double* norms = (double*)malloc(sizeof(double) * (size_t)rows);
  epo_row_rms(Wq, rows, cols, norms);
  int64_t nvec = rows * (cols / 8);
  int32_t* fields = (int32_t*)malloc(sizeof(int32_t) * 9 * (size_t)nvec);
  float s = baseline_scale(Wq, rows, cols, norms, target_bpp, V, route, &b, fields, &t->est_bpp);
  rdo_run(Wq, rows, cols, norms, s, b, K, 1, fields, D, R, row_scales, budget, lambda, sel);
  *s_out = s;
  *b_out = b;
  free(fields);
  free(norms);
  free(Wq);
  epo_tensor_free(t);
  return 0;
}
