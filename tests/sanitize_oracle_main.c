/*
 * Memory- and UB-safety driver for the CPU oracle, built with
 * -fsanitize=address,undefined by tests/test_oracle_sanitized.py.
 *
 * It compresses small seeded matrices with every coding, route and a few
 * precisions, decodes them to every output kind, then decodes damaged copies
 * (flipped payload bits, shortened and swapped offsets, altered states, a
 * payload cut short) with per-tile status.  The sanitizers abort on any
 * out-of-bounds access, leak or undefined operation; the driver itself checks
 * that intact containers decode with every tile OK, that every status is a
 * defined code, and that most damaged tiles are flagged.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "epo.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {   /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

/* heavy-tailed test weights: a sum of uniforms divided by a positive uniform */
static void fill_weights(float* W, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    double a = uniform() + uniform() + uniform() - 1.5;
    W[i] = (float)(0.02 * a / (0.25 + uniform()));
  }
}

typedef struct {
  int64_t rows, cols;
  uint32_t V, T, b, nfreqs;
  float s;
  uint64_t nwords;
  int route;
  double est;
  float* row_scales;
  float* route_scales;
  uint32_t* states;
  uint32_t* offsets;
  uint16_t* payload;
  uint16_t* freqs;
  uint32_t alphabet[EPO_TABLES], freq_base[EPO_TABLES];
  int32_t minval[EPO_TABLES];
} container;

static int failures = 0;

#define CHECK(cond, ...)               \
  do {                                 \
    if (!(cond)) {                     \
      fprintf(stderr, __VA_ARGS__);    \
      fputc('\n', stderr);             \
      ++failures;                      \
    }                                  \
  } while (0)

static void unpack(const epo_tensor* t, container* c) {
  epo_tensor_info(t, &c->rows, &c->cols, &c->V, &c->T, &c->b, &c->s, &c->nwords, &c->nfreqs,
                  &c->route, &c->est);
  epo_tensor_tables(t, c->alphabet, c->minval, c->freq_base);
  c->row_scales = malloc(sizeof(float) * (size_t)(c->rows > 0 ? c->rows : 1));
  c->route_scales = malloc(sizeof(float) * (size_t)(c->rows > 0 ? c->rows : 1));
  c->states = malloc(sizeof(uint32_t) * EPO_LANES * (size_t)(c->T > 0 ? c->T : 1));
  c->offsets = malloc(sizeof(uint32_t) * ((size_t)c->T + 1));
  /* exact sizes, so that the sanitizer sees any read past the payload */
  c->payload = malloc(sizeof(uint16_t) * (size_t)(c->nwords > 0 ? c->nwords : 1));
  c->freqs = malloc(sizeof(uint16_t) * (size_t)(c->nfreqs > 0 ? c->nfreqs : 1));
  epo_tensor_copy(t, c->row_scales, c->route == EPO_ROUTE_DIRECT ? NULL : c->route_scales,
                  c->states, c->offsets, c->payload, c->freqs);
}

static void release(container* c) {
  free(c->row_scales);
  free(c->route_scales);
  free(c->states);
  free(c->offsets);
  free(c->payload);
  free(c->freqs);
}

static size_t out_bytes(int kind, uint64_t numel) {
  switch (kind) {
    case EPO_OUT_FP8: case EPO_OUT_INT8: case EPO_OUT_UINT8: return (size_t)numel;
    case EPO_OUT_BF16: case EPO_OUT_FP16: return 2 * (size_t)numel;
    case EPO_OUT_FIELDS: return sizeof(int32_t) * 9 * (size_t)(numel / 8);
    default: return 4 * (size_t)numel;
  }
}

/* Decode all tiles; returns the number of tiles not OK (or -1 on an argument
 * error).  Statuses must be defined codes. */
static int decode_all(const container* c, int coding, int kind, const uint16_t* payload) {
  const uint64_t numel = (uint64_t)c->rows * (uint64_t)c->cols;
  void* out = malloc(out_bytes(kind, numel) + 1);
  int32_t* st = malloc(sizeof(int32_t) * (size_t)(c->T > 0 ? c->T : 1));
  int rc = epo_decode_coded(c->rows, c->cols, c->V, c->T, c->b, c->s, c->row_scales, c->states,
                            c->offsets, payload, c->freqs, c->freq_base, c->alphabet, c->minval,
                            coding, kind, out, st, 0, c->T);
  int bad = 0;
  if (rc != 0) bad = -1;
  else
    for (uint32_t t = 0; t < c->T; ++t) {
      CHECK(st[t] >= EPO_TILE_OK && st[t] <= EPO_TILE_EMPTY_TABLE, "undefined status %d", st[t]);
      bad += st[t] != EPO_TILE_OK;
    }
  free(out);
  free(st);
  return bad;
}

static void damaged_copies(const container* c, int coding) {
  if (c->T == 0 || c->nwords == 0) return;
  int flagged = 0, trials = 0;
  uint16_t* pl = malloc(sizeof(uint16_t) * (size_t)c->nwords);
  /* flipped payload bits, one tile at a time */
  for (int i = 0; i < 24; ++i) {
    memcpy(pl, c->payload, sizeof(uint16_t) * (size_t)c->nwords);
    uint64_t w = next_u64() % c->nwords;
    pl[w] ^= (uint16_t)(1u << (next_u64() % 16));
    int bad = decode_all(c, coding, EPO_OUT_BF16, pl);
    CHECK(bad >= 0, "argument error on a flipped bit");
    flagged += bad > 0;
    ++trials;
  }
  /* a payload shorter than the offsets claim: the last tile's words are cut */
  {
    container d = *c;
    d.nwords = c->nwords - 1;
    uint16_t* cut = malloc(sizeof(uint16_t) * (size_t)(d.nwords > 0 ? d.nwords : 1));
    memcpy(cut, c->payload, sizeof(uint16_t) * (size_t)d.nwords);
    uint32_t* off = malloc(sizeof(uint32_t) * ((size_t)c->T + 1));
    memcpy(off, c->offsets, sizeof(uint32_t) * ((size_t)c->T + 1));
    off[c->T] = (uint32_t)d.nwords;     /* the container must be self-consistent in size */
    d.offsets = off;
    int bad = decode_all(&d, coding, EPO_OUT_LATTICE2X, cut);
    CHECK(bad >= 0, "argument error on a shortened last tile");
    flagged += bad > 0;
    ++trials;
    free(cut);
    free(off);
  }
  /* swapped neighbouring offsets (a negative tile length) */
  if (c->T >= 2) {
    container d = *c;
    uint32_t* off = malloc(sizeof(uint32_t) * ((size_t)c->T + 1));
    memcpy(off, c->offsets, sizeof(uint32_t) * ((size_t)c->T + 1));
    uint32_t t = (uint32_t)(next_u64() % (c->T - 1)) + 1;
    if (off[t] != off[t + 1]) {
      uint32_t tmp = off[t];
      off[t] = off[t + 1];
      off[t + 1] = tmp;
      d.offsets = off;
      int bad = decode_all(&d, coding, EPO_OUT_FP8, c->payload);
      CHECK(bad > 0, "swapped offsets not flagged");
      ++trials;
      flagged += bad > 0;
    }
    free(off);
  }
  /* altered initial states */
  for (int i = 0; i < 8; ++i) {
    container d = *c;
    uint32_t* st = malloc(sizeof(uint32_t) * EPO_LANES * (size_t)c->T);
    memcpy(st, c->states, sizeof(uint32_t) * EPO_LANES * (size_t)c->T);
    uint64_t j = next_u64() % ((uint64_t)EPO_LANES * c->T);
    st[j] ^= 1u << (next_u64() % 31);
    d.states = st;
    int bad = decode_all(&d, coding, EPO_OUT_INT8, c->payload);
    CHECK(bad >= 0, "argument error on an altered state");
    flagged += bad > 0;
    ++trials;
    free(st);
  }
  free(pl);
  CHECK(2 * flagged > trials, "only %d of %d damaged containers flagged", flagged, trials);
}

static void one_case(int64_t rows, int64_t cols, double target, uint32_t V, uint32_t b, int route,
                     int coding, int rdo) {
  float* W = malloc(sizeof(float) * (size_t)(rows * cols));
  fill_weights(W, rows * cols);
  epo_tensor* t = NULL;
  int rc = rdo ? epo_encode_rdo(W, rows, cols, target, V, b, route, 3, 1, &t)
               : epo_encode_coded(W, rows, cols, target, V, b, route, coding, &t);
  CHECK(rc == 0 && t, "encode failed: %lldx%lld target %.1f route %d coding %d rdo %d",
        (long long)rows, (long long)cols, target, route, coding, rdo);
  if (rc == 0 && t) {
    container c;
    unpack(t, &c);
    static const int kinds[] = {EPO_OUT_BF16, EPO_OUT_FP8, EPO_OUT_INT8, EPO_OUT_FP16,
                                EPO_OUT_UINT8, EPO_OUT_LATTICE2X, EPO_OUT_F32, EPO_OUT_FIELDS};
    for (size_t k = 0; k < sizeof(kinds) / sizeof(kinds[0]); ++k) {
      int bad = decode_all(&c, coding, kinds[k], c.payload);
      CHECK(bad == 0, "intact container: %d tiles not OK (kind %d)", bad, kinds[k]);
    }
    damaged_copies(&c, coding);
    release(&c);
    epo_tensor_free(t);
  }
  free(W);
}

int main(void) {
  /* precisions, ragged last tiles, every coding and route, the refinement */
  one_case(24, 64, 4.0, 40, 0, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 0);
  one_case(17, 48, 2.0, 33, 9, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 0);
  one_case(20, 80, 8.0, 64, 0, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 0);
  one_case(12, 96, 6.0, 50, 15, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 0);
  one_case(16, 64, 4.0, 32, 0, EPO_ROUTE_FP8, EPO_CODING_STANDARD, 0);
  one_case(16, 64, 4.0, 45, 0, EPO_ROUTE_INT8, EPO_CODING_STANDARD, 0);
  one_case(24, 64, 4.0, 40, 0, EPO_ROUTE_DIRECT, EPO_CODING_POOLED, 0);
  one_case(24, 64, 4.0, 40, 0, EPO_ROUTE_DIRECT, EPO_CODING_DIRECT_Z8, 0);
  one_case(32, 64, 3.0, 48, 0, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 1);
  one_case(1, 8, 4.0, 32, 0, EPO_ROUTE_DIRECT, EPO_CODING_STANDARD, 0);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
