/*
 * Oracle: static frequency tables and the tiled, 32-way interleaved rANS
 * coder.  TEST INFRASTRUCTURE ONLY (see epo.h).
 *
 * Passages followed:
 *  - EntroPack paper, section 3.6 "Frequency tables and tiles": 17 shared
 *    integer tables (one for the coset bit c, two per coordinate field, one per
 *    coset), each coordinate table with a minimum-value offset for zero-based
 *    symbol indices; tiles of V vectors = 9V symbols; J = 32 interleaved rANS
 *    states per tile, one state per lane.
 *  - Appendix C.3 "State normalization": 32-bit states kept in [2^15, 2^31),
 *    16-bit payload words, probability precision b in 9..15 so that M = 2^b
 *    and at most one payload word moves per symbol.
 *  - Appendix C.1: b bounds how many distinct symbols can get a positive
 *    frequency.
 *  - Duda (2013), reference 14 of the paper: the rANS state update
 *    x' = floor(x / f) * M + (x mod f) + cum (encode) and
 *    x = f * floor(x' / M) + (x' mod M) - cum (decode).
 *
 * Readings where the pages are silent (listed in the design notes):
 *  - Lane l of a tile owns the tile's vectors l, l+32, l+64, ...; symbols are
 *    decoded vector-round by vector-round, and inside a round field by field
 *    (c, z1..z7, m), lanes in ascending order.  After each symbol a lane whose
 *    state dropped below 2^15 reads the next payload word; reads within one
 *    field step happen in ascending lane order.
 *  - The encoder starts every lane at 2^15, so a correctly decoded tile ends
 *    with every state back at 2^15 and every payload word consumed.
 *  - Frequency normalisation: f = max(1, floor(n * M / N)) for every observed
 *    symbol, 0 otherwise; a deficit goes to the most frequent symbol, an excess
 *    is removed one unit at a time from the currently largest frequency above 1
 *    (ties: lowest index).
 */
#include <stdlib.h>
#include <string.h>

#include "epo.h"

int epo_normalize_freqs(const uint64_t* counts, uint32_t A, uint32_t b, uint16_t* freqs) {
  const uint64_t M = 1ull << b;
  uint64_t N = 0, distinct = 0;
  for (uint32_t i = 0; i < A; ++i) {
    N += counts[i];
    distinct += counts[i] > 0;
  }
  for (uint32_t i = 0; i < A; ++i) freqs[i] = 0;
  if (N == 0) return 0;            /* empty table */
  if (distinct > M) return -1;     /* cannot give every observed symbol f >= 1 */

  uint32_t* f = (uint32_t*)malloc(sizeof(uint32_t) * (A ? A : 1));
  uint64_t sum = 0;
  for (uint32_t i = 0; i < A; ++i) {
    if (counts[i] == 0) {
      f[i] = 0;
    } else {
      uint64_t q = counts[i] * M / N;
      f[i] = (uint32_t)(q < 1 ? 1 : q);
    }
    sum += f[i];
  }
  if (sum < M) {
    uint32_t j = 0;
    for (uint32_t i = 1; i < A; ++i)
      if (counts[i] > counts[j]) j = i;
    f[j] += (uint32_t)(M - sum);
    sum = M;
  }
  if (sum > M) {
    /* candidates: indices whose frequency is still above one, in index order */
    uint32_t* cand = (uint32_t*)malloc(sizeof(uint32_t) * (A ? A : 1));
    uint32_t nc = 0;
    for (uint32_t i = 0; i < A; ++i)
      if (f[i] > 1) cand[nc++] = i;
    while (sum > M) {
      uint32_t best = 0;
      for (uint32_t k = 1; k < nc; ++k)
        if (f[cand[k]] > f[cand[best]]) best = k;   /* strict: lowest index wins ties */
      f[cand[best]] -= 1;
      sum -= 1;
      if (f[cand[best]] == 1) {
        memmove(cand + best, cand + best + 1, sizeof(uint32_t) * (nc - best - 1));
        nc -= 1;
      }
    }
    free(cand);
  }
  for (uint32_t i = 0; i < A; ++i) freqs[i] = (uint16_t)f[i];
  free(f);
  return 0;
}

/* cumulative frequencies of one table: cum[i] = f[0] + ... + f[i-1] */
static uint32_t* make_cum(const uint16_t* f, uint32_t A) {
  uint32_t* cum = (uint32_t*)malloc(sizeof(uint32_t) * (A + 1));
  cum[0] = 0;
  for (uint32_t i = 0; i < A; ++i) cum[i + 1] = cum[i] + f[i];
  return cum;
}

typedef struct {
  uint32_t b;
  uint32_t A[EPO_TABLES];
  const uint16_t* f[EPO_TABLES];
  uint32_t* cum[EPO_TABLES];
} tables_t;

static void tables_init(tables_t* t, const uint16_t* const* freq, const uint32_t* alphabet,
                        uint32_t b) {
  t->b = b;
  for (int k = 0; k < EPO_TABLES; ++k) {
    t->A[k] = alphabet[k];
    t->f[k] = freq[k];
    t->cum[k] = make_cum(freq[k], alphabet[k]);
  }
}

static void tables_free(tables_t* t) {
  for (int k = 0; k < EPO_TABLES; ++k) free(t->cum[k]);
}

/* Encode one tile: n vectors, sym[v*9 + f] = zero-based symbol of field f of
 * vector v (sym[v*9] is the coset bit).  Words are produced in reverse decode
 * order and reversed at the end. */
static int tile_encode(uint32_t n, const int32_t* sym, const tables_t* tb,
                       uint32_t states[EPO_LANES], uint16_t* words, uint32_t cap,
                       uint32_t* nwords) {
  const uint32_t b = tb->b;
  uint32_t x[EPO_LANES];
  for (int l = 0; l < EPO_LANES; ++l) x[l] = EPO_L;
  uint32_t K = (n + EPO_LANES - 1) / EPO_LANES;
  uint32_t np = 0;
  for (int64_t k = (int64_t)K - 1; k >= 0; --k) {
    for (int f = EPO_FIELDS - 1; f >= 0; --f) {
      for (int l = EPO_LANES - 1; l >= 0; --l) {
        uint64_t v = (uint64_t)k * EPO_LANES + (uint64_t)l;
        if (v >= n) continue;
        int c = sym[v * EPO_FIELDS + 0];
        if (c != 0 && c != 1) return -1;
        int t = epo_table_index(f, c);
        int32_t s = sym[v * EPO_FIELDS + f];
        if (s < 0 || (uint32_t)s >= tb->A[t] || tb->f[t][s] == 0) return -2;
        uint32_t fr = tb->f[t][s];
        uint32_t cm = tb->cum[t][s];
        uint64_t xmax = ((uint64_t)(EPO_L >> b) << 16) * fr;   /* 2^(31-b) * f */
        if ((uint64_t)x[l] >= xmax) {
          if (np >= cap) return -3;
          words[np++] = (uint16_t)(x[l] & 0xFFFFu);
          x[l] >>= 16;
        }
        x[l] = ((x[l] / fr) << b) + (x[l] % fr) + cm;
      }
    }
  }
  for (uint32_t i = 0; i < np / 2; ++i) {
    uint16_t tmp = words[i];
    words[i] = words[np - 1 - i];
    words[np - 1 - i] = tmp;
  }
  for (int l = 0; l < EPO_LANES; ++l) states[l] = x[l];
  *nwords = np;
  return 0;
}

/* largest s with cum[s] <= slot (never a zero-frequency symbol, see header) */
static uint32_t find_symbol(const uint32_t* cum, uint32_t A, uint32_t slot) {
  uint32_t lo = 0, hi = A;   /* answer in [lo, hi) */
  while (hi - lo > 1) {
    uint32_t mid = lo + (hi - lo) / 2;
    if (cum[mid] <= slot) lo = mid;
    else hi = mid;
  }
  return lo;
}

static int tile_decode(uint32_t n, const uint32_t states[EPO_LANES], const uint16_t* words,
                       uint32_t nwords, const tables_t* tb, int32_t* sym) {
  const uint32_t b = tb->b;
  const uint32_t mask = (1u << b) - 1u;
  uint32_t x[EPO_LANES];
  for (int l = 0; l < EPO_LANES; ++l) x[l] = states[l];
  uint32_t K = (n + EPO_LANES - 1) / EPO_LANES;
  uint32_t p = 0;
  for (uint32_t k = 0; k < K; ++k) {
    for (int f = 0; f < EPO_FIELDS; ++f) {
      for (int l = 0; l < EPO_LANES; ++l) {
        uint64_t v = (uint64_t)k * EPO_LANES + (uint64_t)l;
        if (v >= n) continue;
        int c = (f == 0) ? 0 : sym[v * EPO_FIELDS + 0];
        int t = epo_table_index(f, c);
        if (tb->A[t] == 0) return EPO_TILE_EMPTY_TABLE;
        uint32_t slot = x[l] & mask;
        uint32_t s = find_symbol(tb->cum[t], tb->A[t], slot);
        x[l] = (uint32_t)tb->f[t][s] * (x[l] >> b) + slot - tb->cum[t][s];
        sym[v * EPO_FIELDS + f] = (int32_t)s;
        if (x[l] < EPO_L) {
          if (p >= nwords) return EPO_TILE_OVERRUN;
          x[l] = (x[l] << 16) | words[p++];
        }
      }
    }
  }
  for (int l = 0; l < EPO_LANES; ++l)
    if (x[l] != EPO_L) return EPO_TILE_BAD_STATE;
  if (p != nwords) return EPO_TILE_BAD_LENGTH;
  return EPO_TILE_OK;
}

int epo_tile_encode(uint32_t n, const int32_t* sym, const uint8_t* coset,
                    const uint16_t* const* freq, const uint32_t* alphabet, uint32_t b,
                    uint32_t states[EPO_LANES], uint16_t* words, uint32_t cap,
                    uint32_t* nwords) {
  (void)coset;
  if (b < 9 || b > 15) return -4;
  tables_t tb;
  tables_init(&tb, freq, alphabet, b);
  int rc = tile_encode(n, sym, &tb, states, words, cap, nwords);
  tables_free(&tb);
  return rc;
}

int epo_tile_decode(uint32_t n, const uint32_t states[EPO_LANES], const uint16_t* words,
                    uint32_t nwords, const uint16_t* const* freq, const uint32_t* alphabet,
                    uint32_t b, int32_t* sym, uint8_t* coset) {
  if (b < 9 || b > 15) return -4;
  tables_t tb;
  tables_init(&tb, freq, alphabet, b);
  int rc = tile_decode(n, states, words, nwords, &tb, sym);
  tables_free(&tb);
  if (coset && rc == EPO_TILE_OK)
    for (uint32_t v = 0; v < n; ++v) coset[v] = (uint8_t)sym[v * EPO_FIELDS];
  return rc;
}

/* Internal entry points used by epo_codec.c with tables prepared once. */
void* epo__tables_new(const uint16_t* const* freq, const uint32_t* alphabet, uint32_t b) {
  tables_t* t = (tables_t*)malloc(sizeof(tables_t));
  tables_init(t, freq, alphabet, b);
  return t;
}
void epo__tables_free(void* t) {
  tables_free((tables_t*)t);
  free(t);
}
int epo__tile_encode(uint32_t n, const int32_t* sym, const void* tb, uint32_t* states,
                     uint16_t* words, uint32_t cap, uint32_t* nwords) {
  return tile_encode(n, sym, (const tables_t*)tb, states, words, cap, nwords);
}
int epo__tile_decode(uint32_t n, const uint32_t* states, const uint16_t* words,
                     uint32_t nwords, const void* tb, int32_t* sym) {
  return tile_decode(n, states, words, nwords, (const tables_t*)tb, sym);
}
