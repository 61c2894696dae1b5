/*
 * EntroPack CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar C implementation of what EntroPack computes, written
 * from the paper "EntroPack: Fast and Accurate Entropy-Coded Weight Compression
 * at Arbitrary Bitrates" (section 3 and appendix C) and the EntroPackPreQuants
 * model card (bpp and relative-L2 definitions).  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It shares
 * no code, header, table or constant with the GPU library.
 *
 * Floating point: encoder-side arithmetic (row statistics, lattice search,
 * scale search, least-squares row refit, rate estimate) is fp64.  The decode
 * side follows the stored FP32 scales: g = fp32(s * r_row), y = fp32(x * g),
 * then BF16 / FP8-e4m3 / INT8 rounding as documented in epo_convert.c.
 *
 * Pins (tests/test_oracle_*.py, tests/golden/): brute force and the E8
 * constants for the lattice, round trips and code-length bounds for rANS,
 * Table 5's tile accounting and Table 4's rate effects, closed forms for the
 * row statistics and the refit, library casts for every container rounding,
 * closed-form candidate ratios, recomputed distortions and brute-force
 * Lagrangian optimality for the per-row refinement.
 * Parity unpinned against the pages (they print no stream bytes, scales,
 * samples or estimates): the E8 tie-breaks, the frequency normalisation rule,
 * the scale search's row sample and rate estimator, and the byte layout; each
 * is pinned only by its invariants.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#ifndef EPO_H
#define EPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* rANS constants (paper, appendix C.3 "State normalization"): 32-bit states
 * kept in [2^15, 2^31), 16-bit payload words, J = 32 states per tile. */
#define EPO_L       32768u
#define EPO_LANES   32
#define EPO_FIELDS  9          /* c, z1..z7, m  (section 3.6: 9V symbols per tile) */
#define EPO_TABLES  17         /* 1 for c + 2 cosets x 8 coordinate fields */

/* Table index of field f (0 = c, 1..7 = z1..z7, 8 = m) for coset c. */
static inline int epo_table_index(int f, int c) { return f == 0 ? 0 : 1 + 2 * (f - 1) + c; }

/* Routes (paper, appendix B.1): direct, row-scaled FP8-e4m3, row-scaled INT8. */
enum { EPO_ROUTE_DIRECT = 0, EPO_ROUTE_FP8 = 1, EPO_ROUTE_INT8 = 2 };

/* Coding of the fields (paper, Table 4 and section "Parity reduction and coset
 * conditioning"): the method's 17 coset-conditioned tables with m = floor(z8/2)
 * as the eighth field, and the two ablations Table 4 measures on the same
 * quantised points -- 9 tables pooled over the two cosets, and z8 coded
 * directly instead of m. */
enum { EPO_CODING_STANDARD = 0, EPO_CODING_POOLED = 1, EPO_CODING_DIRECT_Z8 = 2 };

/* Decode output kinds. */
enum {
  EPO_OUT_BF16 = 0, EPO_OUT_FP8 = 1, EPO_OUT_INT8 = 2, EPO_OUT_FP16 = 3,
  EPO_OUT_UINT8 = 4,         /* unsigned 8-bit codes with offset 128 */
  EPO_OUT_LATTICE2X = 100,   /* int32, 2*x exactly */
  EPO_OUT_F32 = 101,         /* fp32 product x*g before container rounding */
  EPO_OUT_FIELDS = 102       /* int32 [nvec][9]: c, z1..z7, m */
};

/* Per-tile decode status. */
enum { EPO_TILE_OK = 0, EPO_TILE_BAD_STATE = 1, EPO_TILE_BAD_LENGTH = 2,
       EPO_TILE_OVERRUN = 3, EPO_TILE_EMPTY_TABLE = 4 };

typedef struct epo_tensor epo_tensor;

/* ---- lattice (epo_lattice.c) ---- */
void   epo_round_half_even(const double* x, int64_t n, double* out);
void   epo_d8_nearest(const double v[8], double y[8]);
int    epo_e8_nearest(const double v[8], double x[8]);
void   epo_e8_nearest_batch(const double* v, int64_t nvec, double* x, int32_t* coset);
void   epo_point_to_fields(const double x[8], int32_t fields[9]);
void   epo_fields_to_point(const int32_t fields[9], double x[8]);
void   epo_point_to_fields_batch(const double* x, int64_t nvec, int32_t* fields);
void   epo_fields_to_point_batch(const int32_t* fields, int64_t nvec, double* x);
void   epo_row_rms(const float* W, int64_t rows, int64_t cols, double* norms);

/* ---- rANS tables and tiles (epo_rans.c) ---- */
int    epo_normalize_freqs(const uint64_t* counts, uint32_t A, uint32_t b, uint16_t* freqs);
int    epo_tile_encode(uint32_t n, const int32_t* sym, const uint8_t* coset,
                       const uint16_t* const* freq, const uint32_t* alphabet, uint32_t b,
                       uint32_t states[EPO_LANES], uint16_t* words, uint32_t cap,
                       uint32_t* nwords);
int    epo_tile_decode(uint32_t n, const uint32_t states[EPO_LANES],
                       const uint16_t* words, uint32_t nwords,
                       const uint16_t* const* freq, const uint32_t* alphabet, uint32_t b,
                       int32_t* sym, uint8_t* coset);

/* ---- tensor codec (epo_codec.c) ---- */
uint32_t epo_default_vectors_per_tile(double target_bpp);
uint32_t epo_default_prob_bits(double target_bpp);
uint64_t epo_num_tiles(int64_t rows, int64_t cols, uint32_t V);
uint64_t epo_stored_bytes(int64_t rows, uint32_t T, uint64_t nwords,
                          const uint32_t alphabet[EPO_TABLES], int route);
void   epo_sample_rows(int64_t rows, int64_t cols, int64_t* picked, int64_t* npicked);
double epo_estimate_bpp(const float* W, int64_t rows, int64_t cols, const double* norms,
                        const int64_t* sample, int64_t nsample, double s, uint32_t b,
                        uint32_t V, int route);
int    epo_encode(const float* W, int64_t rows, int64_t cols, double target_bpp,
                  uint32_t V, uint32_t b0, int route, epo_tensor** out);
int    epo_encode_fixed_scale(const float* W, int64_t rows, int64_t cols, float s,
                              uint32_t V, uint32_t b, int route, epo_tensor** out);
/* epo_encode with a coding variant: the scale search, the points and the row
 * scales are the standard coding's; only the tables and the payload differ. */
int    epo_encode_coded(const float* W, int64_t rows, int64_t cols, double target_bpp,
                        uint32_t V, uint32_t b0, int route, int coding, epo_tensor** out);
int    epo_tensor_coding(const epo_tensor* t);
/* Stored bytes of a coded container: pooled tables store 8 coordinate tables. */
uint64_t epo_stored_bytes_coded(int64_t rows, uint32_t T, uint64_t nwords,
                                const uint32_t alphabet[EPO_TABLES], int route, int coding);
/* Per-row rate-distortion refinement (section 3.5, appendix C.2): K nested
 * candidate ratios, `sweeps` model-update / selection sweeps, then the same
 * container as epo_encode (standard coding) from the selected fields. */
void   epo_rdo_ratios(uint32_t K, double* rho);
int    epo_encode_rdo(const float* W, int64_t rows, int64_t cols, double target_bpp,
                      uint32_t V, uint32_t b0, int route, uint32_t K, uint32_t sweeps,
                      epo_tensor** out);
/* The first sweep's quantities: D, R [rows*K] (R in 2^-16 bit), candidate row
 * scales [rows*K], the budget, lambda and the selection [rows]; s and b of
 * the baseline. */
int    epo_rdo_trace(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t V,
                     uint32_t b0, int route, uint32_t K, double* D, int64_t* R, float* row_scales,
                     int64_t* budget, double* lambda, int32_t* sel, float* s_out, uint32_t* b_out);
void   epo_tensor_free(epo_tensor* t);
void   epo_tensor_info(const epo_tensor* t, int64_t* rows, int64_t* cols, uint32_t* V,
                       uint32_t* T, uint32_t* b, float* s, uint64_t* nwords,
                       uint32_t* nfreqs, int* route, double* est_bpp);
void   epo_tensor_tables(const epo_tensor* t, uint32_t* alphabet, int32_t* minval,
                         uint32_t* freq_base);
void   epo_tensor_copy(const epo_tensor* t, float* row_scales, float* route_scales,
                       uint32_t* states, uint32_t* offsets, uint16_t* payload,
                       uint16_t* freqs);
int    epo_decode(int64_t rows, int64_t cols, uint32_t V, uint32_t T, uint32_t b, float s,
                  const float* row_scales, const uint32_t* states, const uint32_t* offsets,
                  const uint16_t* payload, const uint16_t* freqs, const uint32_t* freq_base,
                  const uint32_t* alphabet, const int32_t* minval, int out_kind, void* out,
                  int32_t* tile_status, uint32_t tile_begin, uint32_t tile_end);
/* epo_decode of a coded container (EPO_CODING_DIRECT_Z8: field 8 holds z8). */
int    epo_decode_coded(int64_t rows, int64_t cols, uint32_t V, uint32_t T, uint32_t b, float s,
                        const float* row_scales, const uint32_t* states, const uint32_t* offsets,
                        const uint16_t* payload, const uint16_t* freqs, const uint32_t* freq_base,
                        const uint32_t* alphabet, const int32_t* minval, int coding, int out_kind,
                        void* out, int32_t* tile_status, uint32_t tile_begin, uint32_t tile_end);

/* ---- dtype conversion (epo_convert.c) ---- */
uint16_t epo_f32_to_bf16(float y);
uint8_t  epo_f32_to_fp8e4m3(float y);
int8_t   epo_f32_to_int8(float y);
uint8_t  epo_f32_to_uint8(float y);
void     epo_f32_to_uint8_batch(const float* y, int64_t n, uint8_t* out);
uint16_t epo_f32_to_f16(float y);
void     epo_f32_to_f16_batch(const float* y, int64_t n, uint16_t* out);
double   epo_fp8e4m3_value(uint8_t code);
void     epo_f32_to_bf16_batch(const float* y, int64_t n, uint16_t* out);
void     epo_f32_to_fp8e4m3_batch(const float* y, int64_t n, uint8_t* out);
void     epo_f32_to_int8_batch(const float* y, int64_t n, int8_t* out);
void     epo_route_precast(const float* W, int64_t rows, int64_t cols, int route,
                           float* Wq, float* qscale);

/* ---- metrics (epo_convert.c) ---- */
double epo_bpp(const uint64_t* stored_bytes, const uint64_t* numel, int n);
double epo_rel_l2(const float* Wq, const float* W, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
