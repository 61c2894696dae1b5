/*
 * entropack_encode.h -- C ABI of the host-side EntroPack compressor that
 * produces the streams the MI355X decoder (entropack.h) consumes.
 *
 * It follows the encoding pipeline of "EntroPack: Fast and Accurate
 * Entropy-Coded Weight Compression at Arbitrary Bitrates" (Figure 2(a),
 * sections 3.1-3.6, appendix C): row normalisation, nearest-E8 quantisation
 * of blocks of eight weights, parity-reduced fields, sampled scale search with
 * probability-precision escalation and scale coarsening, per-row least-squares
 * reconstruction scales, 17 coset-conditioned static tables and 32-lane
 * interleaved rANS tiles.  Optional route pre-casts convert the input to
 * row-scaled FP8-e4m3 or INT8 values first (appendix B.1).
 *
 * Everything runs on host threads; inputs and outputs are host memory owned by
 * the caller except the opaque encoded tensor, which the library allocates
 * and ep_encoded_free releases.  Functions return EP_OK (0) or a negative
 * status (see entropack.h); ep_last_error-style messages are not kept.
 */
#ifndef ENTROPACK_ENCODE_H
#define ENTROPACK_ENCODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { EP_ROUTE_DIRECT = 0, EP_ROUTE_FP8 = 1, EP_ROUTE_INT8 = 2 } ep_route;

/* Field coding: the method's (17 coset-conditioned tables, m = floor(z8/2) as
 * the eighth field) and the two ablations of the paper's Table 4, which keep
 * the method's quantised points and row scales.  A pooled container lists the
 * shared table under both cosets (equal freq_base, alphabet and min_offset);
 * a direct-z8 container is decoded with ep_tensor_desc.field8 = EP_FIELD8_Z8. */
typedef enum { EP_CODING_STANDARD = 0, EP_CODING_POOLED = 1, EP_CODING_DIRECT_Z8 = 2 } ep_coding;

typedef struct ep_encoded ep_encoded;

typedef struct {
  int64_t rows, cols;
  uint32_t vectors_per_tile, num_tiles, prob_bits;
  float scale;
  int32_t route;
  double estimated_bpp;        /* the scale search's final sampled estimate */
  uint64_t payload_words;
  uint32_t num_freqs;          /* entries in the concatenated frequency tables */
  uint64_t stored_bytes;       /* full stored size (header, tables, scales, tiles, payload) */
  uint32_t alphabet[17];
  int32_t min_offset[17];
  uint32_t freq_base[17];
  int32_t coding;              /* ep_coding (the host compressor always writes EP_CODING_STANDARD) */
} ep_encoded_info;

/*
 * Compress a host float32 matrix W [rows, cols] (row-major, cols % 8 == 0).
 *   target_bpp         requested stored rate (bits per weight, all side information included)
 *   vectors_per_tile   V >= 32, or 0 for the default of the target (appendix C.3, Table 5)
 *   prob_bits          starting b in [9, 15], or 0 for the default (11 up to 7 bpp, else 12)
 *   route              ep_route
 *   threads            worker threads (0 = hardware concurrency)
 * On success *out holds the encoded tensor.
 */
int ep_encode_host(const float* W, int64_t rows, int64_t cols, double target_bpp,
                   uint32_t vectors_per_tile, uint32_t prob_bits, int route, int threads,
                   ep_encoded** out);

/* Header information of an encoded tensor. */
int ep_encoded_get_info(const ep_encoded* e, ep_encoded_info* info);

/*
 * Copy the encoded arrays into caller buffers (any pointer may be NULL):
 * row_scales [rows], route_scales [rows] (FP8/INT8 routes), states [num_tiles*32],
 * offsets [num_tiles+1], payload [payload_words], freqs [num_freqs].
 */
int ep_encoded_copy(const ep_encoded* e, float* row_scales, float* route_scales,
                    uint32_t* states, uint32_t* offsets, uint16_t* payload, uint16_t* freqs);

void ep_encoded_free(ep_encoded* e);

#ifdef __cplusplus
}
#endif
#endif /* ENTROPACK_ENCODE_H */
