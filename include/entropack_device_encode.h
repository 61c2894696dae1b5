/*
 * entropack_device_encode.h -- C ABI of the EntroPack compressor that runs on
 * the MI355X (gfx950), exported by the same library as the decoder
 * (entropack.h).
 *
 * It runs the encoding pipeline of "EntroPack: Fast and Accurate
 * Entropy-Coded Weight Compression at Arbitrary Bitrates" (Figure 2(a),
 * sections 3.1-3.6, appendix C.1 and C.3, appendix B.1 for the FP8 / INT8
 * route pre-casts) and produces the same container as ep_encode_host
 * (entropack_encode.h), byte for byte: same scale, precision, tables, row
 * scales, states, offsets and payload.  The quantisation, histograms, row
 * refit and tile encoding run in kernels; the scale search's decisions
 * (row sample, rate estimate from exact symbol counts, bisection, precision
 * escalation, frequency normalisation) run on the calling host thread.
 *
 * Inputs must be finite.  Statuses are those of entropack.h; EP_ERR_HIP and
 * EP_ERR_INVALID_ARG leave a message for ep_last_error().
 */
#ifndef ENTROPACK_DEVICE_ENCODE_H
#define ENTROPACK_DEVICE_ENCODE_H

#include <stddef.h>
#include <stdint.h>

#include "entropack.h"
#include "entropack_encode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Device workspace bytes ep_encode_device needs for a rows x cols tensor at
 * this target, tile size (0 = the target's default) and route.  Host-only
 * arithmetic.  About 4.5 bytes per weight for the quantised fields, 2.25 for
 * the per-tile word scratch (9 V words per tile), 4 more with a route
 * pre-cast, plus the histogram bound (16 alphabets of up to
 * 2 * 1000 * sqrt(cols) symbols) and small per-row and per-tile arrays.
 */
int ep_encode_device_workspace_size(int64_t rows, int64_t cols, double target_bpp,
                                    uint32_t vectors_per_tile, int route, size_t* bytes);

/*
 * Compress the device float32 matrix W [rows, cols] (row-major, 16-byte
 * aligned, cols % 8 == 0).  target_bpp, vectors_per_tile, prob_bits and
 * route mean what they mean for ep_encode_host; coding is an ep_coding (the
 * ablations reuse the standard coding's scale, points and row scales; an
 * ablation whose alphabet outgrows 2^b returns EP_ERR_UNSUPPORTED).
 * workspace: device buffer of at least ep_encode_device_workspace_size()
 * bytes, 256-byte aligned; it holds
 * the encoded arrays afterwards.  The call enqueues its kernels on `stream`
 * (a hipStream_t) and synchronises that stream several times: it returns when
 * the tensor is encoded, with the header written to *info.  A later call on
 * the same workspace overwrites the result.
 */
int ep_encode_device(const float* W, int64_t rows, int64_t cols, double target_bpp,
                     uint32_t vectors_per_tile, uint32_t prob_bits, int route, int coding,
                     void* workspace, size_t ws_bytes, void* stream, ep_encoded_info* info);

/*
 * Device workspace bytes ep_encode_device_rdo needs with `candidates`
 * resolutions per row: the ep_encode_device_workspace_size() bytes, then the
 * candidates' fields (about 36 bytes per 8 weights each), their row scales,
 * distortions and rates (20 bytes per row each), the choices and a cost
 * table.  Host-only arithmetic; candidates in [1, 32].
 */
int ep_encode_device_rdo_workspace_size(int64_t rows, int64_t cols, double target_bpp,
                                        uint32_t vectors_per_tile, int route, uint32_t candidates,
                                        size_t* bytes);

/*
 * ep_encode_device (standard coding) with the optional per-row
 * rate-distortion refinement of the paper's section 3.5 and appendix C.2
 * (Algorithm 2): after the scale search, every row may take one of
 * `candidates` resolutions rho_k * s (rho_1 = 1, nested bisections of
 * [0.70, 1.45] in log scale) with its own fitted row scale; `sweeps` rounds
 * each rebuild the shared probability model from the selected fields and
 * reselect all rows under one rate penalty, keeping the baseline's total code
 * length.  The container is decoded like any other (only the encoder's
 * choices change), and ep_encode_device_emit reads it from the same
 * workspace.  candidates = 1 or sweeps = 0 give ep_encode_device's container.
 * The result is byte-identical to the CPU reference refinement.  Synchronises
 * `stream` like ep_encode_device, a few more times per sweep.
 */
int ep_encode_device_rdo(const float* W, int64_t rows, int64_t cols, double target_bpp,
                         uint32_t vectors_per_tile, uint32_t prob_bits, int route,
                         uint32_t candidates, uint32_t sweeps, void* workspace, size_t ws_bytes,
                         void* stream, ep_encoded_info* info);

/*
 * Copy the result of the last ep_encode_device on `workspace` (described by
 * its *info) into caller device buffers, enqueued asynchronously on `stream`;
 * any pointer may be NULL.  Sizes: row_scales and route_scales [rows] (the
 * latter only with a route), states [num_tiles * 32], offsets [num_tiles + 1],
 * payload [payload_words], freqs [num_freqs].  The payload words are gathered
 * from the per-tile scratch by a kernel; everything else is a device copy.
 */
int ep_encode_device_emit(const void* workspace, const ep_encoded_info* info, float* row_scales,
                          float* route_scales, uint32_t* states, uint32_t* offsets,
                          uint16_t* payload, uint16_t* freqs, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ENTROPACK_DEVICE_ENCODE_H */
