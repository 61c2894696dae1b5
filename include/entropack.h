/*
 * entropack.h -- C ABI of the MI355X (gfx950) EntroPack weight decoder.
 *
 * The decoder implements the reconstruction path of "EntroPack: Fast and
 * Accurate Entropy-Coded Weight Compression at Arbitrary Bitrates"
 * (Figure 2(b); sections 3.1, 3.6; appendix C.3): for every independent tile
 * it decodes the rANS symbols, rebuilds the E8 lattice points from the
 * parity-reduced fields (c, z1..z7, m), multiplies them by the per-tensor
 * quantisation scale and the fitted per-row scale, and writes BF16, FP8-e4m3
 * or INT8 weights, in one kernel pass with no intermediate symbol tensor and
 * no codebook.
 *
 * Stream format (section 3.6 and appendix C.3 of the paper; the byte order of
 * the fields is this library's, the pages print none):
 *   - tensor [rows, cols] row-major, cols % 8 == 0; vector g covers
 *     elements 8g .. 8g+7 of the flattened tensor (blocks of eight weights);
 *   - tiles of V vectors (32 <= V <= 7200), num_tiles = ceil(rows*cols/8 / V); the
 *     last tile may be partial; tiles may cross row boundaries;
 *   - per tile: 32 u32 terminal rANS states (lane order) and a u32 offset of
 *     the tile's 16-bit payload words; one final offset closes the payload;
 *   - lane l of a tile owns the tile's vectors l, l+32, ...; symbols are coded
 *     vector round by vector round, field by field (c, z1..z7, m), lanes in
 *     ascending order; states live in [2^15, 2^31); after each symbol a lane
 *     whose state fell below 2^15 reads the next payload word;
 *   - 17 static frequency tables, M = 2^prob_bits, prob_bits in 9..15: table 0
 *     codes the coset bit c (alphabet 2), table 1 + 2*(f-1) + c codes field f
 *     (1..7 = z1..z7, 8 = m) of vectors in coset c; symbol i of table k stands
 *     for the value i + min_offset[k]; alphabet[k] = 0 marks an empty table;
 *   - reconstruction: z8 = 2m + ((z1 + ... + z7) & 1) (or z8 as stored, see
 *     ep_tensor_desc.field8), x_i = z_i + c/2,
 *     y = fp32(x_i * fp32(scale * row_scales[row])), then the container
 *     rounding (BF16 round-to-nearest-even; FP8 OCP e4m3fn clamped to +-448
 *     then round-to-nearest-even; INT8 round-half-even then clamp to
 *     [-128, 127]; UINT8 the same integer plus the offset 128, clamped to
 *     [0, 255], the unsigned container of appendix A.6).
 *
 * Ownership: the caller owns every buffer.  Device pointers must stay valid
 * until the work enqueued on `stream` has finished.  The library never
 * allocates or frees device memory and never synchronises the stream; all
 * GPU work is enqueued asynchronously on `stream` (a hipStream_t, NULL = the
 * default stream).  Host arrays passed in (descriptors, dtype and pointer
 * lists) are read before the call returns.
 *
 * Errors: argument problems are reported synchronously as a negative
 * ep_status before any GPU work is enqueued.  Corrupt streams are reported per
 * tile in the optional tile_status arrays; a corrupt tile's output region is
 * left undefined, but every read stays inside the tensor's payload buffer and
 * every write inside the tensor's output.
 */
#ifndef ENTROPACK_H
#define ENTROPACK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 3
#define EP_NUM_TABLES 17
#define EP_LANES 32

typedef enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = -1,   /* a descriptor or argument violates the format above */
  EP_ERR_UNSUPPORTED = -2,   /* valid format, but outside what this build supports */
  EP_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than ep_workspace_size() */
  EP_ERR_HIP = -4            /* a HIP runtime call failed (message: ep_last_error()) */
} ep_status;

typedef enum {
  EP_OUT_BF16 = 0,           /* uint16 bit patterns, [rows, cols] */
  EP_OUT_FP8_E4M3 = 1,       /* uint8 OCP e4m3fn codes, [rows, cols] */
  EP_OUT_INT8 = 2,           /* int8 codes, [rows, cols] */
  EP_OUT_FP16 = 3,           /* uint16 IEEE binary16 bit patterns (RNE, overflow to inf), [rows, cols] */
  EP_OUT_FP32 = 4,           /* float32 products y = fp32(x * fp32(s * r_row)), [rows, cols] */
  EP_OUT_UINT8 = 5,          /* uint8 codes with offset 128: rint(y) + 128 clamped to [0, 255], [rows, cols] */
  EP_OUT_LATTICE2X_I32 = 100 /* int32 2*x_i (exact lattice coordinates), for tests */
} ep_out_dtype;

/* Per-tile status values written to tile_status[t]. */
typedef enum {
  EP_TILE_OK = 0,
  EP_TILE_BAD_STATE = 1,     /* a lane did not end at 2^15 */
  EP_TILE_BAD_LENGTH = 2,    /* payload words left over */
  EP_TILE_OVERRUN = 3,       /* a read would have left the tile's payload range */
  EP_TILE_EMPTY_TABLE = 4    /* a vector decoded into a coset whose table is empty */
} ep_tile_status;

/* One compressed tensor.  Pointers are device pointers. */
typedef struct {
  int64_t rows;                       /* >= 0 */
  int64_t cols;                       /* > 0, multiple of 8; (rows*cols/8 + 64*V + 64) * 32 < 2^32 */
  uint32_t vectors_per_tile;          /* 32 <= V <= 7200 */
  uint32_t num_tiles;                 /* must equal ceil(rows*cols/8 / V) */
  uint32_t prob_bits;                 /* b in [9, 15] */
  float scale;                        /* per-tensor quantisation scale s */
  const float* row_scales;            /* [rows] fitted FP32 row scales */
  const uint32_t* tile_states;        /* [num_tiles * 32] terminal states, lane order */
  const uint32_t* tile_offsets;       /* [num_tiles + 1] offsets in 16-bit words, nondecreasing */
  const uint16_t* payload;            /* [payload_words] words, 16-byte aligned; the buffer must be
                                         readable up to payload_words rounded up to a multiple of 8 */
  uint64_t payload_words;             /* words in the payload; tile ranges beyond it are flagged */
  const uint16_t* freqs;              /* the 17 tables' frequencies, table k at freq_base[k] */
  uint32_t freq_base[EP_NUM_TABLES];  /* start of table k in freqs */
  uint32_t alphabet[EP_NUM_TABLES];   /* A_k <= 2^b; alphabet[0] == 2; 0 = empty table */
  int32_t min_offset[EP_NUM_TABLES];  /* value of symbol 0 of table k (min_offset[0] == 0);
                                         -2^19 <= min_offset[k] and min_offset[k] + A_k <= 2^19,
                                         which keeps every reconstructed 4z + c exact in fp32 */
  uint32_t field8;                    /* EP_FIELD8_M (0): field 8 is m = floor(z8 / 2), the
                                         method's parity-reduced field; EP_FIELD8_Z8 (1): field 8
                                         is z8 itself (the direct-z8 ablation of the paper's
                                         Table 4); other values are rejected */
} ep_tensor_desc;

#define EP_FIELD8_M 0u
#define EP_FIELD8_Z8 1u

/* Human-readable name of a status code (static string). */
const char* ep_status_string(int status);

/* Text of the last EP_ERR_HIP or EP_ERR_INVALID_ARG in this thread (static per thread). */
const char* ep_last_error(void);

/* EP_ABI_VERSION of the loaded library. */
int ep_abi_version(void);

/*
 * Bytes of device workspace ep_decode_batch needs for these n tensors
 * (descriptors, per-tensor decode tables, the tile schedule and its work
 * counters).  Reads only the host-side fields of the descriptors.  Returns
 * EP_OK or EP_ERR_INVALID_ARG; *bytes is set on success.
 */
int ep_workspace_size(const ep_tensor_desc* descs, int n, size_t* bytes);

/*
 * Decode n tensors in one launch sequence on `stream`.
 *   descs[i]       host array of n descriptors (device pointers inside)
 *   dtypes[i]      ep_out_dtype of tensor i
 *   outs[i]        device output of tensor i, [rows, cols] of the dtype's element
 *   tile_status    NULL, or host array of n device pointers (each NULL or int32[num_tiles])
 *   workspace      device buffer of at least ep_workspace_size(descs, n) bytes,
 *                  256-byte aligned; reused and overwritten by every call
 *                  (the decode kernel also updates work counters there)
 *   stream         hipStream_t
 * Calls that share a workspace must be ordered on one stream.
 */
int ep_decode_batch(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                    int32_t* const* tile_status, int n, void* workspace, size_t ws_bytes,
                    void* stream);

/* ep_decode_batch for a single tensor. */
int ep_decode_tensor(const ep_tensor_desc* desc, int dtype, void* out, int32_t* tile_status,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code recorded under stream
 * capture, serving loops that must not allocate, harnesses that forbid
 * hipMalloc.  ep_decode_batch with the library's own workspace, a static
 * device array of EP_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
 * holds from the loading of the library's device code until the process ends.
 * The call allocates no device memory; its address lookup happens once per
 * device, on the first call with that device current.  Buffers and `stream`
 * must belong to the current device.
 *   Limit: batches whose ep_workspace_size() exceeds EP_NOALLOC_SCRATCH_BYTES
 *   are rejected with EP_ERR_WORKSPACE before any GPU work (split them, or use
 *   ep_decode_batch).
 *   Sharing: all calls on one GPU use that GPU's one array, which keeps the
 *   last call's contents; every byte a call reads there it has written first,
 *   except three flag words per tensor, which choose between exact decode
 *   paths (a leftover value can at worst choose the slower one).
 *   Calls that overlap on one GPU (on different streams, or from host threads
 *   without ordering) race on the array and give undefined results: order
 *   them on one stream.
 *   Stream capture: a batch of at most 6 tensors records only kernel launches
 *   (its descriptors travel as kernel arguments); a larger batch also records
 *   a copy from a host buffer that lives only for the call, so a graph that
 *   holds one must not be replayed.
 * Other arguments, errors and tile statuses: as ep_decode_batch.
 */
#define EP_NOALLOC_SCRATCH_BYTES (64u << 20)
int ep_decode_batch_noalloc(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                            int32_t* const* tile_status, int n, void* stream);

/*
 * The two halves of ep_decode_batch, for callers that time the decode kernel
 * on its own.  ep_batch_prepare validates the arguments and enqueues the
 * build of the decode tables and the tile schedule (for a batch of at most 6
 * tensors the descriptors are that kernel's arguments; a larger batch copies
 * them to the workspace first); ep_batch_launch enqueues the fused decode
 * kernel.  `plan` is caller-owned host memory filled by
 * prepare; launch must follow its prepare on the same stream with the same
 * workspace.
 */
typedef struct {
  uint64_t opaque[256];
} ep_batch_plan;

/*
 * Container rounding on its own: out[i] = the dtype's code of the fp32 value
 * in[i], computed with the decode kernel's device conversions (the rules at
 * the top of this file), for callers that hold fp32 products and for testing
 * the rounding in isolation.  in: device float32 [n], 16-byte aligned; out:
 * device [n] of the dtype's element (BF16 / FP16 uint16 bit patterns, FP8 /
 * INT8 / UINT8 bytes), 8-byte aligned; n a multiple of 4.  dtype is one of
 * EP_OUT_BF16, EP_OUT_FP16, EP_OUT_FP8_E4M3, EP_OUT_INT8, EP_OUT_UINT8.
 * Enqueued on `stream`.
 */
int ep_convert_f32(const float* in, void* out, uint64_t n, int dtype, void* stream);

int ep_batch_prepare(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                     int32_t* const* tile_status, int n, void* workspace, size_t ws_bytes,
                     void* stream, ep_batch_plan* plan);
int ep_batch_launch(const ep_batch_plan* plan, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ENTROPACK_H */
