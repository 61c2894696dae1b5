// Fused EntroPack weight reconstruction for MI355X (gfx950).
//
// Implements the decoding path of "EntroPack: Fast and Accurate Entropy-Coded
// Weight Compression at Arbitrary Bitrates" (Figure 2(b), sections 3.1 and
// 3.6, appendix C.3): rANS symbol decoding of independent tiles, algebraic
// reconstruction of E8 points from the parity-reduced fields, per-row
// rescaling and container rounding, fused in one kernel.  The stream format
// and the ABI are documented in include/entropack.h.
//
// Mapping: one wave64 decodes two tiles, one per half-wave; lane l of a half
// owns the tile's rANS state l (the paper assigns one tile per 32-lane warp and
// one state per lane).  Workgroups of 16 waves are persistent, keep the
// current tensor's decode tables in LDS and hand out pairs of tiles to their
// waves through a work counter; each tile streams its payload words through a
// small LDS ring.  Renormalisation reads of a half-wave are located with a
// wave ballot (the popcount of the half's bits below the lane), so the lanes
// that need a word read consecutive ring positions.  Each lane reconstructs
// whole 8-wide vectors and writes them
// with one 16-byte (BF16) or 8-byte (FP8/INT8) buffer store; the 32 lanes of a
// half write 512 (256) contiguous bytes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>

#include "entropack.h"

// global (not flat) addressing for pointers read from the descriptors
#define EP_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr uint32_t kL = 1u << 15;          // lower bound of the state interval
constexpr int kTables = EP_NUM_TABLES;
constexpr int kTilesPerWave = 2;
constexpr int kWavesPerBlock = 16;
constexpr int kBlock = 64 * kWavesPerBlock;
constexpr int kTilesPerChunk = kTilesPerWave * kWavesPerBlock;
constexpr size_t kMaxLds = 160 * 1024;

// ---------------------------------------------------------------- decode tables
// Three layouts of a tensor's coordinate tables t = 2*(field-1) + coset:
//   packed    (LDS, b <= 11, alphabets <= 512): one u32 per slot of each table,
//             (slot - cum) | f << 11 | symbol << 23, so that the state update
//             is one multiply-add after a single lookup; the symbol's value
//             follows from the entry and a per-table constant (kvals).
//   packed wide (LDS, b = 10, 11, alphabets <= 1024, f < 2^11):
//             (slot - cum) | f << 11 | symbol << 22.
//   narrow    (LDS, b = 12, alphabets <= 256): u8 slot -> symbol maps, then per
//             symbol u32 f | (cum + coset*2^b) << 16 (bit 15: parity of z) and
//             the float value 2 z + c (4 m + c for m), at stride 256.
//   workspace (anything else): the narrow scheme with u16 slot maps and stride
//             2^b, read from the workspace through the caches.
//   hybrid    (b = 11, 12 with alphabets too large for the above): the
//             workspace format, with the u16 slot maps (64 / 128 KB) staged in
//             LDS and the per-symbol entries read through the caches.  At
//             b = 11, two per-slot arrays follow it (64 KB each) and, staged in
//             LDS together, replace both lookups when every frequency of the
//             tensor is below 128 (the build checks) and every value fits 16
//             bits (the host checks): u16 f | (slot - cum) << 7 | (parity of
//             z) << 15, and the i16 value 2 z + c (4 m + c for m) of the
//             slot's symbol.  (At b = 12 the two arrays would need 256 KB.)
enum TabLayout : int { kTabPacked = 0, kTabNarrow = 1, kTabWorkspace = 2, kTabPackedWide = 3, kTabHybrid = 4 };
enum Variant : uint32_t {
  kVarP9 = 0, kVarP10, kVarP11, kVarW10, kVarW11, kVarN12, kVarH11, kVarH12, kVarWs, kNumVariants
};

__host__ __device__ constexpr int layout_of(uint32_t v) {
  return v <= kVarP11 ? kTabPacked : v <= kVarW11 ? kTabPackedWide : v == kVarN12 ? kTabNarrow
       : v <= kVarH12 ? kTabHybrid : kTabWorkspace;
}
// format of the table block the build writes (the hybrid layout reuses the workspace format)
__host__ __device__ constexpr int storage_of(int tl) { return tl == kTabHybrid ? kTabWorkspace : tl; }
__host__ __device__ constexpr bool is_packed(int tl) { return tl == kTabPacked || tl == kTabPackedWide; }
__host__ __device__ constexpr uint32_t stride_of(int tl, uint32_t b) {
  return tl == kTabNarrow ? 256u : (tl == kTabWorkspace || tl == kTabHybrid) ? (1u << b) : 0u;
}
__host__ __device__ constexpr size_t lut_bytes_of(int tl, uint32_t b) {
  return (size_t(16) << b) * (is_packed(tl) ? 4 : tl == kTabNarrow ? 1 : 2);
}
__host__ __device__ constexpr size_t table_bytes_of(int tl, uint32_t b) {
  return lut_bytes_of(tl, b) + 2 * size_t(16) * stride_of(tl, b) * 4;
}
// hybrid layout at b = 11: byte offset of the per-slot entry maps after the
// workspace format; the per-slot values follow them
__host__ __device__ constexpr bool has_split(int tl, uint32_t b) { return tl == kTabHybrid && b == 11; }
__host__ __device__ constexpr size_t split_off_of(uint32_t b) { return table_bytes_of(kTabWorkspace, b); }
__host__ __device__ constexpr size_t split_bytes_of(uint32_t b) { return (size_t(16) << b) * 4; }
__host__ __device__ constexpr size_t storage_bytes_of(int tl, uint32_t b) {
  return table_bytes_of(tl, b) + (has_split(tl, b) ? split_bytes_of(b) : 0);
}
// bytes of a tensor's tables that the decode kernel stages in LDS
__host__ __device__ constexpr size_t lds_table_bytes_of(int tl, uint32_t b) {
  return tl == kTabWorkspace ? 0
       : tl == kTabHybrid ? (has_split(tl, b) ? split_bytes_of(b) : lut_bytes_of(tl, b))
       : table_bytes_of(tl, b);
}

// Device-side view of one tensor (lives in the workspace).
struct alignas(16) DevTensor {
  uint64_t nvec;             // rows * cols / 8
  uint32_t vpr;              // vectors per row = cols / 8
  uint32_t V, T, b;
  uint32_t rows;
  float scale;
  uint32_t empty_mask;       // bit k: table k is empty
  uint32_t variant;          // decode-table placement, see Variant
  uint32_t kpar;             // bit c: parity of the minima of fields z1..z7 in coset c
  uint32_t tab_bytes;        // bytes of the table block
  uint32_t payload_bytes;    // readable payload bytes: words rounded up to 8, times 2
  uint32_t out_bytes;        // output bytes (every tile's stores stay below this)
  uint32_t slow_rows;        // set by the table build when some row's g/2 is inexact: use g
  uint32_t f8z8;             // 1: field 8 holds z8 (no parity reduction), 0: it holds m
  uint32_t chunk0;           // index of the tensor's first chunk in the schedule
  uint32_t tpc;              // tiles per chunk of the tensor's launch group
  uint32_t direct;           // packed layouts: entries hold the value 2 z + c - 2 dmin (see kvals)
  uint32_t split;            // hybrid layout: 1 = per-slot entries usable (cleared by the build if some f > 127)
  int32_t dmin[9];           // direct entries: per field, the smaller of the two cosets' minima
  uint64_t payload_words;
  const float* row_scales;
  float* rowv;               // workspace: per row the pair (g/2, g), g = fp32(scale * row scale)
  const uint32_t* states;
  const uint32_t* offsets;
  const uint16_t* payload;
  const uint16_t* freqs;
  unsigned char* tab;        // workspace: decode tables in the variant's layout
  void* out;
  int32_t* status;
  // packed layouts, value constants as fp32 bit patterns, indexed by table t:
  // t < 14: 2^23 + 2^22 + [f = 2^11] - (2 min_t + c) (wide: 2^23 + 2^22 - min_t),
  // t = 14, 15: 2^23 + 2^22 - (4 min_t + c); t = 16, 17: parity of the minima
  // of z1..z7 in coset t - 16, at the symbol's bit position.  Direct entries:
  // t = 18 + (f - 1) for f = 1..7: -(2^23 + 2^22 - 2 dmin[f]); t = 25: the
  // negated field-8 constant; t = 26: the multiplier (+-2, or 0) of the parity
  // bit for field 8
  uint32_t kvals[32];
  int32_t minv[kTables];
  uint32_t freq_base[kTables];
  uint32_t alphabet[kTables];
};

struct Chunk {
  uint32_t tensor;
  uint32_t tile0;
};

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- table build
// One block per (coordinate table, tensor): cumulative frequencies by a block
// scan, then the slot -> symbol map by a binary search per slot.
__global__ __launch_bounds__(256) void build_tables_kernel(DevTensor* __restrict__ tens, Chunk* __restrict__ chunks,
                                                          uint32_t row_blocks) {
  DevTensor& T = tens[blockIdx.y];
  if (T.T == 0) return;
  if (blockIdx.x >= 16 + row_blocks) {
    // the tensor's entries of the tile schedule, 1024 per block
    const uint32_t nch = (T.T + T.tpc - 1) / T.tpc;
    const uint32_t j0 = (blockIdx.x - 16 - row_blocks) * 1024u;
    const uint32_t j1 = min(nch, j0 + 1024u);
    for (uint32_t j = j0 + threadIdx.x; j < j1; j += 256u) chunks[T.chunk0 + j] = Chunk{blockIdx.y, j * T.tpc};
    return;
  }
  if (blockIdx.x >= 16) {
    // per-row multipliers, 1024 rows per block: (2 z + c) * (g / 2) equals
    // (z + c/2) * g exactly whenever g / 2 is exact; the pair (g/2, g) is
    // stored and a tensor with any row where g / 2 is inexact uses g.
    const uint32_t r0 = (blockIdx.x - 16) * 1024u;
    bool inexact = false;
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t r = r0 + threadIdx.x + 256u * i;
      if (r < T.rows) {
        const float gr = __fmul_rn(T.scale, T.row_scales[r]);
        const float h = __fmul_rn(gr, 0.5f);
        inexact |= !(__fmul_rn(h, 2.0f) == gr);
        reinterpret_cast<float2*>(T.rowv)[r] = make_float2(h, gr);
      }
    }
    if (inexact) atomicOr(&T.slow_rows, 1u);
    return;
  }
  const uint32_t k = 1 + blockIdx.x;            // table index 1..16
  const uint32_t t = k - 1;                     // 2 * (field - 1) + coset
  const uint32_t c = t & 1u;
  const uint32_t field = 1 + (t >> 1);
  const uint32_t A = T.alphabet[k];
  const uint32_t b = T.b;
  const uint32_t M = 1u << b;
  const bool split = has_split(layout_of(T.variant), b);
  const int tl = storage_of(layout_of(T.variant));
  uint16_t* fd16 = reinterpret_cast<uint16_t*>(T.tab + split_off_of(b)) + (size_t(t) << b);
  int16_t* sval = reinterpret_cast<int16_t*>(T.tab + split_off_of(b)) + (size_t(16 + t) << b);
  const uint32_t S = stride_of(tl, b);
  unsigned char* lut8 = T.tab + (size_t(t) << b);
  uint16_t* lut16 = reinterpret_cast<uint16_t*>(T.tab) + (size_t(t) << b);
  uint32_t* lut32 = reinterpret_cast<uint32_t*>(T.tab) + (size_t(t) << b);
  const size_t lb = lut_bytes_of(tl, b);
  uint32_t* sym = reinterpret_cast<uint32_t*>(T.tab + lb) + size_t(t) * S;
  float* val = reinterpret_cast<float*>(T.tab + lb + size_t(16) * S * 4) + size_t(t) * S;
  __shared__ uint32_t scan[256];
  __shared__ uint32_t cums[1024];              // packed layouts: f | cum << 16 per symbol
  __shared__ uint32_t carry;
  if (!is_packed(tl)) {
    for (uint32_t i = A + threadIdx.x; i < S; i += blockDim.x) {
      sym[i] = 0;
      val[i] = 0.0f;
    }
  }
  if (A == 0) {   // empty table: never used, the decoder flags the tile
    for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) {
      if (is_packed(tl)) lut32[j] = 1u << 11;      // f = 1, slot - cum = 0, symbol 0
      else if (tl == kTabNarrow) lut8[j] = 0;
      else lut16[j] = 0;
      if (split) {
        fd16[j] = 1;                                // f = 1, slot - cum = 0
        sval[j] = 0;
      }
    }
    return;
  }
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const uint16_t* fr = T.freqs + T.freq_base[k];
  const int32_t mn = T.minv[k];
  for (uint32_t base = 0; base < A; base += blockDim.x) {
    const uint32_t i = base + threadIdx.x;
    const uint32_t f = i < A ? fr[i] : 0u;
    scan[threadIdx.x] = f;
    __syncthreads();
    for (uint32_t off = 1; off < blockDim.x; off <<= 1) {   // inclusive Hillis-Steele scan
      uint32_t v = threadIdx.x >= off ? scan[threadIdx.x - off] : 0u;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    const uint32_t cum = carry + scan[threadIdx.x] - f;
    if (i < A) {
      if (is_packed(tl)) {
        cums[i] = (f & 0xFFFFu) | (cum << 16);
      } else {
        // the narrow layout (b = 12, f <= 4096) keeps the parity of the value z in bit 15
        const uint32_t zpar = (tl == kTabNarrow && field < 8) ? (uint32_t(int32_t(i) + mn) & 1u) << 15 : 0u;
        sym[i] = (f & 0xFFFFu) | zpar | ((cum + (c << b)) << 16);
        const int32_t z = int32_t(i) + mn;
        val[i] = float(field < 8 || T.f8z8 ? 2 * z + int32_t(c) : 4 * z + int32_t(c));
      }
    }
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) carry += scan[threadIdx.x];
    __syncthreads();
  }
  // slot j -> largest i with cum_i <= j (a zero-frequency symbol is never chosen)
  int big = 0;
  for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) {
    uint32_t lo = 0, hi = A;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      const uint32_t cm = is_packed(tl) ? (cums[mid] >> 16) : (sym[mid] >> 16) - (c << b);
      if (cm <= j) lo = mid;
      else hi = mid;
    }
    if (is_packed(tl)) {
      const uint32_t e = cums[lo];
      // the entry's top bits: the symbol index, or (direct entries) the value
      // 2 z + c (4 m + c for field 8) relative to the field's smaller minimum
      uint32_t top = lo << (tl == kTabPacked ? 23 : 22);
      if (tl == kTabPacked && T.direct) {
        const int32_t d = int32_t(lo) + mn - T.dmin[field];
        top = uint32_t((field < 8 || T.f8z8 ? 2 * d : 4 * d) + int32_t(c)) << 22;
      }
      lut32[j] = (j - (e >> 16)) | ((e & 0xFFFFu) << 11) | top;
    } else if (tl == kTabNarrow) {
      lut8[j] = uint8_t(lo);
    } else {
      lut16[j] = uint16_t(lo);
      if (split) {
        const uint32_t e = sym[lo];
        const uint32_t f = e & 0xFFFFu, d = j - ((e >> 16) - (c << b));
        const uint32_t zp = field < 8 ? (uint32_t(int32_t(lo) + mn) & 1u) : 0u;
        big |= f > 127u;
        fd16[j] = uint16_t((f & 0x7Fu) | (d << 7) | (zp << 15));
        sval[j] = int16_t(val[lo]);                  // |value| < 2^15: checked on the host
      }
    }
  }
  // per-slot entries hold f in 7 bits: any larger frequency disables them for the tensor
  if (__syncthreads_or(big) && threadIdx.x == 0) atomicAnd(&T.split, 0u);
}

// ---------------------------------------------------------------- container rounding
// OCP e4m3fn codes of four values, bytes in order: clamp to +-448 (v_med3_f32),
// then gfx950's conversion to OCP FP8 (round to nearest even, subnormals and
// signed zeros kept), two values per instruction.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const float lo = -448.0f, hi = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi), __builtin_amdgcn_fmed3f(b, lo, hi),
                                          0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi), __builtin_amdgcn_fmed3f(d, lo, hi), w,
                                      true);
  return uint32_t(w);
}

// INT8 (or, with kUnsigned, UINT8 = INT8 + 128) codes of four values, bytes in
// order.  Clamping to [-128, 127] first is the same as rounding first (the
// bounds are integers); adding 2^23 + 2^22 (+ 128) then rounds to nearest
// even and leaves the two's-complement code (or the offset code) in the low
// byte of the sum's bit pattern, and byte permutes gather the four low bytes.
template <bool kUnsigned>
__device__ __forceinline__ uint32_t int8_codes4(float a, float b, float c, float d) {
  constexpr float kMagic = kUnsigned ? 12583040.0f : 12582912.0f;
  const uint32_t ta = __float_as_uint(__builtin_amdgcn_fmed3f(a, -128.0f, 127.0f) + kMagic);
  const uint32_t tb = __float_as_uint(__builtin_amdgcn_fmed3f(b, -128.0f, 127.0f) + kMagic);
  const uint32_t tc = __float_as_uint(__builtin_amdgcn_fmed3f(c, -128.0f, 127.0f) + kMagic);
  const uint32_t td = __float_as_uint(__builtin_amdgcn_fmed3f(d, -128.0f, 127.0f) + kMagic);
  const uint32_t lo = __builtin_amdgcn_perm(tb, ta, 0x0C0C0400u);   // a.b0, b.b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(td, tc, 0x0C0C0400u);   // c.b0, d.b0, 0, 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));      // RNE, overflow to inf
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));   // v_cvt_pk_bf16_f32 (RNE)
}

// ---------------------------------------------------------------- decode
// Per-tile payload staging: each half-wave streams its tile's words through an
// LDS ring of kRingWords, filled kChunkWords at a time (one 8-byte load per
// lane).  Every vector round issues exactly three memory operations -- the
// row-scale load, the next ring chunk and the output store -- all as raw
// buffer operations, whose out-of-range lanes the hardware turns into zero
// loads and dropped stores.  With a fixed count per round the waits stay
// precise: waiting for this round's row scale never waits for the chunk in
// flight behind it.
constexpr uint32_t kRingWords = 512;
constexpr uint32_t kChunkWords = 128;
constexpr uint32_t kRoundWords = 9 * 32;                 // most words one vector round can read
constexpr uint32_t kRingSlack = kRingWords - kChunkWords; // a chunk fits while fill <= read + slack
constexpr size_t kRingBytes = size_t(kTilesPerChunk) * kRingWords * sizeof(uint16_t);

enum OutKind : int {
  kOutBF16 = 0, kOutFP8 = 1, kOutINT8 = 2, kOutLattice = 3, kOutFP16 = 4, kOutFP32 = 5, kOutUINT8 = 6,
  kNumOutKinds = 7
};

__host__ __device__ constexpr uint32_t out_vec_bytes(int ok) {
  return ok == kOutBF16 || ok == kOutFP16 ? 16u : ok == kOutLattice || ok == kOutFP32 ? 32u : 8u;
}

// lane mask with the lanes of half-wave 0 if h0 and those of half-wave 1 if h1
__device__ __forceinline__ uint64_t half_mask(bool h0, bool h1) {
  return (h0 ? 0x00000000FFFFFFFFull : 0ull) | (h1 ? 0xFFFFFFFF00000000ull : 0ull);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(bytes), 0x00020000);
}

// Decode the two tiles of one wave (tile0 + 2*wave + half, if that slot is below
// the chunk's tile count).  BT is the
// probability precision when known at compile time (0: read T.b), TL the
// table layout (LDS tables start at LDS address 0), OK the output kind, SP
// (hybrid layout) whether the per-slot entry maps are the ones staged in LDS.
template <int BT, int TL, int OK, bool SP>
__device__ __forceinline__ void decode_pair(const DevTensor& T, uint32_t tile0, uint32_t tile_end,
                                            const unsigned char* __restrict__ lds,
                                            uint16_t* __restrict__ ring) {
  constexpr bool kWs = TL == kTabWorkspace;
  constexpr bool kHyb = TL == kTabHybrid;
  constexpr bool kGlobalEntries = kWs || kHyb;             // per-symbol entries read from the workspace
  const uint32_t B = BT ? uint32_t(BT) : T.b;
  const uint32_t M = 1u << B;
  const uint32_t MASK = M - 1u;
  const uint32_t S = kGlobalEntries ? M : 256u;             // sym / val stride (narrow, workspace, hybrid)
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t half = lane >> 5;
  const uint32_t hs = half << 4;                            // selects this half's packed 16 bits
  const uint32_t l = lane & 31u;
  const uint32_t t = tile0 + half;                          // tile of this half-wave
  const bool tile_ok = t < tile_end;                        // tile_end <= T.T

  // ---- per-lane tile start
  uint32_t n = 0, x = kL, p = 0, pend = 0;
  bool bad_len = false;
  if (tile_ok) {
    const uint64_t first = uint64_t(t) * T.V;
    n = uint32_t(min(uint64_t(T.V), T.nvec - first));
    x = ((const EP_GLOBAL uint32_t*)T.states)[size_t(t) * EP_LANES + l];
    p = ((const EP_GLOBAL uint32_t*)T.offsets)[t];
    pend = ((const EP_GLOBAL uint32_t*)T.offsets)[t + 1];
    if (pend < p || pend > T.payload_words) {
      bad_len = true;
      n = 0;
      pend = p;
    }
  }
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(T.payload, T.payload_bytes);
  // descriptor fields used inside the round loop, read once: the output
  // stores could alias the descriptor as far as the compiler knows
  const uint32_t vpr = T.vpr;
  const uint32_t out_bytes = T.out_bytes;
  const __amdgpu_buffer_rsrc_t rO = make_rsrc(T.out, out_bytes);
  const __amdgpu_buffer_rsrc_t rR = make_rsrc(T.rowv, T.rows * 8u);

  // ---- per-half-wave uniform state (scalar registers)
  const uint32_t n0 = __builtin_amdgcn_readlane(n, 0), n1 = __builtin_amdgcn_readlane(n, 32);
  const uint32_t st0 = __builtin_amdgcn_readlane(p, 0), st1 = __builtin_amdgcn_readlane(p, 32);
  const uint32_t a00 = st0 & ~3u, a01 = st1 & ~3u;          // 8-byte aligned first word
  const uint32_t end0 = __builtin_amdgcn_readlane(pend, 0) - a00;
  const uint32_t end1 = __builtin_amdgcn_readlane(pend, 32) - a01;
  uint32_t P0 = st0 - a00, P1 = st1 - a01;                  // ring-relative read pointers
  // the read pointer of this lane's half, kept per lane so that the
  // renormalisation needs no scalar bookkeeping; P0 / P1 are refreshed from it
  // once per round for the ring fill
  uint32_t vP = half ? P1 : P0;
  const uint32_t hs32 = half << 5;                          // selects this half's 32 ballot bits
  uint32_t F0 = 0, F1 = 0;                                  // words written to the ring
  uint64_t empty_err = 0;
  const uint32_t lane4 = 4u * l;                            // this lane's words inside a chunk
  const uint32_t chunk_lane = 2u * ((half ? a01 : a00) + lane4);   // byte offset of this lane's part
  const uint32_t kmax = max((n0 + 31u) >> 5, (n1 + 31u) >> 5);

  const uint32_t f0 = ((const EP_GLOBAL uint16_t*)T.freqs)[T.freq_base[0]];   // coset bit: frequency of c = 0
  uint32_t f0v = f0, f1v = M - f0;                          // per-lane copies for the selects
  asm volatile("" : "+v"(f0v), "+v"(f1v));
  const uint32_t kpar = T.kpar;
  // field 8: m (value 4 s + 2 parity + const) or z8 itself (2 s + const, no parity)
  const uint32_t pw = T.f8z8 ? 0u : 1u;                     // width of the parity bit field
  const uint32_t sh8 = T.f8z8 ? 1u : 2u;
  const uint32_t empty = T.empty_mask;
  const bool slow_rows = T.slow_rows != 0;
  const unsigned char* tbase = kGlobalEntries ? T.tab : lds;
  const uint32_t lut_bytes = uint32_t(lut_bytes_of(TL, B));
  // packed tables: fields 5..8 of b = 11 lie beyond the 16-bit LDS offset of
  // the lookup instruction, so they get a second coset base
  constexpr bool kSplit = is_packed(TL) && (size_t(14) << BT) * 4u > 65535u;
  constexpr bool kWide = TL == kTabPackedWide;
  constexpr uint32_t kSymShift = kWide ? 22 : 23;         // symbol index position in packed entries
  // packed tables: lane i < 18 holds value constant i (see DevTensor::kvals);
  // a lane fetches the one for its coset with ds_bpermute
  const uint32_t kreg = is_packed(TL) ? ((const EP_GLOBAL uint32_t*)T.kvals)[l] : 0u;
  // direct entries (packed layout): uniform value constants (stored negated:
  // the adds cannot be merged with the symbol form's subtractions, which keeps
  // the constants in scalar registers), no per-lane fetch
  constexpr bool kDirectable = TL == kTabPacked;
  const bool direct = kDirectable && T.direct != 0;
  const uint32_t fw = kWide || direct ? 11u : 12u;           // width of f in the entry
  float kd[7] = {0, 0, 0, 0, 0, 0, 0}, k8d = 0.0f;
  int32_t m8d = 0;
  if (kDirectable) {
#pragma unroll
    for (int f = 0; f < 7; ++f) kd[f] = __builtin_bit_cast(float, T.kvals[18 + f]);
    k8d = __builtin_bit_cast(float, T.kvals[25]);
    m8d = int32_t(T.kvals[26]);
  }

  // the chunk held in registers is always the one starting at word F of the half
  u32x2 pf = __builtin_amdgcn_raw_buffer_load_b64(rP, chunk_lane, 0, 0);
  // A store past the end of the output (dropped by the hardware): it makes the
  // first round see the same queue of outstanding memory operations as every
  // later round (chunk, then store), so the compiler's waits stay exact.
  __builtin_amdgcn_raw_buffer_store_b32(0u, rO, out_bytes, 0, 0);

  uint32_t g = t * T.V + l;                                 // < 2^32: checked on the host
  // rowb: byte offset of the row multiplier, g/2 or (slow rows) g of the row's pair
  uint32_t rowb = slow_rows ? 4u : 0u, col = 0;
  if (tile_ok) {
    const uint32_t row = g / vpr;
    col = g - row * vpr;
    rowb += 8u * row;
  }

  // One vector round.  In full rounds every lane of both halves has a vector,
  // so the active-lane masks fold away.
  auto round = [&](const uint32_t k, auto full) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full)::value;
    const bool active = kFull || (k * 32u + l) < n;
    const uint32_t x_saved = x;
    // Issued before the ring prefetch below: loads retire in order, so waiting
    // for this one later does not also wait for the prefetch.
    const float rv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, rowb, 0, 0));

    P0 = __builtin_amdgcn_readlane(vP, 0);
    P1 = __builtin_amdgcn_readlane(vP, 32);
    // ---- ring: store the held chunk if it is useful and fits ...
    {
      const bool w0 = F0 < end0 && F0 <= P0 + kRingSlack;
      const bool w1 = F1 < end1 && F1 <= P1 + kRingSlack;
      // both halves' predicates as one lane mask (the branch takes it as exec);
      // the fill pointers packed in one scalar, a lane extracts its half's 16
      // bits (tile payloads stay below 2^16 words)
      if (__builtin_amdgcn_inverse_ballot_w64(half_mask(w0, w1))) {
        const uint32_t F = __builtin_amdgcn_ubfe(F0 | (F1 << 16), hs, 16);
        *reinterpret_cast<u32x2*>(ring + ((F & (kRingWords - 1u)) | lane4)) = pf;
      }
      F0 += w0 ? kChunkWords : 0u;
      F1 += w1 ? kChunkWords : 0u;
    }
    // ... catch up synchronously if this round could read past the staged words
    // (tile starts, and long runs above kChunkWords words per round) ...
    for (;;) {
      const bool c0 = F0 < min(P0 + kRoundWords, end0);
      const bool c1 = F1 < min(P1 + kRoundWords, end1);
      if (!(c0 || c1)) break;
      if (__builtin_amdgcn_inverse_ballot_w64(half_mask(c0, c1))) {
        const uint32_t F = __builtin_amdgcn_ubfe(F0 | (F1 << 16), hs, 16);
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rP, chunk_lane + 2u * F, 0, 0);
        *reinterpret_cast<u32x2*>(ring + ((F & (kRingWords - 1u)) | lane4)) = v;
      }
      F0 += c0 ? kChunkWords : 0u;
      F1 += c1 ? kChunkWords : 0u;
    }
    // ... and fetch the chunk at the new fill position for a later round.
    pf = __builtin_amdgcn_raw_buffer_load_b64(rP, chunk_lane + 2u * __builtin_amdgcn_ubfe(F0 | (F1 << 16), hs, 16),
                                              0, 0);

// Renormalisation: the lanes of a half whose state fell below 2^15 read the
// next words of their tile in lane order.  A lane's word is its half's pointer
// plus the number of reading lanes below it in the half (popcount of the
// half's ballot bits under the lane).  Every lane reads (the index stays
// inside the ring) and keeps the word only if it needed one: no exec masking
// and no scalar pointer updates on the serial path.
#define EP_RENORM()                                                                   \
  {                                                                                   \
    const bool rn = (x < kL) & active;                                                \
    const uint32_t hm = uint32_t(__builtin_amdgcn_ballot_w64(rn) >> hs32);            \
    const uint32_t idx = __builtin_popcount(__builtin_amdgcn_ubfe(hm, 0, l)) + vP;    \
    uint32_t w = ring[idx & (kRingWords - 1u)];                                       \
    asm volatile("" : "+v"(w)); /* keep the read unconditional */                    \
    x = rn ? ((x << 16) | w) : x;                                                     \
    vP += __builtin_popcount(hm);                                                     \
  }

    // ---- field 0: coset bit (two-symbol table, resolved by one compare)
    uint32_t q = x >> B;
    uint32_t slot = x & MASK;
    const bool c = slot >= f0v;
    x = __umul24(c ? f1v : f0v, q) + slot - (c ? f0v : 0u);
    EP_RENORM();
    if (empty & 6u) empty_err |= __builtin_amdgcn_ballot_w64(active && ((empty >> (c ? 2 : 1)) & 1u));

    // ---- fields z1..z7, m; vv[f] becomes 2 z_f + c (exact in fp32)
    float vv[9];
    uint32_t par;
    if (is_packed(TL)) {
      uint32_t ev[9];
      uint32_t lbl = c ? (M << 2) : 0u;                  // byte offset of the coset's table
      uint32_t lbh = lbl + (kSplit ? (8u << B) * 4u : 0u);
      // opaque to the optimiser, so that the lookup address stays one
      // v_and_or_b32 with the table offset folded into the LDS instruction
      asm volatile("" : "+v"(lbl), "+v"(lbh));
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        const bool hi = kSplit && f >= 5;
        const uint32_t toff = (uint32_t(2 * (f - 1) - (hi ? 8 : 0)) << B) * 4u;
        const uint32_t e = *reinterpret_cast<const uint32_t*>(lds + (((x << 2) & (MASK << 2)) | (hi ? lbh : lbl)) + toff);
        q = x >> B;
        x = __umul24(__builtin_amdgcn_ubfe(e, 11, fw), q) + (e & 0x7FFu);
        ev[f] = e;
        EP_RENORM();
      }
      if (kDirectable && direct) {
        // direct entries: 0x4B400000 | (e >> 22) is the float 2^23 + 2^22 +
        // (2 z + c - 2 dmin), and one constant per field (the same for both
        // cosets) turns it into 2 z + c.  Bit 23 of an entry is the parity of
        // z - dmin, so the XOR of z1..z7's entries gives the parity of their
        // sum up to the parity of the minima, which the field-8 constant and
        // multiplier absorb: 2 z8 + c = (4 (m - dmin8) + c) + 2 par + 4 dmin8.
#pragma unroll
        for (int f = 1; f <= 7; ++f)
          vv[f] = __builtin_bit_cast(float, __builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[f], 22)) + kd[f - 1];
        const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
            __builtin_amdgcn_bitop3_b32(ev[1], ev[2], ev[3], 0x96),
            __builtin_amdgcn_bitop3_b32(ev[4], ev[5], ev[6], 0x96), ev[7], 0x96);
        par = __builtin_amdgcn_ubfe(x3, 23, pw);
        const int32_t u8 = __mul24(int32_t(par), m8d) + int32_t(__builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[8], 22));
        vv[8] = __builtin_bit_cast(float, u8) + k8d;
      } else {
      // value of z_f.  Packed: 0x4B400000 | (e >> 22) is the float
      // 2^23 + 2^22 + 2 s (+1 when f = 2^11), and the per-table constant turns
      // it into 2 z + c.  Wide: the same bits give 2^23 + 2^22 + s, the
      // constant turns it into z, and an exact fma makes 2 z + c.
      const int kaddr = c ? 4 : 0;
      const float cf = c ? 1.0f : 0.0f;
#pragma unroll
      for (int f = 1; f <= 7; ++f) {
        const float u = __builtin_bit_cast(float, __builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[f], 22));
        const float kf = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(kaddr + 8 * (f - 1), int(kreg)));
        vv[f] = kWide ? __builtin_fmaf(u - kf, 2.0f, cf) : u - kf;
      }
      // parity of z1 + ... + z7: bit kSymShift of each entry is the parity of
      // its symbol index, the constant supplies the parity of the minima
      const uint32_t kp = uint32_t(__builtin_amdgcn_ds_bpermute(kaddr + 64, int(kreg)));
      const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
          __builtin_amdgcn_bitop3_b32(ev[1], ev[2], ev[3], 0x96),
          __builtin_amdgcn_bitop3_b32(ev[4], ev[5], ev[6], 0x96),
          ev[7] ^ kp, 0x96);
      par = __builtin_amdgcn_ubfe(x3, kSymShift, pw);
      // z8 = 2 m + parity: 2 z8 + c = 4 s8 + 2 par + (c + 4 min), the
      // parenthesis being part of the per-table constant (a directly coded
      // z8: 2 s8 + (c + 2 min), with the parity field of width 0)
      const uint32_t u8 = ((ev[8] >> kSymShift) << sh8) + ((par << 1) | 0x4B400000u);
      const float k8 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(kaddr + 56, int(kreg)));
      vv[8] = __builtin_bit_cast(float, u8) - k8;
      }
    } else if constexpr (SP) {
      // per-slot entries f | (slot - cum) << 7 | parity << 15 and the slot
      // symbol's value 2 z + c (i16), both in LDS (b = 11: 64 KB each)
      static_assert(BT == 11, "per-slot entries are built for b = 11");
      uint32_t ev[9];
      uint32_t lbl = c ? (M << 1) : 0u;                  // byte offset of the coset's map
      asm volatile("" : "+v"(lbl));
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        const uint32_t toff = (uint32_t(2 * (f - 1)) << B) * 2u;       // at most 57344
        const uint32_t a = ((x << 1) & (MASK << 1)) | lbl;
        const uint32_t e = *reinterpret_cast<const uint16_t*>(lds + a + toff);
        // the values follow the 16 entry maps (64 KB): a second base register
        const uint32_t av = a | (uint32_t(16) << (B + 1));
        vv[f] = float(*reinterpret_cast<const int16_t*>(lds + av + toff));
        q = x >> B;
        x = __umul24(e & 0x7Fu, q) + __builtin_amdgcn_ubfe(e, 7, 7);
        ev[f] = e;
        EP_RENORM();
      }
      const uint32_t x3 = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_bitop3_b32(ev[1], ev[2], ev[3], 0x96),
                                                      __builtin_amdgcn_bitop3_b32(ev[4], ev[5], ev[6], 0x96),
                                                      ev[7], 0x96);
      par = __builtin_amdgcn_ubfe(x3, 15, pw);
      vv[8] = vv[8] + float(par << 1);                   // the m values are 4 m + c (z8: 2 z8 + c)
    } else {
      uint32_t sv[9];
      const uint32_t lb = c ? M : 0u;                    // coset offset inside each table pair
      // symbol tables: coset base including the block's own offset, so that
      // the per-field LDS offsets fit the 16-bit immediate
      uint32_t cb = c ? lut_bytes + S * 4u : lut_bytes;
      if (TL == kTabNarrow) asm volatile("" : "+v"(cb));
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        const uint32_t addr = (x & MASK) | lb;           // slot + coset * 2^b
        uint32_t s;
        if (kWs) s = reinterpret_cast<const uint16_t*>(tbase)[(uint32_t(2 * (f - 1)) << B) + addr];
        else if (kHyb) s = reinterpret_cast<const uint16_t*>(lds)[(uint32_t(2 * (f - 1)) << B) + addr];
        else s = lds[(uint32_t(2 * (f - 1)) << B) + addr];
        const uint32_t eo = cb + s * 4u + uint32_t(f - 1) * 2u * S * 4u;
        const uint32_t e = *reinterpret_cast<const uint32_t*>(tbase + eo);
        vv[f] = *reinterpret_cast<const float*>(tbase + eo + 16u * S * 4u);
        q = x >> B;
        x = __umul24(e & (kGlobalEntries ? 0xFFFFu : 0x7FFFu), q) + (addr - (e >> 16));
        sv[f] = kGlobalEntries ? s : e;
        EP_RENORM();
      }
      const uint32_t x3 = __builtin_amdgcn_bitop3_b32(__builtin_amdgcn_bitop3_b32(sv[1], sv[2], sv[3], 0x96),
                                                      __builtin_amdgcn_bitop3_b32(sv[4], sv[5], sv[6], 0x96),
                                                      sv[7], 0x96);
      // narrow: bit 15 of the symbol entries is the parity of z; workspace:
      // parity of the symbol indices, corrected by the parity of the minima
      par = TL == kTabNarrow ? __builtin_amdgcn_ubfe(x3, 15, pw) : (x3 ^ (kpar >> (c ? 1 : 0))) & pw;
      vv[8] = vv[8] + float(par << 1);                   // the m table holds 4 m + c (z8: 2 z8 + c)
    }
#undef EP_RENORM
    x = active ? x : x_saved;

    // ---- y = (z + c/2) * g, computed as (2 z + c) * (g/2) when g/2 is exact
    // (the row multiplier array then holds g/2; otherwise g and the slow form)
    const uint32_t ob = active ? (g + k * 32u) * out_vec_bytes(OK) : out_bytes;
    if (OK == kOutLattice) {
      const i32x4 lo4 = {int(vv[1]), int(vv[2]), int(vv[3]), int(vv[4])};
      const i32x4 hi4 = {int(vv[5]), int(vv[6]), int(vv[7]), int(vv[8])};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo4), rO, ob, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi4), rO, ob + 16u, 0, 0);
    } else {
      // slow rows: rv is g and 2 z + c is halved first (exactly)
      if (slow_rows) {
#pragma unroll
        for (int i = 1; i <= 8; ++i) vv[i] = __fmul_rn(vv[i], 0.5f);
      }
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = __fmul_rn(vv[i + 1], rv);
      if (OK == kOutBF16) {
        const u32x4 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                         pack_bf16x2(y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w, rO, ob, 0, 0);
      } else if (OK == kOutFP16) {
        const u32x4 w = {pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]), pack_f16x2(y[4], y[5]),
                         pack_f16x2(y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w, rO, ob, 0, 0);
      } else if (OK == kOutFP32) {
        const u32x4 lo = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
        const u32x4 hi = {__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]), __float_as_uint(y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(lo, rO, ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(hi, rO, ob + 16u, 0, 0);
      } else if (OK == kOutFP8) {
        const u32x2 w = {pack_fp8x4(y[0], y[1], y[2], y[3]), pack_fp8x4(y[4], y[5], y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b64(w, rO, ob, 0, 0);
      } else {
        // INT8 codes; UINT8 adds the offset 128
        const u32x2 w = {int8_codes4<OK == kOutUINT8>(y[0], y[1], y[2], y[3]),
                         int8_codes4<OK == kOutUINT8>(y[4], y[5], y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b64(w, rO, ob, 0, 0);
      }
    }
    col += 32u;
    if (col >= vpr) {                       // rows of at least 32 vectors wrap at most once
      col -= vpr;
      rowb += 8u;
      while (col >= vpr) {
        col -= vpr;
        rowb += 8u;
      }
    }
  };
  const uint32_t kfull = min(n0, n1) >> 5;
  uint32_t k = 0;
  for (; k < kfull; ++k) round(k, std::true_type{});
  for (; k < kmax; ++k) round(k, std::false_type{});

  // ---- end-of-tile invariants: every state back at 2^15, every word consumed
  const uint64_t bad_state = __builtin_amdgcn_ballot_w64(x != kL);
  const uint64_t bad_len_m = __builtin_amdgcn_ballot_w64(bad_len);
  if (tile_ok && l == 0 && T.status) {
    const uint32_t Pm = vP, Em = half ? end1 : end0;
    const uint32_t sh = half ? 32u : 0u;
    int st = EP_TILE_OK;
    if (uint32_t(bad_len_m >> sh)) st = EP_TILE_BAD_LENGTH;
    else if (Pm > Em) st = EP_TILE_OVERRUN;
    else if (uint32_t(empty_err >> sh)) st = EP_TILE_EMPTY_TABLE;
    else if (uint32_t(bad_state >> sh)) st = EP_TILE_BAD_STATE;
    else if (Pm != Em) st = EP_TILE_BAD_LENGTH;
    ((EP_GLOBAL int32_t*)T.status)[t] = st;
  }
}

// Persistent decode kernel.  Block i owns a contiguous range of chunks (up to
// tiles_per_chunk tiles of one tensor each), which splits into runs of chunks
// from the same tensor.  For each run the block stages the tensor's decode
// tables (LDS layouts); then each wave takes pairs of consecutive tiles (one
// per half-wave) from a counter until the run is exhausted.  Taking work
// dynamically keeps all of a block's waves busy to the end: the SIMD's issue
// arbitration favours older waves, so equal static shares finish at very
// different times.  The counter of a run is the word of `ctr` at the run's
// first chunk (LDS is fully used by the tables and rings); a wave claims its
// next pair before decoding the current one, so the atomic's latency is hidden.
template <int BT, int TL, int OK>
__global__ __launch_bounds__(kBlock) void decode_kernel(const DevTensor* __restrict__ tens,
                                                        const Chunk* __restrict__ chunks,
                                                        uint32_t* __restrict__ ctr,
                                                        uint32_t nchunks, uint32_t tiles_per_chunk) {
  constexpr size_t kTab = lds_table_bytes_of(TL, BT);
  __shared__ __align__(16) unsigned char smem[kTab + kRingBytes];
  const uint32_t per = (nchunks + gridDim.x - 1) / gridDim.x;
  const uint32_t c0 = blockIdx.x * per;
  const uint32_t c1 = min(nchunks, c0 + per);
  const bool lane0 = (threadIdx.x & 63u) == 0;
  // LDS: [decode tables (LDS layouts)][32 rings of kRingWords]
  uint16_t* ring = reinterpret_cast<uint16_t*>(smem + kTab) + (threadIdx.x >> 5) * kRingWords;
  for (uint32_t ci = c0; ci < c1;) {
    const Chunk ch = chunks[ci];
    const DevTensor& T = tens[ch.tensor];
    // a tensor's chunks are consecutive: the run ends with the tensor or the range
    const uint32_t left = (T.T - ch.tile0 + tiles_per_chunk - 1) / tiles_per_chunk;
    const uint32_t cn = min(c1, ci + left);
    const uint32_t t_end = min(T.T, ch.tile0 + (cn - ci) * tiles_per_chunk);
    const uint32_t npairs = (t_end - ch.tile0 + 1) / 2;
    __syncthreads();                       // every wave is done with the previous run
    if (threadIdx.x == 0) __hip_atomic_store(ctr + ci, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // hybrid layout: the per-slot entry maps when the build kept them, else the slot maps
    const bool split = has_split(TL, BT) && T.split != 0;
    if (TL != kTabWorkspace) {
      const EP_GLOBAL u32x4* src = (const EP_GLOBAL u32x4*)(T.tab + (split ? split_off_of(BT) : 0));
      u32x4* dst = reinterpret_cast<u32x4*>(smem);
      const uint32_t n16 = uint32_t((has_split(TL, BT) && !split ? lut_bytes_of(TL, BT) : kTab) / 16u);
      for (uint32_t i = threadIdx.x; i < n16; i += kBlock) dst[i] = src[i];
    }
    __syncthreads();
    // the first pair of each wave is its own index, which spreads a short run
    // over the SIMDs (wave w runs on SIMD w mod 4); later pairs come from the counter
    uint32_t pr = threadIdx.x >> 6, nx = 0;
    while (pr < npairs) {
      if (lane0) nx = kWavesPerBlock + atomicAdd(ctr + ci, 1u);
      if constexpr (has_split(TL, BT)) {
        if (split) decode_pair<BT, TL, OK, true>(T, ch.tile0 + 2u * pr, t_end, smem, ring);
        else decode_pair<BT, TL, OK, false>(T, ch.tile0 + 2u * pr, t_end, smem, ring);
      } else {
        decode_pair<BT, TL, OK, false>(T, ch.tile0 + 2u * pr, t_end, smem, ring);
      }
      pr = __builtin_amdgcn_readfirstlane(nx);
    }
    ci = cn;
  }
}

// Container rounding of n4 groups of four fp32 values with the decode
// kernel's own conversions (ep_convert_f32).
template <int OK>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in, void* __restrict__ out,
                                                     uint64_t n4) {
  for (uint64_t q = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < n4;
       q += uint64_t(gridDim.x) * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(in)[q];
    if (OK == kOutBF16) {
      reinterpret_cast<u32x2*>(out)[q] = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
    } else if (OK == kOutFP16) {
      reinterpret_cast<u32x2*>(out)[q] = u32x2{pack_f16x2(v.x, v.y), pack_f16x2(v.z, v.w)};
    } else if (OK == kOutFP8) {
      reinterpret_cast<uint32_t*>(out)[q] = pack_fp8x4(v.x, v.y, v.z, v.w);
    } else {
      reinterpret_cast<uint32_t*>(out)[q] = int8_codes4<OK == kOutUINT8>(v.x, v.y, v.z, v.w);
    }
  }
}

// ---------------------------------------------------------------- host side
uint32_t choose_variant(const ep_tensor_desc& d) {
  uint32_t amax = 0;
  for (int k = 1; k < kTables; ++k) amax = std::max(amax, d.alphabet[k]);
  bool single = false;                                 // a one-symbol table (f = 2^b)
  for (int k = 1; k < kTables; ++k) single |= d.alphabet[k] == 1;
  if (d.prob_bits <= 11 && amax <= 512 && table_bytes_of(kTabPacked, d.prob_bits) + kRingBytes <= kMaxLds)
    return kVarP9 + (d.prob_bits - 9);
  // the wide entry holds f in 11 bits: every f < 2^11 (no one-symbol table at b = 11)
  if ((d.prob_bits == 10 || d.prob_bits == 11) && amax <= 1024 && !(d.prob_bits == 11 && single) &&
      table_bytes_of(kTabPackedWide, d.prob_bits) + kRingBytes <= kMaxLds)
    return kVarW10 + (d.prob_bits - 10);
  if (d.prob_bits == 12 && amax <= 256 && table_bytes_of(kTabNarrow, 12) + kRingBytes <= kMaxLds)
    return kVarN12;
  if ((d.prob_bits == 11 || d.prob_bits == 12) && lds_table_bytes_of(kTabHybrid, d.prob_bits) + kRingBytes <= kMaxLds)
    return kVarH11 + (d.prob_bits - 11);
  return kVarWs;
}

constexpr uint32_t kNumGroups = kNumVariants * kNumOutKinds;   // one launch per non-empty group

int out_kind_of(int dtype) {
  switch (dtype) {
    case EP_OUT_BF16: return kOutBF16;
    case EP_OUT_FP8_E4M3: return kOutFP8;
    case EP_OUT_INT8: return kOutINT8;
    case EP_OUT_LATTICE2X_I32: return kOutLattice;
    case EP_OUT_FP16: return kOutFP16;
    case EP_OUT_FP32: return kOutFP32;
    case EP_OUT_UINT8: return kOutUINT8;
    default: return -1;
  }
}

struct Layout {
  size_t tens_off, chunk_off, ctr_off, total;
  std::vector<size_t> tab_off, tab_bytes, row_off;
  std::vector<uint32_t> variant, group;
  size_t max_chunks;                  // chunk slots for the smallest chunk (2 tiles)
  size_t group_tiles[kNumGroups];
};

int validate(const ep_tensor_desc& d, int i) {
  auto bad = [&](const char* what) {
    return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": " + what);
  };
  if (d.rows < 0) return bad("rows < 0");
  if (d.cols <= 0 || d.cols % 8 != 0) return bad("cols must be a positive multiple of 8");
  if (d.vectors_per_tile < 32) return bad("vectors_per_tile < 32");
  // a tile's payload (at most 9 words per vector) is addressed with 16-bit offsets
  if (d.vectors_per_tile > 7200) return bad("vectors_per_tile > 7200");
  if (d.prob_bits < 9 || d.prob_bits > 15) return bad("prob_bits outside [9, 15]");
  const unsigned __int128 nvec = (unsigned __int128)(uint64_t)d.rows * (uint64_t)d.cols / 8u;
  if (nvec >= ((unsigned __int128)1 << 32)) return bad("rows*cols/8 must be < 2^32");
  const uint64_t nv = uint64_t(nvec);
  const uint64_t T = (nv + d.vectors_per_tile - 1) / d.vectors_per_tile;
  if (T != d.num_tiles) return bad("num_tiles != ceil(rows*cols/8 / vectors_per_tile)");
  if (d.alphabet[0] != 2 || d.min_offset[0] != 0) return bad("table 0 must be the coset bit (alphabet 2, min 0)");
  if (d.field8 != EP_FIELD8_M && d.field8 != EP_FIELD8_Z8) return bad("field8 must be EP_FIELD8_M or EP_FIELD8_Z8");
  for (int k = 1; k < kTables; ++k) {
    if (d.alphabet[k] > (1u << d.prob_bits)) return bad("alphabet exceeds 2^prob_bits");
    // |4 z + c| < 2^22 keeps every reconstructed value exact in fp32
    const int64_t lo = d.min_offset[k], hi = lo + int64_t(d.alphabet[k]);
    if (lo < -(int64_t(1) << 19) || hi > (int64_t(1) << 19)) return bad("lattice coordinates beyond +-2^19");
  }
  if (2 * ((d.payload_words + 7) / 8 * 8) >= (uint64_t(1) << 32)) return bad("payload must be < 4 GiB");
  // 32-bit output offsets: every vector a tile's lanes can address stays below 2^32 bytes
  if ((nv + 64ull * d.vectors_per_tile + 64) * 32ull >= (uint64_t(1) << 32))
    return bad("tensor too large for one descriptor (split it)");
  if (d.num_tiles > 0) {
    if (!d.row_scales || !d.tile_states || !d.tile_offsets || !d.payload || !d.freqs)
      return bad("NULL device pointer");
    if (reinterpret_cast<uintptr_t>(d.payload) % 16 != 0) return bad("payload must be 16-byte aligned");
  }
  return EP_OK;
}

int make_layout(const ep_tensor_desc* descs, const int* dtypes, int n, Layout& L) {
  if (n < 0 || (n > 0 && !descs)) return fail(EP_ERR_INVALID_ARG, "bad tensor count or NULL descriptors");
  size_t off = 0;
  L.tens_off = off;
  off = align256(off + sizeof(DevTensor) * size_t(n));
  L.max_chunks = 0;
  L.tab_off.resize(n);
  L.tab_bytes.resize(n);
  L.row_off.resize(n);
  L.variant.resize(n);
  L.group.resize(n);
  for (uint32_t v = 0; v < kNumGroups; ++v) L.group_tiles[v] = 0;
  for (int i = 0; i < n; ++i) {
    int rc = validate(descs[i], i);
    if (rc != EP_OK) return rc;
    const ep_tensor_desc& d = descs[i];
    const int ok = dtypes ? out_kind_of(dtypes[i]) : kOutBF16;
    if (ok < 0) return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": unknown output dtype");
    L.variant[i] = choose_variant(d);
    L.group[i] = L.variant[i] * kNumOutKinds + uint32_t(ok);
    L.tab_bytes[i] = storage_bytes_of(layout_of(L.variant[i]), d.prob_bits);
    L.max_chunks += (d.num_tiles + 1) / 2;
    L.group_tiles[L.group[i]] += d.num_tiles;
  }
  if (L.max_chunks >= (size_t(1) << 31)) return fail(EP_ERR_UNSUPPORTED, "too many tiles in one call");
  L.chunk_off = off;
  off = align256(off + sizeof(Chunk) * L.max_chunks);
  L.ctr_off = off;                    // one work counter per chunk slot
  off = align256(off + sizeof(uint32_t) * L.max_chunks);
  for (int i = 0; i < n; ++i) {
    L.tab_off[i] = off;
    off = align256(off + (descs[i].num_tiles ? L.tab_bytes[i] : 0));
    L.row_off[i] = off;
    off = align256(off + (descs[i].num_tiles ? 8 * size_t(descs[i].rows) : 0));
  }
  L.total = std::max<size_t>(off, 256);
  return EP_OK;
}

struct Group {
  uint32_t chunk_begin, nchunks, grid, tiles_per_chunk;
};

struct PlanImpl {
  void* ws;
  uint64_t magic;
  uint64_t ntensors;
  uint64_t ctr_off;                   // workspace offset of the per-chunk work counters
  Group groups[kNumGroups];
};
static_assert(sizeof(PlanImpl) <= sizeof(ep_batch_plan), "plan record too large");
constexpr uint64_t kPlanMagic = 0x45504c414e763036ull;

using KernelFn = void (*)(const DevTensor*, const Chunk*, uint32_t*, uint32_t, uint32_t);

template <int BT, int TL>
KernelFn kernel_for_kind(int ok) {
  switch (ok) {
    case kOutBF16: return decode_kernel<BT, TL, kOutBF16>;
    case kOutFP8: return decode_kernel<BT, TL, kOutFP8>;
    case kOutINT8: return decode_kernel<BT, TL, kOutINT8>;
    case kOutFP16: return decode_kernel<BT, TL, kOutFP16>;
    case kOutFP32: return decode_kernel<BT, TL, kOutFP32>;
    case kOutUINT8: return decode_kernel<BT, TL, kOutUINT8>;
    default: return decode_kernel<BT, TL, kOutLattice>;
  }
}

KernelFn kernel_of(uint32_t group) {
  const int ok = int(group % kNumOutKinds);
  switch (group / kNumOutKinds) {
    case kVarP9: return kernel_for_kind<9, kTabPacked>(ok);
    case kVarP10: return kernel_for_kind<10, kTabPacked>(ok);
    case kVarP11: return kernel_for_kind<11, kTabPacked>(ok);
    case kVarW10: return kernel_for_kind<10, kTabPackedWide>(ok);
    case kVarW11: return kernel_for_kind<11, kTabPackedWide>(ok);
    case kVarN12: return kernel_for_kind<12, kTabNarrow>(ok);
    case kVarH11: return kernel_for_kind<11, kTabHybrid>(ok);
    case kVarH12: return kernel_for_kind<12, kTabHybrid>(ok);
    default: return kernel_for_kind<0, kTabWorkspace>(ok);
  }
}

// Persistent grid: as many blocks as can be resident at once (at least one).
int resident_grid(uint32_t group, uint32_t* grid) {
  static int cus = 0;
  hipError_t e;
  if (cus == 0) {
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("device query: ") + hipGetErrorString(e));
  }
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel_of(group)),
                                                   kBlock, 0);
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("occupancy query: ") + hipGetErrorString(e));
  const uint64_t g = uint64_t(std::max(per_cu, 1)) * uint64_t(std::max(cus, 1));
  *grid = uint32_t(std::max<uint64_t>(1, std::min<uint64_t>(g, 1u << 20)));
  return EP_OK;
}

// Tiles per chunk: full blocks (kTilesPerChunk) when there is enough work to
// fill every resident block many times over; otherwise spread the tiles over
// all resident blocks (even counts, one tile per half-wave), since a tile is a
// sequential unit and a small batch is bound by the per-tile decode latency.
uint32_t tiles_per_chunk(size_t tiles, uint32_t resident) {
  if (tiles >= size_t(kTilesPerChunk) * resident) return kTilesPerChunk;
  const size_t per = (tiles + 2 * size_t(resident) - 1) / (2 * size_t(resident));
  return uint32_t(std::min<size_t>(kTilesPerChunk, std::max<size_t>(2, 2 * per)));
}

}  // namespace

// Lets the device compressor (ep_encode_gpu.hip) report through ep_last_error.
__attribute__((visibility("hidden"))) int ep_record_error(int code, const std::string& msg) {
  return fail(code, msg);
}

extern "C" {

const char* ep_status_string(int s) {
  switch (s) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
    case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE";
    case EP_ERR_HIP: return "EP_ERR_HIP";
    default: return "EP_UNKNOWN_STATUS";
  }
}

const char* ep_last_error(void) { return g_last_error.c_str(); }

int ep_abi_version(void) { return EP_ABI_VERSION; }

int ep_workspace_size(const ep_tensor_desc* descs, int n, size_t* bytes) {
  if (!bytes) return fail(EP_ERR_INVALID_ARG, "bytes is NULL");
  Layout L;
  int rc = make_layout(descs, nullptr, n, L);
  if (rc != EP_OK) return rc;
  *bytes = L.total;
  return EP_OK;
}

int ep_batch_prepare(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                     int32_t* const* tile_status, int n, void* workspace, size_t ws_bytes,
                     void* stream, ep_batch_plan* plan) {
  if (!plan) return fail(EP_ERR_INVALID_ARG, "plan is NULL");
  std::memset(plan, 0, sizeof(*plan));
  if (n > 0 && (!dtypes || !outs)) return fail(EP_ERR_INVALID_ARG, "NULL dtypes or outs");
  Layout L;
  int rc = make_layout(descs, dtypes, n, L);
  if (rc != EP_OK) return rc;
  if (!workspace || ws_bytes < L.total)
    return fail(EP_ERR_WORKSPACE, "workspace smaller than ep_workspace_size()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(EP_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  // only the descriptors travel; the build kernel writes the tile schedule
  std::vector<unsigned char> host(L.chunk_off, 0);
  DevTensor* ht = reinterpret_cast<DevTensor*>(host.data() + L.tens_off);
  uint32_t chunk_blocks = 0;
  char* wsb = static_cast<char*>(workspace);
  // chunks are grouped by (table placement, output kind); each group is one
  // launch with its own chunk size
  PlanImpl* P = reinterpret_cast<PlanImpl*>(plan);
  size_t group_chunks[kNumGroups] = {};
  for (uint32_t v = 0; v < kNumGroups; ++v) {
    Group& G = P->groups[v];
    G.grid = 0;
    G.tiles_per_chunk = kTilesPerChunk;
    if (L.group_tiles[v] == 0) continue;
    uint32_t resident = 0;
    rc = resident_grid(v, &resident);
    if (rc != EP_OK) return rc;
    G.tiles_per_chunk = tiles_per_chunk(L.group_tiles[v], resident);
    for (int i = 0; i < n; ++i)
      if (L.group[i] == v) group_chunks[v] += (descs[i].num_tiles + G.tiles_per_chunk - 1) / G.tiles_per_chunk;
    G.grid = uint32_t(std::min<size_t>(resident, group_chunks[v]));
  }
  size_t group_pos[kNumGroups];
  for (size_t v = 0, acc = 0; v < kNumGroups; ++v) {
    group_pos[v] = acc;
    P->groups[v].chunk_begin = uint32_t(acc);
    P->groups[v].nchunks = uint32_t(group_chunks[v]);
    acc += group_chunks[v];
  }
  for (int i = 0; i < n; ++i) {
    const ep_tensor_desc& d = descs[i];
    const int dt = dtypes[i];
    const int ok = out_kind_of(dt);
    const size_t align = out_vec_bytes(ok) >= 16 ? 16 : 8;
    if (d.num_tiles > 0 && (!outs[i] || reinterpret_cast<uintptr_t>(outs[i]) % align != 0))
      return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": output NULL or misaligned");
    DevTensor& D = ht[i];
    D.nvec = uint64_t(d.rows) * uint64_t(d.cols) / 8u;
    D.vpr = uint32_t(d.cols / 8);
    D.V = d.vectors_per_tile;
    D.T = d.num_tiles;
    D.b = d.prob_bits;
    D.rows = uint32_t(d.rows);
    D.scale = d.scale;
    D.variant = L.variant[i];
    D.tab_bytes = uint32_t(L.tab_bytes[i]);
    D.payload_words = d.payload_words;
    D.payload_bytes = uint32_t(2 * ((d.payload_words + 7) / 8 * 8));
    D.out_bytes = uint32_t(D.nvec * out_vec_bytes(ok));
    D.row_scales = d.row_scales;
    D.states = d.tile_states;
    D.offsets = d.tile_offsets;
    D.payload = d.payload;
    D.freqs = d.freqs;
    D.tab = reinterpret_cast<unsigned char*>(wsb + L.tab_off[i]);
    D.rowv = reinterpret_cast<float*>(wsb + L.row_off[i]);
    D.slow_rows = 0;
    D.f8z8 = d.field8 == EP_FIELD8_Z8 ? 1u : 0u;
    D.out = outs[i];
    D.status = tile_status ? tile_status[i] : nullptr;
    uint32_t em = 0, kpar = 0;
    for (int k = 0; k < kTables; ++k) {
      D.alphabet[k] = d.alphabet[k];
      D.freq_base[k] = d.freq_base[k];
      D.minv[k] = d.min_offset[k];
      if (k > 0 && d.alphabet[k] == 0) em |= 1u << k;
    }
    for (int c = 0; c < 2; ++c) {
      int64_t sum = 0;
      for (int f = 1; f <= 7; ++f) sum += d.min_offset[1 + 2 * (f - 1) + c];
      kpar |= uint32_t(sum & 1) << c;
    }
    const bool wide = layout_of(L.variant[i]) == kTabPackedWide;
    for (int t = 0; t < 32; ++t) D.kvals[t] = 0;
    for (int t = 0; t < 16; ++t) {
      const int64_t mn = d.min_offset[1 + t], c = t & 1;
      // f = 2^11 (a one-symbol table at b = 11) sets bit 22 of the packed entry
      const int64_t fb = (d.prob_bits == 11 && d.alphabet[1 + t] == 1) ? 1 : 0;
      // field 8: 4 m + c (2 z8 + c when z8 is coded directly)
      const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
      const int64_t kv = t >= 14 ? 12582912 - (k8 * mn + c) : wide ? 12582912 - mn : 12582912 + fb - (2 * mn + c);
      const float kf = float(kv);                   // exact: kv lies in [2^23, 2^24)
      std::memcpy(&D.kvals[t], &kf, 4);
    }
    const uint32_t psh = wide ? 22 : 23;
    D.kvals[16] = (kpar & 1u) << psh;
    D.kvals[17] = ((kpar >> 1) & 1u) << psh;
    // direct entries (packed layout): each field's values over both cosets
    // must fit the entry's 10 top bits as 2 (z - dmin) + c (4 (m - dmin) + c
    // for field 8), and every f must fit 11 bits
    {
      bool direct = layout_of(L.variant[i]) == kTabPacked;
      int64_t dsum = 0;
      const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
      for (int f = 1; f <= 8; ++f) {
        int64_t mn = 0, mx = -1;
        for (int c = 0; c < 2; ++c) {
          const int k = 1 + 2 * (f - 1) + c;
          if (d.alphabet[k] == 0) continue;
          if (d.prob_bits == 11 && d.alphabet[k] == 1) direct = false;   // f = 2^11
          const int64_t lo = d.min_offset[k], hi = lo + d.alphabet[k] - 1;
          if (mx < mn) mn = lo, mx = hi;
          else mn = std::min(mn, lo), mx = std::max(mx, hi);
        }
        if (mx < mn) mn = mx = 0;
        if ((f < 8 ? 2 : k8) * (mx - mn) + 1 > 1023) direct = false;
        D.dmin[f] = int32_t(mn);
        if (f < 8) {
          dsum += mn;
          const float kf = -float(12582912 - 2 * mn);
          std::memcpy(&D.kvals[18 + f - 1], &kf, 4);
        }
      }
      D.dmin[0] = 0;
      // field 8: 2 z8 + c = v8 + k8 dmin8 + 2 par (coded m), par = p ^ parity(sum of dmin1..7)
      const int64_t kd8 = (d.field8 == EP_FIELD8_Z8) ? 0 : (dsum & 1);
      const float k8f = -float(12582912 - k8 * D.dmin[8] - 2 * kd8);
      std::memcpy(&D.kvals[25], &k8f, 4);
      D.kvals[26] = uint32_t(d.field8 == EP_FIELD8_Z8 ? 0 : (kd8 ? -2 : 2));
      D.direct = direct ? 1u : 0u;
    }
    // hybrid at b = 11: per-slot entries when every value 2 z + c (4 m + c) fits
    // 16 bits; the build clears the flag if some f > 127
    {
      bool fits = has_split(layout_of(L.variant[i]), d.prob_bits);
      const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
      for (int k = 1; k < kTables && fits; ++k) {
        if (d.alphabet[k] == 0) continue;
        const int64_t mul = k >= 15 ? k8 : 2, c = (k - 1) & 1;
        const int64_t lo = mul * int64_t(d.min_offset[k]) + c;
        const int64_t hi = mul * (int64_t(d.min_offset[k]) + d.alphabet[k] - 1) + c;
        fits = lo >= -32768 && hi <= 32767;
      }
      D.split = fits ? 1u : 0u;
    }
    D.empty_mask = em;
    D.kpar = kpar;
    // the tensor's chunks (consecutive in its group's range) are written by the table build
    const uint32_t tpc = P->groups[L.group[i]].tiles_per_chunk;
    const uint32_t nch = uint32_t((uint64_t(d.num_tiles) + tpc - 1) / tpc);
    D.tpc = tpc;
    D.chunk0 = uint32_t(group_pos[L.group[i]]);
    group_pos[L.group[i]] += nch;
    chunk_blocks = std::max<uint32_t>(chunk_blocks, (nch + 1023u) / 1024u);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = host.empty() ? hipSuccess
                              : hipMemcpyAsync(wsb, host.data(), host.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
  if (n > 0) {
    uint64_t max_rows = 1;
    for (int i = 0; i < n; ++i) max_rows = std::max<uint64_t>(max_rows, uint64_t(descs[i].rows));
    const uint32_t row_blocks = uint32_t((max_rows + 1023) / 1024);
    hipLaunchKernelGGL(build_tables_kernel, dim3(16 + row_blocks + chunk_blocks, n), dim3(256), 0, st,
                       reinterpret_cast<DevTensor*>(wsb + L.tens_off), reinterpret_cast<Chunk*>(wsb + L.chunk_off),
                       row_blocks);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("table build launch: ") + hipGetErrorString(e));
  }
  P->ws = workspace;
  P->ctr_off = L.ctr_off;
  P->ntensors = uint64_t(n);
  P->magic = kPlanMagic;
  return EP_OK;
}

int ep_batch_launch(const ep_batch_plan* plan, void* stream) {
  if (!plan) return fail(EP_ERR_INVALID_ARG, "plan is NULL");
  const PlanImpl* P = reinterpret_cast<const PlanImpl*>(plan);
  if (P->magic != kPlanMagic) return fail(EP_ERR_INVALID_ARG, "plan was not filled by ep_batch_prepare");
  char* wsb = static_cast<char*>(P->ws);
  const DevTensor* tens = reinterpret_cast<const DevTensor*>(wsb);
  const Chunk* chunks = reinterpret_cast<const Chunk*>(wsb + align256(sizeof(DevTensor) * size_t(P->ntensors)));
  for (uint32_t v = 0; v < kNumGroups; ++v) {
    const Group& G = P->groups[v];
    if (G.nchunks == 0) continue;
    hipLaunchKernelGGL(kernel_of(v), dim3(G.grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream), tens,
                       chunks + G.chunk_begin, reinterpret_cast<uint32_t*>(wsb + P->ctr_off) + G.chunk_begin,
                       G.nchunks, G.tiles_per_chunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  }
  return EP_OK;
}

int ep_decode_batch(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                    int32_t* const* tile_status, int n, void* workspace, size_t ws_bytes,
                    void* stream) {
  ep_batch_plan plan;
  int rc = ep_batch_prepare(descs, dtypes, outs, tile_status, n, workspace, ws_bytes, stream, &plan);
  if (rc != EP_OK) return rc;
  return ep_batch_launch(&plan, stream);
}

int ep_decode_tensor(const ep_tensor_desc* desc, int dtype, void* out, int32_t* tile_status,
                     void* workspace, size_t ws_bytes, void* stream) {
  if (!desc) return fail(EP_ERR_INVALID_ARG, "desc is NULL");
  void* outs[1] = {out};
  int32_t* sts[1] = {tile_status};
  return ep_decode_batch(desc, &dtype, outs, sts, 1, workspace, ws_bytes, stream);
}

int ep_convert_f32(const float* in, void* out, uint64_t n, int dtype, void* stream) {
  if (n % 4 != 0) return fail(EP_ERR_INVALID_ARG, "n must be a multiple of 4");
  if (n == 0) return EP_OK;
  if (!in || !out || reinterpret_cast<uintptr_t>(in) % 16 || reinterpret_cast<uintptr_t>(out) % 8)
    return fail(EP_ERR_INVALID_ARG, "in must be 16-byte and out 8-byte aligned device pointers");
  const uint64_t n4 = n / 4;
  const dim3 grid(uint32_t(std::min<uint64_t>((n4 + 255) / 256, 1u << 16)));
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case EP_OUT_BF16: hipLaunchKernelGGL(convert_kernel<kOutBF16>, grid, dim3(256), 0, st, in, out, n4); break;
    case EP_OUT_FP16: hipLaunchKernelGGL(convert_kernel<kOutFP16>, grid, dim3(256), 0, st, in, out, n4); break;
    case EP_OUT_FP8_E4M3: hipLaunchKernelGGL(convert_kernel<kOutFP8>, grid, dim3(256), 0, st, in, out, n4); break;
    case EP_OUT_INT8: hipLaunchKernelGGL(convert_kernel<kOutINT8>, grid, dim3(256), 0, st, in, out, n4); break;
    case EP_OUT_UINT8: hipLaunchKernelGGL(convert_kernel<kOutUINT8>, grid, dim3(256), 0, st, in, out, n4); break;
    default: return fail(EP_ERR_INVALID_ARG, "dtype must be BF16, FP16, FP8_E4M3, INT8 or UINT8");
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("convert launch: ") + hipGetErrorString(e));
  return EP_OK;
}

}  // extern "C"
