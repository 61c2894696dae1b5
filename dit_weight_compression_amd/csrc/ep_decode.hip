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
#include <atomic>
#include <chrono>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "entropack.h"

// global (not flat) addressing for pointers read from the descriptors
#define EP_GLOBAL __attribute__((address_space(1)))
#define EP_LDS __attribute__((address_space(3)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// ring words are written as 32-bit pairs and read as 16-bit words: the stores go
// through a type that may alias any other, so type-based alias analysis can
// never move a ring read across the write of the words it reads
typedef uint32_t __attribute__((may_alias)) u32_ring;

namespace {

constexpr uint32_t kL = 1u << 15;          // lower bound of the state interval
constexpr int kTables = EP_NUM_TABLES;
constexpr int kWavesPerBlock = 16;
constexpr int kBlock = 64 * kWavesPerBlock;
constexpr int kMaxChains = 2;                // independent tile pairs a wave decodes together
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
//             symbol a pair of words, u32 f | (cum + coset*2^b) << 16 (bit 15:
//             parity of z) and the float value 2 z + c (4 m + c for m), at a
//             stride of 256 pairs, so that one 8-byte read gets both.
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
// packed and wide layouts: the byte-entry tables (when the tensor can use them)
// follow the 16 packed tables in the workspace: fields 1..7 in the fp16 form,
// or all 16 tables in the i16 form (see DevTensor::byte_cand)
__host__ __device__ constexpr size_t byte_off_of(uint32_t b) { return size_t(16) << (b + 2); }
__host__ __device__ constexpr size_t byte_bytes_of(uint32_t b) { return size_t(14) << (b + 2); }
__host__ __device__ constexpr size_t byte16_bytes_of(uint32_t b) { return size_t(16) << (b + 2); }
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
  uint32_t call;             // the preparing call's number (never 0); a bad_* word holding it is set
  uint32_t f8z8;             // 1: field 8 holds z8 (no parity reduction), 0: it holds m
  uint32_t chunk0;           // index of the tensor's first chunk in the schedule
  uint32_t tpc;              // tiles per chunk of the tensor's launch group
  uint32_t direct;           // packed layouts: entries hold the value 2 z + c - 2 dmin (see kvals)
  uint32_t split;            // hybrid layout: 1 = per-slot entries usable, unless bad_split says otherwise
  uint32_t byte_cand;        // byte-entry tables in the workspace (set by the host): 0 none; 1 fields 1..7 as
                             // f | (slot - cum) << 8 | fp16(1024 + 2 (z - dmin) + c) << 16 (direct packed
                             // tensors); 2 all 16 tables as f | (slot - cum) << 8 | i16 value << 16
  uint32_t bytev;            // ... and they are usable, unless bad_bytes says otherwise
  uint32_t kbyte[4];         // byte entries: fp16 pairs (2 dmin_f - 1024) for fields (1,2), (3,4), (5,6), (-,7)
  int32_t dmin[9];           // direct entries: per field, the smaller of the two cosets' minima
  uint64_t payload_words;
  const float* row_scales;
  float* rowv;               // workspace: g/2 of rows 0..rows-1, then g of the same rows, g = fp32(scale * row scale)
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
  // Flags that depend on device data, stored by the table build's blocks as
  // the call number when the condition holds (never written otherwise, so no
  // word has to be cleared first; a stale or unrelated value that happens to
  // equal the number only selects the slower exact path):
  uint32_t bad_split;        // a table of the hybrid layout has f > 127: the per-slot entries are unusable
  uint32_t bad_bytes;        // a byte-entry table has f > 255: the byte entries are unusable
  uint32_t bad_rows;         // some row's g / 2 is inexact: multiply by g
};

// The layout checks in the tests read these fields of the workspace copy
// (descriptor i at byte i * sizeof(DevTensor)) back after ep_batch_prepare.
static_assert(sizeof(DevTensor) == 576, "DevTensor layout read by the tests");
static_assert(offsetof(DevTensor, variant) == 36 && offsetof(DevTensor, call) == 56 &&
                  offsetof(DevTensor, direct) == 72 && offsetof(DevTensor, split) == 76 &&
                  offsetof(DevTensor, byte_cand) == 80 && offsetof(DevTensor, bytev) == 84 &&
                  offsetof(DevTensor, bad_split) == 556 && offsetof(DevTensor, bad_bytes) == 560 &&
                  offsetof(DevTensor, bad_rows) == 564,
              "DevTensor layout read by the tests");

struct Chunk {
  uint32_t tensor;
  uint32_t tile0;
};

thread_local std::string g_last_error;

// A number per ep_batch_prepare call, never 0, starting from a clock-derived
// value so that numbers left in reused memory by another process rarely match.
uint32_t next_call_number() {
  static std::atomic<uint32_t> counter{
      uint32_t(std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B1ull) | 1u};
  uint32_t v;
  do v = counter.fetch_add(1u, std::memory_order_relaxed);
  while (v == 0u);
  return v;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- table build
// Exclusive scan (sum or max, identity 0) of one value per thread over a
// 256-thread block: a shuffle scan inside each wave, then the wave totals.
template <bool kMax>
__device__ __forceinline__ uint32_t block_scan256_excl(uint32_t v, uint32_t* __restrict__ part) {
  const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) {
    const uint32_t u = uint32_t(__shfl_up(int(incl), d, 64));
    if (lane >= d) incl = kMax ? max(incl, u) : incl + u;
  }
  if (lane == 63u) part[w] = incl;
  uint32_t ex = uint32_t(__shfl_up(int(incl), 1u, 64));
  if (lane == 0u) ex = 0u;
  __syncthreads();
  uint32_t pre = 0;
  for (uint32_t i = 0; i < w; ++i) pre = kMax ? max(pre, part[i]) : pre + part[i];
  __syncthreads();                               // part is reusable after this
  return kMax ? max(pre, ex) : pre + ex;
}

// Dynamic LDS of the table build for one tensor's tables: packed layouts
// first stage their entries (two u32 per slot: packed and byte entries) so
// that the copy to the workspace is coalesced; then the slot marks (u16 per
// slot) and the table's frequencies (u16 per symbol).  The launch takes the
// largest over the batch.
__host__ __device__ constexpr size_t build_lds_bytes(bool packed, uint32_t b, uint32_t alphabet) {
  return (packed ? size_t(8) << b : 0) + (((size_t(2) << b) + 2u * size_t(alphabet) + 15u) / 16u * 16u);
}

// Batches of up to kArgTensors tensors pass their descriptors to the table
// build as kernel arguments (576 bytes each; the argument block stays under
// 4 KiB), so no host-to-device copy precedes the build, and one more block per
// tensor writes the descriptor to the workspace; larger batches copy the
// descriptors to the workspace before the build.
constexpr int kArgTensors = 6;
template <int NA>
struct DescArgs {
  DevTensor t[NA];
};
template <>
struct DescArgs<0> {};

// Per tensor (blockIdx.y): 16 table blocks, row_blocks blocks of row
// multipliers, the blocks of its tile schedule and, with descriptors in the
// kernel arguments, the block that writes the descriptor.
//
// A table block: cumulative frequencies by a block scan over per-thread symbol
// ranges; every symbol with f > 0 marks the slot where its interval starts, and
// a forward scan over the slots carries the last mark, which is the slot's
// symbol (a zero-frequency symbol never marks).
template <int NA>
__global__ __launch_bounds__(256) void build_tables_kernel(DevTensor* __restrict__ tens, Chunk* __restrict__ chunks,
                                                          uint32_t row_blocks, DescArgs<NA> args) {
  const DevTensor& T = [&]() -> const DevTensor& {
    if constexpr (NA > 0) return args.t[blockIdx.y];
    else return tens[blockIdx.y];
  }();
  DevTensor& W = tens[blockIdx.y];             // the workspace copy: flags are stored there
  if constexpr (NA > 0) {
    if (blockIdx.x == gridDim.x - 1u) {
      // every word up to the flags, which only the blocks that find a condition write
      constexpr uint32_t kWords = offsetof(DevTensor, bad_split) / 4u;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(&T);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&W);
      for (uint32_t i = threadIdx.x; i < kWords; i += blockDim.x) dst[i] = src[i];
      return;
    }
  }
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
    // (z + c/2) * g exactly whenever g / 2 is exact; g/2 and g are stored in
    // two arrays (the decoder reads one of them, 4 bytes per row) and a
    // tensor with any row where g / 2 is inexact uses g.
    const uint32_t r0 = (blockIdx.x - 16) * 1024u;
    bool inexact = false;
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i) {
      const uint32_t r = r0 + threadIdx.x + 256u * i;
      if (r < T.rows) {
        const float gr = __fmul_rn(T.scale, T.row_scales[r]);
        const float h = __fmul_rn(gr, 0.5f);
        inexact |= !(__fmul_rn(h, 2.0f) == gr);
        T.rowv[r] = h;
        T.rowv[T.rows + r] = gr;
      }
    }
    if (__syncthreads_or(inexact) && threadIdx.x == 0) W.bad_rows = T.call;
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
  // byte entries: fields 1..7 as f | (slot - cum) << 8 | fp16(1024 + n) << 16 with
  // n = 2 z + c - 2 dmin_f (the value relative to the field's smaller minimum), or
  // every table as f | (slot - cum) << 8 | i16(2 z + c, or 4 m + c) << 16
  const bool by16 = T.byte_cand == 2u;
  const bool bywrite = (T.byte_cand == 1u && field <= 7) || by16;
  uint32_t* lutb = reinterpret_cast<uint32_t*>(T.tab + byte_off_of(b)) + (size_t(t) << b);
  const size_t lb = lut_bytes_of(tl, b);
  // per-symbol pairs (entry, value) of the narrow, workspace and hybrid layouts
  uint32_t* sym = reinterpret_cast<uint32_t*>(T.tab + lb) + size_t(t) * S * 2u;
  float* val = reinterpret_cast<float*>(sym) + 1;
  extern __shared__ __align__(16) uint32_t build_lds[];
  uint32_t* st32 = build_lds;                  // packed layouts: staged entries, packed then byte
  uint32_t* stb = build_lds + M;
  uint16_t* mark = reinterpret_cast<uint16_t*>(build_lds + (is_packed(tl) ? 2u * M : 0u));
  uint16_t* fl = mark + M;                     // the table's frequencies
  // per slot, mark: 1 + the symbol whose interval starts there, else 0
  __shared__ uint32_t part[4];
  if (!is_packed(tl)) {
    for (uint32_t i = A + threadIdx.x; i < S; i += blockDim.x) {
      sym[2u * i] = 0;
      val[2u * i] = 0.0f;
    }
  }
  if (A == 0) {   // empty table: never used, the decoder flags the tile
    for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) {
      if (is_packed(tl)) {
        lut32[j] = 1u << 11;                          // f = 1, slot - cum = 0, symbol 0
        if (bywrite) lutb[j] = by16 ? 1u : 1u | (0x6400u << 16);  // f = 1, slot - cum = 0, value / n = 0
      } else if (tl == kTabNarrow) lut8[j] = 0;
      else lut16[j] = 0;
      if (split) {
        fd16[j] = 1;                                // f = 1, slot - cum = 0
        sval[j] = 0;
      }
    }
    return;
  }
  const uint16_t* fr = T.freqs + T.freq_base[k];
  const int32_t mn = T.minv[k];
  for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) mark[j] = 0;
  for (uint32_t i = threadIdx.x; i < A; i += blockDim.x) fl[i] = fr[i];
  __syncthreads();
  // cumulative frequencies: thread tid owns the symbols [tid Q, tid Q + Q)
  {
    const uint32_t Q = (A + 255u) / 256u;
    const uint32_t i0 = min(A, threadIdx.x * Q), i1 = min(A, i0 + Q);
    uint32_t sum = 0;
    for (uint32_t i = i0; i < i1; ++i) sum += fl[i];
    uint32_t cum = block_scan256_excl<false>(sum, part);
    for (uint32_t i = i0; i < i1; ++i) {
      const uint32_t f = fl[i];
      if (f > 0u && cum < M) mark[cum] = uint16_t(i + 1u);       // distinct slots: cum grows with f > 0
      if (!is_packed(tl)) {
        // the narrow layout (b = 12, f <= 4096) keeps the parity of the value z in bit 15
        const uint32_t zpar = (tl == kTabNarrow && field < 8) ? (uint32_t(int32_t(i) + mn) & 1u) << 15 : 0u;
        sym[2u * i] = (f & 0xFFFFu) | zpar | ((cum + (c << b)) << 16);
        const int32_t z = int32_t(i) + mn;
        val[2u * i] = float(field < 8 || T.f8z8 ? 2 * z + int32_t(c) : 4 * z + int32_t(c));
      }
      cum += f;
    }
  }
  __syncthreads();
  // slot j -> the last mark at or below it: thread tid owns the slots [tid R, tid R + R)
  const uint32_t R = M / 256u;
  const uint32_t j0 = threadIdx.x * R;
  uint32_t last = 0;                           // (slot + 1) << 16 | (symbol + 1) of a mark
  for (uint32_t q = 0; q < R; ++q) {
    const uint32_t mk = mark[j0 + q];
    if (mk) last = ((j0 + q + 1u) << 16) | mk;
  }
  uint32_t key = block_scan256_excl<true>(last, part);
  int big = 0, big8 = 0;
  for (uint32_t q = 0; q < R; ++q) {
    const uint32_t j = j0 + q;
    const uint32_t mk = mark[j];
    if (mk) key = ((j + 1u) << 16) | mk;
    // with sum f = M slot 0 always holds a mark; a table without one decodes garbage, in bounds
    const uint32_t lo = key ? (key & 0xFFFFu) - 1u : 0u;
    const uint32_t cum = key ? (key >> 16) - 1u : 0u;
    const uint32_t f = fl[lo];
    if (is_packed(tl)) {
      // the entry's top bits: the symbol index, or (direct entries) the value
      // 2 z + c (4 m + c for field 8) relative to the field's smaller minimum
      uint32_t top = lo << (tl == kTabPacked ? 23 : 22);
      if (tl == kTabPacked && T.direct) {
        const int32_t d = int32_t(lo) + mn - T.dmin[field];
        top = uint32_t((field < 8 || T.f8z8 ? 2 * d : 4 * d) + int32_t(c)) << 22;
      }
      st32[j] = (j - cum) | ((f & 0xFFFFu) << 11) | top;
      if (bywrite) {
        big8 |= f > 255u;
        if (by16) {
          const int32_t z = int32_t(lo) + mn;
          const int32_t v = field < 8 || T.f8z8 ? 2 * z + int32_t(c) : 4 * z + int32_t(c);   // i16: checked on the host
          stb[j] = (f & 0xFFu) | ((j - cum) << 8) | (uint32_t(uint16_t(int16_t(v))) << 16);
        } else {
          const uint32_t n = uint32_t(2 * (int32_t(lo) + mn - T.dmin[field]) + int32_t(c));   // < 1024: checked on the host
          stb[j] = (f & 0xFFu) | ((j - cum) << 8) | ((0x6400u | n) << 16);
        }
      }
    } else if (tl == kTabNarrow) {
      lut8[j] = uint8_t(lo);
    } else {
      lut16[j] = uint16_t(lo);
      if (split) {
        const uint32_t d = j - cum;
        const int32_t z = int32_t(lo) + mn;
        const uint32_t zp = field < 8 ? (uint32_t(z) & 1u) : 0u;
        big |= f > 127u;
        fd16[j] = uint16_t((f & 0x7Fu) | (d << 7) | (zp << 15));
        // |value| < 2^15: checked on the host
        sval[j] = int16_t(field < 8 || T.f8z8 ? 2 * z + int32_t(c) : 4 * z + int32_t(c));
      }
    }
  }
  if (is_packed(tl)) {
    // the staged entries to the workspace, 16 bytes per thread and store
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < M / 4u; i += blockDim.x) {
      reinterpret_cast<u32x4*>(lut32)[i] = reinterpret_cast<const u32x4*>(st32)[i];
      if (bywrite) reinterpret_cast<u32x4*>(lutb)[i] = reinterpret_cast<const u32x4*>(stb)[i];
    }
  }
  // per-slot entries hold f in 7 bits: any larger frequency disables them for the tensor
  if (__syncthreads_or(big) && threadIdx.x == 0) W.bad_split = T.call;
  // byte entries hold f in 8 bits: any larger frequency disables them for the tensor
  if (__syncthreads_or(big8) && threadIdx.x == 0) W.bad_bytes = T.call;
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
// byte of the sum's bit pattern.  The first sum is a whole word; the other
// three are sub-dword adds that write their low byte into byte 1, 2, 3 of that
// word and keep the rest, so the word ends up holding the four codes.
template <int BYTE>
__device__ __forceinline__ void add_f32_to_byte(uint32_t& w, float x, float m) {
  if constexpr (BYTE == 1)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(x), "v"(m));
  else if constexpr (BYTE == 2)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(x), "v"(m));
  else
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(w) : "v"(x), "v"(m));
}
template <bool kUnsigned>
__device__ __forceinline__ uint32_t int8_codes4(float a, float b, float c, float d) {
  constexpr float kMagic = kUnsigned ? 12583040.0f : 12582912.0f;
  float m = kMagic;
  asm volatile("" : "+v"(m));                                     // the sub-dword adds take it from a VGPR
  uint32_t w = __float_as_uint(__builtin_amdgcn_fmed3f(a, -128.0f, 127.0f) + m);
  add_f32_to_byte<1>(w, __builtin_amdgcn_fmed3f(b, -128.0f, 127.0f), m);
  add_f32_to_byte<2>(w, __builtin_amdgcn_fmed3f(c, -128.0f, 127.0f), m);
  add_f32_to_byte<3>(w, __builtin_amdgcn_fmed3f(d, -128.0f, 127.0f), m);
  return w;
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
// LDS ring of kRingWords, filled kChunkWords at a time (one 4-byte load per
// lane).  Before a round starts, the words its first five fields can read are
// staged; after field 4 a check makes sure the words the last four fields can
// read are there too (rarely not: a round reads about a fifth of its worst
// case).  Every memory operation is a raw buffer operation, whose out-of-range
// lanes the hardware turns into zero loads and dropped stores; a prefetch at or
// past the tile's last word gets an out-of-range offset and reads nothing.
constexpr uint32_t kRingWords = 256;
constexpr uint32_t kChunkWords = 64;
constexpr uint32_t kHead0 = 5 * 32;                       // most words fields 0..4 of a round read
constexpr uint32_t kHead1 = 4 * 32;                       // most words fields 5..8 read
constexpr uint32_t kRingSlack = kRingWords - kChunkWords; // a chunk fits while fill <= read + slack
static_assert(kHead0 + kChunkWords <= kRingWords && kHead1 + kChunkWords <= kRingWords,
              "a staged segment and the chunk being written must fit the ring");

// LDS of the payload rings: every wave holds 2 * CH rings (CH chains of two tiles)
__host__ __device__ constexpr size_t ring_bytes_of(int ch) {
  return size_t(kWavesPerBlock) * 2u * size_t(ch) * kRingWords * sizeof(uint16_t);
}
constexpr size_t kRingBytesMax = ring_bytes_of(kMaxChains);

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

// Byte entries (see build_tables_kernel): the state update f * q + (slot - cum)
// with f and slot - cum taken straight from bytes 0 and 1 of the entry by the
// sub-dword operand selects of gfx950's VOP2 encoding, two instructions.
__device__ __forceinline__ uint32_t mul_byte0(uint32_t e, uint32_t q) {
  uint32_t r;
  asm("v_mul_u32_u24_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
      : "=v"(r) : "v"(e), "v"(q));
  return r;
}
__device__ __forceinline__ uint32_t add_byte1(uint32_t e, uint32_t a) {
  uint32_t r;
  asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
      : "=v"(r) : "v"(e), "v"(a));
  return r;
}
// fp32(v * h) for the fp16 value v in the low (HI = false) or high half of p:
// one fused mixed-precision multiply-add with the addend -0, which rounds the
// exact product once and keeps the sign of a zero product, as a plain fp32
// multiply of float(v) by h does.
template <bool HI>
__device__ __forceinline__ float mul_f16_f32(uint32_t p, float h) {
  float r;
  if (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(p), "v"(h), "s"(-0.0f));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(p), "v"(h), "s"(-0.0f));
  return r;
}
typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));
// exact fp16 additions: (1024 + n) + (2 dmin - 1024) = 2 z + c, both halves
__device__ __forceinline__ uint32_t add_f16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h16x2_t, a) + __builtin_bit_cast(h16x2_t, b));
}

// Decode the 2*CH consecutive tiles tile0 .. tile0 + 2*CH - 1 of one wave (those
// below tile_end).  Chain c of the wave is the tile pair tile0 + 2c, tile0 + 2c + 1,
// one tile per half-wave; lane l of a half owns the tile's rANS state l.  The CH
// chains are independent and advance round by round together: while one
// chain waits for a table lookup, the other's arithmetic can issue, so a wave
// exposes less of the LDS latency of its serial per-symbol chain.
//
// BT is the probability precision when known at compile time (0: read T.b),
// TL the table layout (LDS tables start at LDS address 0), OK the output kind,
// SP (hybrid layout) whether the per-slot entry maps are the ones staged in
// LDS, CH the number of chains, BY (packed and wide layouts) which byte entries
// are staged: 0 none, 1 fields 1..7 in the fp16 form, 2 every table in the i16
// form (DevTensor::byte_cand).  `rings` points to this wave's 2*CH rings.
template <int BT, int TL, int OK, bool SP, int CH, int BY>
__device__ __forceinline__ void decode_tiles(const DevTensor& T, uint32_t tile0, uint32_t tile_end,
                                             const unsigned char* __restrict__ lds,
                                             uint16_t* __restrict__ rings) {
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
  const uint32_t hs32 = half << 5;                          // selects this half's 32 ballot bits
  const uint32_t l = lane & 31u;
  const uint32_t lane2 = 2u * l;                            // this lane's words inside a chunk

  const __amdgpu_buffer_rsrc_t rP = make_rsrc(T.payload, T.payload_bytes);
  // descriptor fields used inside the round loop, read once: the output
  // stores could alias the descriptor as far as the compiler knows
  const uint32_t vpr = T.vpr;
  const uint32_t out_bytes = T.out_bytes;
  const uint32_t payload_bytes = T.payload_bytes;
  const __amdgpu_buffer_rsrc_t rO = make_rsrc(T.out, out_bytes);
  const __amdgpu_buffer_rsrc_t rR = make_rsrc(T.rowv, T.rows * 8u);
  const bool slow_rows = T.bad_rows == T.call;

  // ---- per-chain tile start.  Uniform values of a chain's two tiles live in
  // scalar registers; each lane keeps its half's ring read pointer (vP) so
  // that the renormalisation needs no scalar bookkeeping.
  uint32_t n[CH], x[CH], vP[CH], F0[CH], F1[CH], end0[CH], end1[CH], n0[CH], n1[CH];
  uint32_t chunk_lane[CH], endl[CH], pf[CH], g[CH], rowb[CH], col[CH];
  uint64_t empty_err[CH];
  bool bad_len[CH], tile_ok[CH];
  uint32_t kfull = ~0u, kmax = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t t = tile0 + 2u * uint32_t(c) + half;     // tile of this half-wave
    tile_ok[c] = t < tile_end;                               // tile_end <= T.T
    uint32_t p = 0, pend = 0;
    n[c] = 0;
    x[c] = kL;
    bad_len[c] = false;
    if (tile_ok[c]) {
      const uint64_t first = uint64_t(t) * T.V;
      n[c] = uint32_t(min(uint64_t(T.V), T.nvec - first));
      x[c] = ((const EP_GLOBAL uint32_t*)T.states)[size_t(t) * EP_LANES + l];
      p = ((const EP_GLOBAL uint32_t*)T.offsets)[t];
      pend = ((const EP_GLOBAL uint32_t*)T.offsets)[t + 1];
      if (pend < p || pend > T.payload_words) {
        bad_len[c] = true;
        n[c] = 0;
        pend = p;
      }
    }
    n0[c] = __builtin_amdgcn_readlane(n[c], 0);
    n1[c] = __builtin_amdgcn_readlane(n[c], 32);
    const uint32_t st0 = __builtin_amdgcn_readlane(p, 0), st1 = __builtin_amdgcn_readlane(p, 32);
    const uint32_t a00 = st0 & ~1u, a01 = st1 & ~1u;         // 4-byte aligned first word
    end0[c] = __builtin_amdgcn_readlane(pend, 0) - a00;       // ring-relative word counts
    end1[c] = __builtin_amdgcn_readlane(pend, 32) - a01;
    vP[c] = half ? st1 - a01 : st0 - a00;                     // ring-relative read pointer
    F0[c] = 0;                                                // words written to the ring
    F1[c] = 0;
    empty_err[c] = 0;
    chunk_lane[c] = 2u * ((half ? a01 : a00) + lane2);       // byte offset of this lane's part
    // chunks that start at word F: this lane's two words hold some of the
    // tile's payload while F < endl (lanes past the tile's last word load
    // nothing, so no cache line beyond the tile is fetched for them)
    const uint32_t Eh = half ? end1[c] : end0[c];
    endl[c] = Eh > lane2 ? Eh - lane2 : 0u;
    // the chunk held in registers is always the one starting at word F of the half
    pf[c] = __builtin_amdgcn_raw_buffer_load_b32(rP, endl[c] > 0u ? chunk_lane[c] : payload_bytes, 0, 0);
    kfull = min(kfull, min(n0[c], n1[c]) >> 5);
    kmax = max(kmax, max((n0[c] + 31u) >> 5, (n1[c] + 31u) >> 5));
    g[c] = t * T.V + l;                                       // < 2^32: checked on the host
    // rowb: byte offset of the row multiplier, g/2 or (slow rows) g
    rowb[c] = slow_rows ? 4u * T.rows : 0u;
    col[c] = 0;
    if (tile_ok[c]) {
      const uint32_t row = g[c] / vpr;
      col[c] = g[c] - row * vpr;
      rowb[c] += 4u * row;
    }
  }
  // A store past the end of the output per chain (dropped by the hardware): it
  // makes the first round see the same queue of outstanding memory operations
  // as every later round, so the compiler's waits stay exact.
#pragma unroll
  for (int c = 0; c < CH; ++c) __builtin_amdgcn_raw_buffer_store_b32(0u, rO, out_bytes, 0, 0);

  const uint32_t f0 = ((const EP_GLOBAL uint16_t*)T.freqs)[T.freq_base[0]];   // coset bit: frequency of c = 0
  uint32_t f0v = f0, f1v = M - f0;                          // per-lane copies for the selects
  asm volatile("" : "+v"(f0v), "+v"(f1v));
  const uint32_t kpar = T.kpar;
  // field 8: m (value 4 s + 2 parity + const) or z8 itself (2 s + const, no parity)
  const uint32_t pw = T.f8z8 ? 0u : 1u;                     // width of the parity bit field
  const uint32_t sh8 = T.f8z8 ? 1u : 2u;
  const uint32_t empty = T.empty_mask;
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
  uint32_t kb[4] = {0, 0, 0, 0};
  if (BY == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = T.kbyte[i];
  }
  if (kDirectable) {
#pragma unroll
    for (int f = 0; f < 7; ++f) kd[f] = __builtin_bit_cast(float, T.kvals[18 + f]);
    k8d = __builtin_bit_cast(float, T.kvals[25]);
    m8d = int32_t(T.kvals[26]);
  }

  // ---- ring staging of chain c before a segment of fields that reads at most
  // `head` words per half: store the held chunk if it is useful and fits,
  // catch up synchronously while the segment could read past the staged words
  // (tile starts, dense runs), then fetch the chunk at the new fill position.
  auto stage = [&](const int c, const uint32_t head) __attribute__((always_inline)) {
    uint16_t* ring = rings + (2u * uint32_t(c) + half) * kRingWords;
    const uint32_t P0 = __builtin_amdgcn_readlane(vP[c], 0);
    const uint32_t P1 = __builtin_amdgcn_readlane(vP[c], 32);
    {
      const bool w0 = F0[c] < end0[c] && F0[c] <= P0 + kRingSlack;
      const bool w1 = F1[c] < end1[c] && F1[c] <= P1 + kRingSlack;
      // both halves' predicates as one lane mask (the branch takes it as exec);
      // the fill pointers packed in one scalar, a lane extracts its half's 16
      // bits (tile payloads stay below 2^16 words)
      if (__builtin_amdgcn_inverse_ballot_w64(half_mask(w0, w1))) {
        const uint32_t F = __builtin_amdgcn_ubfe(F0[c] | (F1[c] << 16), hs, 16);
        *reinterpret_cast<u32_ring*>(ring + ((F + lane2) & (kRingWords - 1u))) = pf[c];
      }
      F0[c] += w0 ? kChunkWords : 0u;
      F1[c] += w1 ? kChunkWords : 0u;
    }
    for (;;) {
      const bool c0 = F0[c] < min(P0 + head, end0[c]);
      const bool c1 = F1[c] < min(P1 + head, end1[c]);
      if (!(c0 || c1)) break;
      if (__builtin_amdgcn_inverse_ballot_w64(half_mask(c0, c1))) {
        const uint32_t F = __builtin_amdgcn_ubfe(F0[c] | (F1[c] << 16), hs, 16);
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rP, F < endl[c] ? chunk_lane[c] + 2u * F
                                                                                : payload_bytes, 0, 0);
        *reinterpret_cast<u32_ring*>(ring + ((F + lane2) & (kRingWords - 1u))) = v;
      }
      F0[c] += c0 ? kChunkWords : 0u;
      F1[c] += c1 ? kChunkWords : 0u;
    }
    const uint32_t F = __builtin_amdgcn_ubfe(F0[c] | (F1[c] << 16), hs, 16);
    pf[c] = __builtin_amdgcn_raw_buffer_load_b32(rP, F < endl[c] ? chunk_lane[c] + 2u * F : payload_bytes, 0, 0);
  };

  // Renormalisation of every chain: the lanes of a half whose state fell below
  // 2^15 read the next words of their tile in lane order.  A lane's word is its
  // half's pointer plus the number of reading lanes below it in the half
  // (popcount of the half's ballot bits under the lane).  Every lane reads (the
  // index stays inside the ring) and keeps the word only if it needed one: no
  // exec masking and no scalar pointer updates on the serial path.  The chains
  // go through each step together, so that their reads are in flight at the
  // same time.
  auto renorm = [&](const bool (&active)[CH]) __attribute__((always_inline)) {
    bool rn[CH];
    uint32_t hm[CH], w[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) rn[c] = (x[c] < kL) & active[c];
#pragma unroll
    for (int c = 0; c < CH; ++c) hm[c] = uint32_t(__builtin_amdgcn_ballot_w64(rn[c]) >> hs32);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint16_t* ring = rings + (2u * uint32_t(c) + half) * kRingWords;
      const uint32_t idx = __builtin_popcount(__builtin_amdgcn_ubfe(hm[c], 0, l)) + vP[c];
      // a volatile read: it stays unconditional (not sunk into a branch on rn)
      w[c] = *(const volatile EP_LDS uint16_t*)(ring + (idx & (kRingWords - 1u)));
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      x[c] = rn[c] ? ((x[c] << 16) | w[c]) : x[c];
      vP[c] += __builtin_popcount(hm[c]);
    }
  };

  // One vector round of every chain.  In full rounds every lane of every
  // chain has a vector, so the active-lane masks fold away.
  auto round = [&](const uint32_t k, auto full) __attribute__((always_inline)) {
    constexpr bool kFull = decltype(full)::value;
    bool active[CH];
    uint32_t x_saved[CH], cs[CH];
    float vv[CH][9];
    float yb[CH][7];                                          // byte entries: the products of fields 1..7
    float rv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      active[c] = kFull || (k * 32u + l) < n[c];
      x_saved[c] = x[c];
      // issued before the ring prefetch: loads retire in order, so waiting for
      // the row multiplier later does not also wait for the prefetch
      rv[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, rowb[c], 0, 0));
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) stage(c, kHead0);

    // ---- field 0: coset bit (two-symbol table, resolved by one compare)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t q = x[c] >> B;
      const uint32_t slot = x[c] & MASK;
      const bool cb = slot >= f0v;
      cs[c] = cb ? 1u : 0u;
      x[c] = __umul24(cb ? f1v : f0v, q) + slot - (cb ? f0v : 0u);
    }
    renorm(active);
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (empty & 6u) empty_err[c] |= __builtin_amdgcn_ballot_w64(active[c] && ((empty >> (cs[c] ? 2 : 1)) & 1u));

    // ---- fields z1..z7, m; vv[c][f] becomes 2 z_f + c (exact in fp32)
    uint32_t par[CH];
    if constexpr (is_packed(TL)) {
      uint32_t ev[CH][9], lbl[CH], lbh[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        lbl[c] = cs[c] ? (M << 2) : 0u;                    // byte offset of the coset's table
        lbh[c] = lbl[c] + (kSplit ? (8u << B) * 4u : 0u);
        // opaque to the optimiser, so that the lookup address stays one
        // v_and_or_b32 with the table offset folded into the LDS instruction
        asm volatile("" : "+v"(lbl[c]), "+v"(lbh[c]));
      }
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        const bool hi = kSplit && f >= 5;
        const uint32_t toff = (uint32_t(2 * (f - 1) - (hi ? 8 : 0)) << B) * 4u;
        uint32_t e[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c)
          e[c] = *reinterpret_cast<const uint32_t*>(lds + (((x[c] << 2) & (MASK << 2)) | (hi ? lbh[c] : lbl[c])) +
                                                    toff);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t q = x[c] >> B;
          if (BY == 2 || (BY == 1 && f <= 7)) x[c] = add_byte1(e[c], mul_byte0(e[c], q));
          else x[c] = __umul24(__builtin_amdgcn_ubfe(e[c], 11, fw), q) + (e[c] & 0x7FFu);
          ev[c][f] = e[c];
        }
        if (f == 5) {
          // the words fields 5..8 can read must be staged (rarely not yet)
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const uint32_t P0 = __builtin_amdgcn_readlane(vP[c], 0);
            const uint32_t P1 = __builtin_amdgcn_readlane(vP[c], 32);
            if (F0[c] < min(P0 + kHead1, end0[c]) || F1[c] < min(P1 + kHead1, end1[c]))
              stage(c, kHead1);
          }
        }
        renorm(active);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (BY == 1) {
          // byte entries: the high halves hold fp16(1024 + 2 (z - dmin) + c);
          // pairs of them gathered by one permute and shifted by the fields'
          // constants 2 dmin - 1024 in one packed fp16 add are 2 z + c exactly,
          // and fed as fp16 to the multiply by the row scale.  Bit 17 of an
          // entry (bit 1 of n) is the parity of z - dmin, as bit 23 of a direct
          // entry, so the parity and field 8 follow the direct form.
          const uint32_t p12 = add_f16x2(__builtin_amdgcn_perm(ev[c][2], ev[c][1], 0x07060302u), kb[0]);
          const uint32_t p34 = add_f16x2(__builtin_amdgcn_perm(ev[c][4], ev[c][3], 0x07060302u), kb[1]);
          const uint32_t p56 = add_f16x2(__builtin_amdgcn_perm(ev[c][6], ev[c][5], 0x07060302u), kb[2]);
          const uint32_t p77 = add_f16x2(ev[c][7], kb[3]);
          const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
              __builtin_amdgcn_bitop3_b32(ev[c][1], ev[c][2], ev[c][3], 0x96),
              __builtin_amdgcn_bitop3_b32(ev[c][4], ev[c][5], ev[c][6], 0x96), ev[c][7], 0x96);
          par[c] = __builtin_amdgcn_ubfe(x3, 17, pw);
          const int32_t u8 = __mul24(int32_t(par[c]), m8d) +
                             int32_t(__builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[c][8], 22));
          vv[c][8] = __builtin_bit_cast(float, u8) + k8d;
          // slow rows: the value is halved first (exactly), then multiplied by g
          const float hv = slow_rows ? 0.5f : rv[c];
          yb[c][0] = mul_f16_f32<false>(p12, hv);
          yb[c][1] = mul_f16_f32<true>(p12, hv);
          yb[c][2] = mul_f16_f32<false>(p34, hv);
          yb[c][3] = mul_f16_f32<true>(p34, hv);
          yb[c][4] = mul_f16_f32<false>(p56, hv);
          yb[c][5] = mul_f16_f32<true>(p56, hv);
          yb[c][6] = mul_f16_f32<true>(p77, hv);
          if (slow_rows) {
#pragma unroll
            for (int i = 0; i < 7; ++i) yb[c][i] = __fmul_rn(yb[c][i], rv[c]);
          }
        } else if constexpr (BY == 2) {
          // i16 byte entries: the high half is the value 2 z + c (4 m + c for
          // field 8, or 2 z8 + c), converted by one sign-extending select of
          // the conversion; its bit 1 (bit 17 of the entry) is the parity of z,
          // so the XOR over z1..z7 gives the parity of their sum, and
          // 2 z8 + c = (4 m + c) + 2 par
#pragma unroll
          for (int f = 1; f <= 7; ++f) vv[c][f] = float(int32_t(ev[c][f]) >> 16);
          const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
              __builtin_amdgcn_bitop3_b32(ev[c][1], ev[c][2], ev[c][3], 0x96),
              __builtin_amdgcn_bitop3_b32(ev[c][4], ev[c][5], ev[c][6], 0x96), ev[c][7], 0x96);
          par[c] = __builtin_amdgcn_ubfe(x3, 17, pw);
          vv[c][8] = float((int32_t(ev[c][8]) >> 16) + int32_t(par[c] << 1));
        } else if (kDirectable && direct) {
          // direct entries: 0x4B400000 | (e >> 22) is the float 2^23 + 2^22 +
          // (2 z + c - 2 dmin), and one constant per field (the same for both
          // cosets) turns it into 2 z + c.  Bit 23 of an entry is the parity of
          // z - dmin, so the XOR of z1..z7's entries gives the parity of their
          // sum up to the parity of the minima, which the field-8 constant and
          // multiplier absorb: 2 z8 + c = (4 (m - dmin8) + c) + 2 par + 4 dmin8.
#pragma unroll
          for (int f = 1; f <= 7; ++f)
            vv[c][f] = __builtin_bit_cast(float, __builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[c][f], 22)) +
                       kd[f - 1];
          const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
              __builtin_amdgcn_bitop3_b32(ev[c][1], ev[c][2], ev[c][3], 0x96),
              __builtin_amdgcn_bitop3_b32(ev[c][4], ev[c][5], ev[c][6], 0x96), ev[c][7], 0x96);
          par[c] = __builtin_amdgcn_ubfe(x3, 23, pw);
          const int32_t u8 = __mul24(int32_t(par[c]), m8d) +
                             int32_t(__builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[c][8], 22));
          vv[c][8] = __builtin_bit_cast(float, u8) + k8d;
        } else {
          // value of z_f.  Packed: 0x4B400000 | (e >> 22) is the float
          // 2^23 + 2^22 + 2 s (+1 when f = 2^11), and the per-table constant turns
          // it into 2 z + c.  Wide: the same bits give 2^23 + 2^22 + s, the
          // constant turns it into z, and an exact fma makes 2 z + c.
          const int kaddr = cs[c] ? 4 : 0;
          const float cf = cs[c] ? 1.0f : 0.0f;
#pragma unroll
          for (int f = 1; f <= 7; ++f) {
            const float u = __builtin_bit_cast(float, __builtin_amdgcn_alignbit(0x4B400000u >> 10, ev[c][f], 22));
            const float kf = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(kaddr + 8 * (f - 1), int(kreg)));
            vv[c][f] = kWide ? __builtin_fmaf(u - kf, 2.0f, cf) : u - kf;
          }
          // parity of z1 + ... + z7: bit kSymShift of each entry is the parity of
          // its symbol index, the constant supplies the parity of the minima
          const uint32_t kp = uint32_t(__builtin_amdgcn_ds_bpermute(kaddr + 64, int(kreg)));
          const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
              __builtin_amdgcn_bitop3_b32(ev[c][1], ev[c][2], ev[c][3], 0x96),
              __builtin_amdgcn_bitop3_b32(ev[c][4], ev[c][5], ev[c][6], 0x96), ev[c][7] ^ kp, 0x96);
          par[c] = __builtin_amdgcn_ubfe(x3, kSymShift, pw);
          // z8 = 2 m + parity: 2 z8 + c = 4 s8 + 2 par + (c + 4 min), the
          // parenthesis being part of the per-table constant (a directly coded
          // z8: 2 s8 + (c + 2 min), with the parity field of width 0)
          const uint32_t u8 = ((ev[c][8] >> kSymShift) << sh8) + ((par[c] << 1) | 0x4B400000u);
          const float k8 = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(kaddr + 56, int(kreg)));
          vv[c][8] = __builtin_bit_cast(float, u8) - k8;
        }
      }
    } else if constexpr (SP) {
      // per-slot entries f | (slot - cum) << 7 | parity << 15 and the slot
      // symbol's value 2 z + c (i16), both in LDS (b = 11: 64 KB each)
      static_assert(BT == 11, "per-slot entries are built for b = 11");
      uint32_t ev[CH][9], lbl[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        lbl[c] = cs[c] ? (M << 1) : 0u;                    // byte offset of the coset's map
        asm volatile("" : "+v"(lbl[c]));
      }
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        const uint32_t toff = (uint32_t(2 * (f - 1)) << B) * 2u;       // at most 57344
        uint32_t e[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t a = ((x[c] << 1) & (MASK << 1)) | lbl[c];
          e[c] = *reinterpret_cast<const uint16_t*>(lds + a + toff);
          // the values follow the 16 entry maps (64 KB): a second base register
          const uint32_t av = a | (uint32_t(16) << (B + 1));
          vv[c][f] = float(*reinterpret_cast<const int16_t*>(lds + av + toff));
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t q = x[c] >> B;
          x[c] = __umul24(e[c] & 0x7Fu, q) + __builtin_amdgcn_ubfe(e[c], 7, 7);
          ev[c][f] = e[c];
        }
        if (f == 5) {
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const uint32_t P0 = __builtin_amdgcn_readlane(vP[c], 0);
            const uint32_t P1 = __builtin_amdgcn_readlane(vP[c], 32);
            if (F0[c] < min(P0 + kHead1, end0[c]) || F1[c] < min(P1 + kHead1, end1[c]))
              stage(c, kHead1);
          }
        }
        renorm(active);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
            __builtin_amdgcn_bitop3_b32(ev[c][1], ev[c][2], ev[c][3], 0x96),
            __builtin_amdgcn_bitop3_b32(ev[c][4], ev[c][5], ev[c][6], 0x96), ev[c][7], 0x96);
        par[c] = __builtin_amdgcn_ubfe(x3, 15, pw);
        vv[c][8] = vv[c][8] + float(par[c] << 1);           // the m values are 4 m + c (z8: 2 z8 + c)
      }
    } else {
      uint32_t sv[CH][9], lb[CH], cb[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        lb[c] = cs[c] ? M : 0u;                            // coset offset inside each table pair
        // symbol tables: coset base including the block's own offset, so that
        // the per-field LDS offsets fit the 16-bit immediate
        cb[c] = cs[c] ? lut_bytes + S * 8u : lut_bytes;
        if (TL == kTabNarrow) asm volatile("" : "+v"(cb[c]));
      }
#pragma unroll
      for (int f = 1; f <= 8; ++f) {
        uint32_t e[CH], addr[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          addr[c] = (x[c] & MASK) | lb[c];                 // slot + coset * 2^b
          uint32_t s;
          if (kWs) s = reinterpret_cast<const uint16_t*>(tbase)[(uint32_t(2 * (f - 1)) << B) + addr[c]];
          else if (kHyb) s = reinterpret_cast<const uint16_t*>(lds)[(uint32_t(2 * (f - 1)) << B) + addr[c]];
          else s = lds[(uint32_t(2 * (f - 1)) << B) + addr[c]];
          // the symbol's entry and value in one 8-byte read
          const uint32_t eo = cb[c] + s * 8u + uint32_t(f - 1) * 2u * S * 8u;
          const uint64_t ev2 = *reinterpret_cast<const uint64_t*>(tbase + eo);
          e[c] = uint32_t(ev2);
          vv[c][f] = __uint_as_float(uint32_t(ev2 >> 32));
          sv[c][f] = kGlobalEntries ? s : e[c];
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const uint32_t q = x[c] >> B;
          x[c] = __umul24(e[c] & (kGlobalEntries ? 0xFFFFu : 0x7FFFu), q) + (addr[c] - (e[c] >> 16));
        }
        if (f == 5) {
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const uint32_t P0 = __builtin_amdgcn_readlane(vP[c], 0);
            const uint32_t P1 = __builtin_amdgcn_readlane(vP[c], 32);
            if (F0[c] < min(P0 + kHead1, end0[c]) || F1[c] < min(P1 + kHead1, end1[c]))
              stage(c, kHead1);
          }
        }
        renorm(active);
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t x3 = __builtin_amdgcn_bitop3_b32(
            __builtin_amdgcn_bitop3_b32(sv[c][1], sv[c][2], sv[c][3], 0x96),
            __builtin_amdgcn_bitop3_b32(sv[c][4], sv[c][5], sv[c][6], 0x96), sv[c][7], 0x96);
        // narrow: bit 15 of the symbol entries is the parity of z; workspace:
        // parity of the symbol indices, corrected by the parity of the minima
        par[c] = TL == kTabNarrow ? __builtin_amdgcn_ubfe(x3, 15, pw) : (x3 ^ (kpar >> (cs[c] ? 1 : 0))) & pw;
        vv[c][8] = vv[c][8] + float(par[c] << 1);           // the m table holds 4 m + c (z8: 2 z8 + c)
      }
    }

    // ---- y = (z + c/2) * g, computed as (2 z + c) * (g/2) when g/2 is exact
    // (the row multiplier array then holds g/2; otherwise g and the slow form)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      x[c] = active[c] ? x[c] : x_saved[c];
      const uint32_t ob = active[c] ? (g[c] + k * 32u) * out_vec_bytes(OK) : out_bytes;
      float* v = vv[c];
      if (OK == kOutLattice) {
        const i32x4 lo4 = {int(v[1]), int(v[2]), int(v[3]), int(v[4])};
        const i32x4 hi4 = {int(v[5]), int(v[6]), int(v[7]), int(v[8])};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo4), rO, ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi4), rO, ob + 16u, 0, 0);
      } else {
        // slow rows: rv is g and 2 z + c is halved first (exactly)
        if (slow_rows) {
#pragma unroll
          for (int i = BY == 1 ? 8 : 1; i <= 8; ++i) v[i] = __fmul_rn(v[i], 0.5f);
        }
        float y[8];
        if constexpr (BY == 1) {
#pragma unroll
          for (int i = 0; i < 7; ++i) y[i] = yb[c][i];
          y[7] = __fmul_rn(v[8], rv[c]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = __fmul_rn(v[i + 1], rv[c]);
        }
        if (OK == kOutBF16) {
          const u32x4 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                           pack_bf16x2(y[6], y[7])};
          __builtin_amdgcn_raw_buffer_store_b128(w, rO, ob, 0, 0);
        } else if (OK == kOutFP16) {
          const u32x4 w = {pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]), pack_f16x2(y[4], y[5]),
                           pack_f16x2(y[6], y[7])};
          __builtin_amdgcn_raw_buffer_store_b128(w, rO, ob, 0, 0);
        } else if (OK == kOutFP32) {
          const u32x4 lo = {__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                            __float_as_uint(y[3])};
          const u32x4 hi = {__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                            __float_as_uint(y[7])};
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
      col[c] += 32u;
      if (col[c] >= vpr) {                  // rows of at least 32 vectors wrap at most once
        col[c] -= vpr;
        rowb[c] += 4u;
        while (col[c] >= vpr) {
          col[c] -= vpr;
          rowb[c] += 4u;
        }
      }
    }
  };
  uint32_t k = 0;
  for (; k < kfull; ++k) round(k, std::true_type{});
  for (; k < kmax; ++k) round(k, std::false_type{});

  // ---- end-of-tile invariants: every state back at 2^15, every word consumed
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint64_t bad_state = __builtin_amdgcn_ballot_w64(x[c] != kL);
    const uint64_t bad_len_m = __builtin_amdgcn_ballot_w64(bad_len[c]);
    if (tile_ok[c] && l == 0 && T.status) {
      const uint32_t Pm = vP[c], Em = half ? end1[c] : end0[c];
      const uint32_t sh = half ? 32u : 0u;
      int st = EP_TILE_OK;
      if (uint32_t(bad_len_m >> sh)) st = EP_TILE_BAD_LENGTH;
      else if (Pm > Em) st = EP_TILE_OVERRUN;
      else if (uint32_t(empty_err[c] >> sh)) st = EP_TILE_EMPTY_TABLE;
      else if (uint32_t(bad_state >> sh)) st = EP_TILE_BAD_STATE;
      else if (Pm != Em) st = EP_TILE_BAD_LENGTH;
      ((EP_GLOBAL int32_t*)T.status)[tile0 + 2u * uint32_t(c) + half] = st;
    }
  }
}

// One unit of work: the 2*CH tiles from tile0 with the entry form the build kept.
template <int BT, int TL, int OK, int CH>
__device__ __forceinline__ void decode_group(const DevTensor& T, uint32_t tile0, uint32_t t_end,
                                             const unsigned char* __restrict__ smem,
                                             uint16_t* __restrict__ rings, bool split, uint32_t bmode) {
  constexpr bool kByteOk = (TL == kTabPacked || TL == kTabPackedWide) && OK != kOutLattice;
  if constexpr (has_split(TL, BT)) {
    if (split) decode_tiles<BT, TL, OK, true, CH, 0>(T, tile0, t_end, smem, rings);
    else decode_tiles<BT, TL, OK, false, CH, 0>(T, tile0, t_end, smem, rings);
  } else if constexpr (kByteOk) {
    if (bmode == 2u) decode_tiles<BT, TL, OK, false, CH, 2>(T, tile0, t_end, smem, rings);
    else if (TL == kTabPacked && bmode == 1u)
      decode_tiles<BT, TL, OK, false, CH, (TL == kTabPacked ? 1 : 0)>(T, tile0, t_end, smem, rings);
    else decode_tiles<BT, TL, OK, false, CH, 0>(T, tile0, t_end, smem, rings);
  } else {
    decode_tiles<BT, TL, OK, false, CH, 0>(T, tile0, t_end, smem, rings);
  }
}

// Persistent decode kernel.  Block i owns a contiguous range of chunks (up to
// tiles_per_chunk tiles of one tensor each), which splits into runs of chunks
// from the same tensor.  For each run the block stages the tensor's decode
// tables (LDS layouts); then each wave takes groups of 2 * CH consecutive tiles
// (CH chains of one tile per half-wave) from a counter until the run is
// exhausted.  Taking work dynamically keeps all of a block's waves busy to the
// end: the SIMD's issue arbitration favours older waves, so equal static shares
// finish at very different times.  The counter of a run is the word of `ctr`
// at the run's first chunk (LDS is fully used by the tables and rings); a wave
// claims its next group before decoding the current one, so the atomic's
// latency is hidden.
template <int BT, int TL, int OK, int CH>
__global__ __launch_bounds__(kBlock) void decode_kernel(const DevTensor* __restrict__ tens,
                                                        const Chunk* __restrict__ chunks,
                                                        uint32_t* __restrict__ ctr,
                                                        uint32_t nchunks, uint32_t tiles_per_chunk) {
  constexpr size_t kTab = lds_table_bytes_of(TL, BT);
  constexpr uint32_t kGroup = 2u * CH;                     // tiles per wave group
  __shared__ __align__(16) unsigned char smem[kTab + ring_bytes_of(CH)];
  // an even share of the chunks per block (chunks are one group of tiles, so
  // the blocks' shares differ by at most one group).  Blocks go to the eight
  // XCDs in turn (block b to XCD b mod 8), each with its own L2: the blocks of
  // one XCD take consecutive shares, so that a tensor's tables and the cache
  // lines that neighbouring tiles share are fetched into one L2 rather than
  // into the L2s of every XCD that holds a neighbouring block.
  constexpr uint32_t kXcds = 8;
  const uint32_t nb = gridDim.x, xcd = blockIdx.x % kXcds;
  const uint32_t lblock = xcd * (nb / kXcds) + min(xcd, nb % kXcds) + blockIdx.x / kXcds;
  const uint32_t c0 = uint32_t((uint64_t(lblock) * nchunks) / nb);
  const uint32_t c1 = uint32_t((uint64_t(lblock + 1u) * nchunks) / nb);
  const bool lane0 = (threadIdx.x & 63u) == 0;
  // LDS: [decode tables (LDS layouts)][2 * CH rings of kRingWords per wave]
  uint16_t* rings = reinterpret_cast<uint16_t*>(smem + kTab) + (threadIdx.x >> 6) * (kGroup * kRingWords);
  for (uint32_t ci = c0; ci < c1;) {
    const Chunk ch = chunks[ci];
    const DevTensor& T = tens[ch.tensor];
    // a tensor's chunks are consecutive: the run ends with the tensor or the range
    const uint32_t left = (T.T - ch.tile0 + tiles_per_chunk - 1) / tiles_per_chunk;
    const uint32_t cn = min(c1, ci + left);
    const uint32_t t_end = min(T.T, ch.tile0 + (cn - ci) * tiles_per_chunk);
    const uint32_t ngroups = (t_end - ch.tile0 + kGroup - 1) / kGroup;
    __syncthreads();                       // every wave is done with the previous run
    if (threadIdx.x == 0) __hip_atomic_store(ctr + ci, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // hybrid layout: the per-slot entry maps when the build kept them, else the slot maps
    const bool split = has_split(TL, BT) && T.split != 0 && T.bad_split != T.call;
    // packed layout: the byte entries of fields 1..7 when the build kept them
    // packed and wide layouts: the byte entries when the build kept them
    constexpr bool kByteOk = (TL == kTabPacked || TL == kTabPackedWide) && OK != kOutLattice;
    const uint32_t bmode = kByteOk && T.bytev != 0 && T.bad_bytes != T.call ? T.byte_cand : 0u;
    if (TL != kTabWorkspace) {
      const EP_GLOBAL u32x4* src = (const EP_GLOBAL u32x4*)(T.tab + (split ? split_off_of(BT) : 0));
      u32x4* dst = reinterpret_cast<u32x4*>(smem);
      const uint32_t n16 = uint32_t((has_split(TL, BT) && !split ? lut_bytes_of(TL, BT) : kTab) / 16u);
      if (kByteOk && bmode != 0u) {
        // the byte tables: fields 1..7 (field 8, at the same offset, from the
        // packed ones), or all 16 tables
        const EP_GLOBAL u32x4* srcb = (const EP_GLOBAL u32x4*)(T.tab + byte_off_of(BT));
        const uint32_t nb16 = bmode == 1u ? uint32_t(byte_bytes_of(BT) / 16u) : n16;
        for (uint32_t i = threadIdx.x; i < n16; i += kBlock) dst[i] = i < nb16 ? srcb[i] : src[i];
      } else {
        for (uint32_t i = threadIdx.x; i < n16; i += kBlock) dst[i] = src[i];
      }
    }
    __syncthreads();
    // Units of work: groups of kGroup tiles, except that a run's last partial
    // round is split into tile pairs run as one chain each, so that more waves
    // share it (a run ends at a block barrier, so its last round sets the run's
    // time).  With every table in LDS a round is bound by VALU issue, which the
    // partial round leaves spare: one-chain pairs finish sooner even where some
    // waves take two of them in turn.  Where the tables are read through the
    // caches (hybrid and workspace layouts) a round waits on those reads and a
    // wave's two chains hide each other's waits, so the split is taken only when
    // the pairs need no more than one round (at most half as many groups as the
    // block has waves).  The first unit of each wave is its own index, which
    // spreads a short run over the SIMDs (wave w runs on SIMD w mod 4); later
    // units come from the counter.
    uint32_t u4 = ngroups;
    if constexpr (CH > 1) {
      constexpr bool kLdsTables = storage_of(TL) != kTabWorkspace;
      const uint32_t r = ngroups % uint32_t(kWavesPerBlock);
      if (r != 0u && (kLdsTables || r <= uint32_t(kWavesPerBlock) / 2u)) u4 = ngroups - r;
    }
    const uint32_t t4 = ch.tile0 + kGroup * u4;              // first tile of the pairs
    const uint32_t nunits = u4 + (t_end > t4 ? (t_end - t4 + 1u) / 2u : 0u);
    uint32_t gr = threadIdx.x >> 6, nx = 0;
    while (gr < nunits) {
      if (lane0) nx = kWavesPerBlock + atomicAdd(ctr + ci, 1u);
      if (CH == 1 || gr < u4) decode_group<BT, TL, OK, CH>(T, ch.tile0 + kGroup * gr, t_end, smem, rings, split, bmode);
      else decode_group<BT, TL, OK, 1>(T, t4 + 2u * (gr - u4), t_end, smem, rings, split, bmode);
      gr = __builtin_amdgcn_readfirstlane(nx);
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
  if (d.prob_bits <= 11 && amax <= 512 && table_bytes_of(kTabPacked, d.prob_bits) + kRingBytesMax <= kMaxLds)
    return kVarP9 + (d.prob_bits - 9);
  // the wide entry holds f in 11 bits: every f < 2^11 (no one-symbol table at b = 11)
  if ((d.prob_bits == 10 || d.prob_bits == 11) && amax <= 1024 && !(d.prob_bits == 11 && single) &&
      table_bytes_of(kTabPackedWide, d.prob_bits) + kRingBytesMax <= kMaxLds)
    return kVarW10 + (d.prob_bits - 10);
  if (d.prob_bits == 12 && amax <= 256 && table_bytes_of(kTabNarrow, 12) + kRingBytesMax <= kMaxLds)
    return kVarN12;
  if ((d.prob_bits == 11 || d.prob_bits == 12) && lds_table_bytes_of(kTabHybrid, d.prob_bits) + kRingBytesMax <= kMaxLds)
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
  std::vector<char> byte_cand;
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

// Direct entries (packed layout): each field's values over both cosets must fit
// the entry's 10 top bits as 2 (z - dmin) + c (4 (m - dmin) + c for field 8), and
// no table may be a one-symbol table at b = 11 (f = 2^11).  Fills dmin[1..8]
// with each field's smaller minimum over the two cosets.
bool direct_minima(const ep_tensor_desc& d, uint32_t variant, int32_t dmin[9]) {
  bool direct = layout_of(variant) == kTabPacked;
  const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
  dmin[0] = 0;
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
    dmin[f] = int32_t(mn);
  }
  return direct;
}

// Byte entries for fields 1..7 (the table build still checks every f < 256):
// direct entries, with every field's smaller minimum within +-512, so that the
// fp16 constants 2 dmin - 1024, the values 1024 + n and 2 z + c are all exact.
bool byte_candidate(const ep_tensor_desc& d, uint32_t variant) {
  int32_t dmin[9];
  if (!direct_minima(d, variant, dmin)) return false;
  for (int f = 1; f <= 7; ++f)
    if (dmin[f] < -512 || dmin[f] > 512) return false;
  return true;
}

// Which byte entries a tensor gets (the table build still checks every f < 256
// of the tables it writes and drops them otherwise): 1 (fields 1..7, fp16 form)
// for the candidates above; 2 (all 16 tables, i16 form) for any other packed or
// wide tensor whose values 2 z + c and 4 m + c (2 z8 + c) all fit 16 bits.
uint32_t byte_mode(const ep_tensor_desc& d, uint32_t variant) {
  if (byte_candidate(d, variant)) return 1;
  const int tl = layout_of(variant);
  if (tl != kTabPacked && tl != kTabPackedWide) return 0;
  const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
  for (int k = 1; k < kTables; ++k) {
    if (d.alphabet[k] == 0) continue;
    const int64_t mul = k >= 15 ? k8 : 2, c = (k - 1) & 1;
    const int64_t lo = mul * int64_t(d.min_offset[k]) + c;
    const int64_t hi = mul * (int64_t(d.min_offset[k]) + d.alphabet[k] - 1) + c;
    if (lo < -32768 || hi > 32767) return 0;
  }
  return 2;
}

// IEEE binary16 bits of an integer v, |v| <= 2048 (exactly representable)
uint32_t f16_bits_of_int(int32_t v) {
  if (v == 0) return 0;
  const uint32_t s = v < 0 ? 0x8000u : 0u;
  const uint32_t a = uint32_t(v < 0 ? -v : v);
  const int e = 31 - __builtin_clz(a);                        // a in [2^e, 2^(e+1)), e <= 11
  const uint32_t m = (e <= 10 ? (a << (10 - e)) : (a >> (e - 10))) & 0x3FFu;
  return s | (uint32_t(e + 15) << 10) | m;
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
  L.byte_cand.resize(n);
  for (uint32_t v = 0; v < kNumGroups; ++v) L.group_tiles[v] = 0;
  bool has_wide[2] = {false, false};               // a tensor of the batch needs the wide layout at b = 10, 11
  for (int i = 0; i < n; ++i) {
    int rc = validate(descs[i], i);
    if (rc != EP_OK) return rc;
    L.variant[i] = choose_variant(descs[i]);
    if (L.variant[i] == kVarW10 || L.variant[i] == kVarW11) has_wide[L.variant[i] - kVarW10] = true;
  }
  // Each layout is a launch of its own, and a launch ends with a partial last
  // round.  Where a batch holds wide tensors, its packed tensors of the same b
  // that the wide entries can hold (no one-symbol table at b = 11) join the wide
  // launch: one launch and one tail instead of two.  The choice depends on the
  // descriptors only, so the workspace size is the same with and without dtypes.
  for (int i = 0; i < n; ++i) {
    const ep_tensor_desc& d = descs[i];
    if ((L.variant[i] == kVarP10 || L.variant[i] == kVarP11) && has_wide[L.variant[i] - kVarP10]) {
      bool single = false;
      for (int k = 1; k < kTables; ++k) single |= d.alphabet[k] == 1;
      if (!(d.prob_bits == 11 && single)) L.variant[i] = kVarW10 + (L.variant[i] - kVarP10);
    }
  }
  for (int i = 0; i < n; ++i) {
    const ep_tensor_desc& d = descs[i];
    const int ok = dtypes ? out_kind_of(dtypes[i]) : kOutBF16;
    if (ok < 0) return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": unknown output dtype");
    L.group[i] = L.variant[i] * kNumOutKinds + uint32_t(ok);
    L.tab_bytes[i] = storage_bytes_of(layout_of(L.variant[i]), d.prob_bits);
    L.byte_cand[i] = char(byte_mode(d, L.variant[i]));
    if (L.byte_cand[i] == 1) L.tab_bytes[i] += byte_bytes_of(d.prob_bits);
    if (L.byte_cand[i] == 2) L.tab_bytes[i] += byte16_bytes_of(d.prob_bits);
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
  uint32_t chunk_begin, nchunks, grid, tiles_per_chunk, chains;
};

struct PlanImpl {
  void* ws;
  uint64_t magic;
  uint64_t ntensors;
  uint64_t ctr_off;                   // workspace offset of the per-chunk work counters
  Group groups[kNumGroups];
};
static_assert(sizeof(PlanImpl) <= sizeof(ep_batch_plan), "plan record too large");
constexpr uint64_t kPlanMagic = 0x45504c414e763037ull;

using KernelFn = void (*)(const DevTensor*, const Chunk*, uint32_t*, uint32_t, uint32_t);

template <int BT, int TL, int CH>
KernelFn kernel_for_kind(int ok) {
  switch (ok) {
    case kOutBF16: return decode_kernel<BT, TL, kOutBF16, CH>;
    case kOutFP8: return decode_kernel<BT, TL, kOutFP8, CH>;
    case kOutINT8: return decode_kernel<BT, TL, kOutINT8, CH>;
    case kOutFP16: return decode_kernel<BT, TL, kOutFP16, CH>;
    case kOutFP32: return decode_kernel<BT, TL, kOutFP32, CH>;
    case kOutUINT8: return decode_kernel<BT, TL, kOutUINT8, CH>;
    default: return decode_kernel<BT, TL, kOutLattice, CH>;
  }
}

template <int CH>
KernelFn kernel_of_chains(uint32_t group) {
  const int ok = int(group % kNumOutKinds);
  switch (group / kNumOutKinds) {
    case kVarP9: return kernel_for_kind<9, kTabPacked, CH>(ok);
    case kVarP10: return kernel_for_kind<10, kTabPacked, CH>(ok);
    case kVarP11: return kernel_for_kind<11, kTabPacked, CH>(ok);
    case kVarW10: return kernel_for_kind<10, kTabPackedWide, CH>(ok);
    case kVarW11: return kernel_for_kind<11, kTabPackedWide, CH>(ok);
    case kVarN12: return kernel_for_kind<12, kTabNarrow, CH>(ok);
    case kVarH11: return kernel_for_kind<11, kTabHybrid, CH>(ok);
    case kVarH12: return kernel_for_kind<12, kTabHybrid, CH>(ok);
    default: return kernel_for_kind<0, kTabWorkspace, CH>(ok);
  }
}

KernelFn kernel_of(uint32_t group, uint32_t chains) {
  return chains == 2 ? kernel_of_chains<2>(group) : kernel_of_chains<1>(group);
}

// Persistent grid: as many blocks as can be resident at once (at least one).
int resident_grid(uint32_t group, uint32_t chains, uint32_t* grid) {
  static int cus = 0;
  hipError_t e;
  if (cus == 0) {
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("device query: ") + hipGetErrorString(e));
  }
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel_of(group, chains)),
                                                   kBlock, 0);
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("occupancy query: ") + hipGetErrorString(e));
  const uint64_t g = uint64_t(std::max(per_cu, 1)) * uint64_t(std::max(cus, 1));
  *grid = uint32_t(std::max<uint64_t>(1, std::min<uint64_t>(g, 1u << 20)));
  return EP_OK;
}

// Chains per wave: two tile pairs decoded together hide more of the per-symbol
// latency, but need four tiles per wave; a batch too small to give every
// resident wave several groups of four runs one pair per wave.
uint32_t chains_for(size_t tiles, uint32_t resident) {
  return tiles >= size_t(4) * 2 * kMaxChains * kWavesPerBlock * resident ? 2u : 1u;
}

// Tiles per chunk: one group (2 * chains tiles, the unit a wave decodes), so
// that the blocks' even shares of the chunks differ by at most one group.  A
// block's consecutive chunks of one tensor form one run; a small batch spreads
// over every resident block.
uint32_t tiles_per_chunk(uint32_t chains) { return 2u * chains; }

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

  // only the descriptors travel (for small batches as the table build's kernel
  // arguments); the build kernel writes the tile schedule
  std::vector<unsigned char> host(L.chunk_off, 0);
  const uint32_t call = next_call_number();
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
    G.chains = 1;
    G.tiles_per_chunk = 2u * kWavesPerBlock;
    if (L.group_tiles[v] == 0) continue;
    uint32_t resident = 0;
    rc = resident_grid(v, kMaxChains, &resident);
    if (rc != EP_OK) return rc;
    G.chains = chains_for(L.group_tiles[v], resident);
    if (G.chains != kMaxChains) {
      rc = resident_grid(v, G.chains, &resident);
      if (rc != EP_OK) return rc;
    }
    G.tiles_per_chunk = tiles_per_chunk(G.chains);
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
    D.call = call;
    D.bad_split = D.bad_bytes = D.bad_rows = 0;
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
    // direct entries (packed layout): uniform value constants per field
    {
      const bool direct = direct_minima(d, L.variant[i], D.dmin);
      const int64_t k8 = d.field8 == EP_FIELD8_Z8 ? 2 : 4;
      int64_t dsum = 0;
      for (int f = 1; f <= 7; ++f) {
        dsum += D.dmin[f];
        const float kf = -float(12582912 - 2 * int64_t(D.dmin[f]));
        std::memcpy(&D.kvals[18 + f - 1], &kf, 4);
      }
      // field 8: 2 z8 + c = v8 + k8 dmin8 + 2 par (coded m), par = p ^ parity(sum of dmin1..7)
      const int64_t kd8 = (d.field8 == EP_FIELD8_Z8) ? 0 : (dsum & 1);
      const float k8f = -float(12582912 - k8 * D.dmin[8] - 2 * kd8);
      std::memcpy(&D.kvals[25], &k8f, 4);
      D.kvals[26] = uint32_t(d.field8 == EP_FIELD8_Z8 ? 0 : (kd8 ? -2 : 2));
      D.direct = direct ? 1u : 0u;
      // byte entries: the fp16 constants 2 dmin_f - 1024 of fields 1..7, in pairs
      D.byte_cand = uint32_t(L.byte_cand[i]);
      D.bytev = D.byte_cand != 0u ? 1u : 0u;
      uint32_t kh[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (D.byte_cand == 1u)
        for (int f = 1; f <= 7; ++f) kh[f] = f16_bits_of_int(2 * D.dmin[f] - 1024);   // in [-2048, 0]
      D.kbyte[0] = kh[1] | (kh[2] << 16);
      D.kbyte[1] = kh[3] | (kh[4] << 16);
      D.kbyte[2] = kh[5] | (kh[6] << 16);
      D.kbyte[3] = kh[7] << 16;
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
  hipError_t e = hipSuccess;
  const bool by_args = n <= kArgTensors;
  if (n > 0 && !by_args) {
    e = hipMemcpyAsync(wsb, host.data(), host.size(), hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
  }
  if (n > 0) {
    uint64_t max_rows = 1;
    for (int i = 0; i < n; ++i) max_rows = std::max<uint64_t>(max_rows, uint64_t(descs[i].rows));
    const uint32_t row_blocks = uint32_t((max_rows + 1023) / 1024);
    size_t lds_bytes = 16;
    for (int i = 0; i < n; ++i) {
      if (descs[i].num_tiles == 0) continue;
      uint32_t amax = 0;
      for (int k = 1; k < kTables; ++k) amax = std::max(amax, descs[i].alphabet[k]);
      lds_bytes = std::max(lds_bytes, build_lds_bytes(is_packed(layout_of(L.variant[i])), descs[i].prob_bits, amax));
    }
    DevTensor* tens = reinterpret_cast<DevTensor*>(wsb + L.tens_off);
    Chunk* chunks = reinterpret_cast<Chunk*>(wsb + L.chunk_off);
    if (by_args) {
      DescArgs<kArgTensors> a;
      std::memset(&a, 0, sizeof(a));
      std::memcpy(a.t, ht, sizeof(DevTensor) * size_t(n));
      hipLaunchKernelGGL(build_tables_kernel<kArgTensors>, dim3(16 + row_blocks + chunk_blocks + 1, n), dim3(256),
                         uint32_t(lds_bytes), st, tens, chunks, row_blocks, a);
    } else {
      hipLaunchKernelGGL(build_tables_kernel<0>, dim3(16 + row_blocks + chunk_blocks, n), dim3(256),
                         uint32_t(lds_bytes), st, tens, chunks, row_blocks, DescArgs<0>{});
    }
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
    hipLaunchKernelGGL(kernel_of(v, G.chains), dim3(G.grid), dim3(kBlock), 0, static_cast<hipStream_t>(stream), tens,
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

// ---------------------------------------------------------------- static scratch
// The workspace of ep_decode_batch_noalloc: a device array the code object's
// loader places on every GPU the library runs on, so the call allocates
// nothing.  In host code `scratch` only names the array; its device address on
// the current GPU comes from hipGetSymbolAddress, looked up once per device.
static_assert(EP_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(EP_ERR_UNSUPPORTED, "device index " + std::to_string(dev) + " beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0)
      return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) gave a NULL or misaligned address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return EP_OK;
}
}  // namespace

int ep_decode_batch_noalloc(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                            int32_t* const* tile_status, int n, void* stream) {
  if (n > 0 && (!dtypes || !outs)) return fail(EP_ERR_INVALID_ARG, "NULL dtypes or outs");
  Layout L;
  int rc = make_layout(descs, dtypes, n, L);
  if (rc != EP_OK) return rc;
  if (L.total > size_t(EP_NOALLOC_SCRATCH_BYTES))
    return fail(EP_ERR_WORKSPACE, "batch needs " + std::to_string(L.total) + " bytes of workspace; the static "
                "scratch holds " + std::to_string(size_t(EP_NOALLOC_SCRATCH_BYTES)) +
                " (split the batch, or call ep_decode_batch with a workspace)");
  void* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != EP_OK) return rc;
  return ep_decode_batch(descs, dtypes, outs, tile_status, n, ws, size_t(EP_NOALLOC_SCRATCH_BYTES), stream);
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
