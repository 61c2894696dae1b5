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
// one state per lane).  Renormalisation reads of a half-wave are located with
// a wave ballot and per-half popcounts, so the lanes that need a word read
// consecutive payload words.  Each lane reconstructs whole 8-wide vectors and
// writes them with one 16-byte (BF16) or 8-byte (FP8/INT8) store; the 32 lanes
// of a half write 512 (256) contiguous bytes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "entropack.h"

namespace {

constexpr uint32_t kL = 1u << 15;          // lower bound of the state interval
constexpr int kTables = EP_NUM_TABLES;
constexpr int kTilesPerWave = 2;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;
constexpr int kTilesPerChunk = kTilesPerWave * kWavesPerBlock;

// Device-side view of one tensor (lives in the workspace).
struct alignas(16) DevTensor {
  uint64_t nvec;             // rows * cols / 8
  uint32_t vpr;              // vectors per row = cols / 8
  uint32_t V, T, b;
  float scale;
  uint32_t empty_mask;       // bit k: table k is empty
  int32_t dtype;
  const float* row_scales;
  const uint32_t* states;
  const uint32_t* offsets;
  const uint16_t* payload;
  uint64_t payload_words;
  const uint16_t* freqs;
  uint16_t* lut;             // [16][2^b] slot -> zero-based symbol (workspace)
  uint32_t* symtab;          // per coordinate table: f | cum << 16 (workspace)
  void* out;
  int32_t* status;
  uint32_t sym_base[kTables];
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
// scan, then the slot -> symbol table by a binary search per slot.
__global__ __launch_bounds__(256) void build_tables_kernel(const DevTensor* __restrict__ tens) {
  const DevTensor& T = tens[blockIdx.y];
  const int k = 1 + blockIdx.x;
  const uint32_t A = T.alphabet[k];
  const uint32_t M = 1u << T.b;
  uint16_t* lut = T.lut + (size_t(k - 1) << T.b);
  uint32_t* sym = T.symtab + T.sym_base[k];
  __shared__ uint32_t scan[256];
  __shared__ uint32_t carry;
  if (A == 0) {
    for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) lut[j] = 0;
    if (threadIdx.x == 0) sym[0] = M & 0xFFFFu;   // never used: the decoder flags the tile
    return;
  }
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const uint16_t* fr = T.freqs + T.freq_base[k];
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
    if (i < A) sym[i] = (f & 0xFFFFu) | (cum << 16);
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) carry += scan[threadIdx.x];
    __syncthreads();
  }
  // slot j -> largest i with cum_i <= j (a zero-frequency symbol is never chosen)
  for (uint32_t j = threadIdx.x; j < M; j += blockDim.x) {
    uint32_t lo = 0, hi = A;
    while (hi - lo > 1) {
      uint32_t mid = (lo + hi) >> 1;
      if ((sym[mid] >> 16) <= j) lo = mid;
      else hi = mid;
    }
    lut[j] = uint16_t(lo);
  }
}

// ---------------------------------------------------------------- container rounding
__device__ __forceinline__ uint32_t bf16_rne(float y) {
  uint32_t u = __float_as_uint(y);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP e4m3fn: clamp to +-448, then round to nearest even at the format's quantum.
__device__ __forceinline__ uint32_t fp8_e4m3_rne(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  float a = fminf(fabsf(y), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                        // below 2^-6: subnormal quantum 2^-9
    code = uint32_t(__builtin_rintf(a * 512.0f));
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);         // keep 3 mantissa bits, ties to even
    code = (u >> 20) - (120u << 3);           // rebias the exponent from 127 to 7
  }
  return sign | code;
}

__device__ __forceinline__ uint32_t int8_rne(float y) {
  float r = __builtin_rintf(y);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return uint32_t(int32_t(r)) & 0xFFu;
}

// ---------------------------------------------------------------- decode
__device__ __forceinline__ uint32_t half_bits(uint64_t bal, int half) {
  return half ? uint32_t(bal >> 32) : uint32_t(bal);
}

__global__ __launch_bounds__(kBlock) void decode_kernel(const DevTensor* __restrict__ tens,
                                                        const Chunk* __restrict__ chunks) {
  const Chunk ch = chunks[blockIdx.x];
  const DevTensor& T = tens[ch.tensor];
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const uint32_t l = lane & 31;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t t = ch.tile0 + wave * kTilesPerWave + half;
  const bool tile_ok = t < T.T;

  const uint32_t b = T.b;
  const uint32_t M = 1u << b;
  const uint32_t mask = M - 1u;
  const uint32_t f0 = T.freqs[T.freq_base[0]];   // table 0: frequency of c = 0
  const uint32_t V = T.V;

  uint32_t n = 0, x = kL, p = 0, pend = 0;
  int err = 0;
  if (tile_ok) {
    const uint64_t first = uint64_t(t) * V;
    n = uint32_t(min(uint64_t(V), T.nvec - first));
    x = T.states[size_t(t) * EP_LANES + l];
    p = T.offsets[t];
    pend = T.offsets[t + 1];
    if (pend < p || pend > T.payload_words) {
      err = EP_TILE_BAD_LENGTH;
      n = 0;
    }
  }
  const uint32_t nk = (n + 31u) >> 5;
  const uint32_t kmax = max(__shfl(nk, 0), __shfl(nk, 32));

  // position of this lane's first vector: row and vector-in-row
  uint64_t g = uint64_t(t) * V + l;
  uint32_t row = 0, col = 0;
  if (tile_ok) {
    row = uint32_t(g / T.vpr);
    col = uint32_t(g - uint64_t(row) * T.vpr);
  }

  for (uint32_t k = 0; k < kmax; ++k) {
    const bool active = (k * 32u + l) < n;

    // field 0: coset bit c (two-symbol table, resolved by one compare)
    uint32_t slot = x & mask;
    const uint32_t c = slot >= f0 ? 1u : 0u;
    if (active) x = (c ? (M - f0) : f0) * (x >> b) + slot - (c ? f0 : 0u);
    {
      const bool need = active && x < kL;
      const uint32_t hb = half_bits(__ballot(need), half);
      if (need) {
        const uint32_t idx = p + __popc(hb & ((1u << l) - 1u));
        if (idx < pend) x = (x << 16) | T.payload[idx];
        else err = EP_TILE_OVERRUN;
      }
      p += __popc(hb);
    }
    if (active && ((T.empty_mask >> (1u + c)) & 1u)) err = EP_TILE_EMPTY_TABLE;

    int32_t val[9];
#pragma unroll
    for (int f = 1; f <= 8; ++f) {
      const int k0 = 1 + 2 * (f - 1);
      const uint32_t sbase = c ? T.sym_base[k0 + 1] : T.sym_base[k0];
      const int32_t mn = c ? T.minv[k0 + 1] : T.minv[k0];
      const uint16_t* lut = T.lut + (size_t(k0 - 1 + c) << b);
      slot = x & mask;
      const uint32_t s = lut[slot];
      const uint32_t e = T.symtab[sbase + s];
      if (active) x = (e & 0xFFFFu) * (x >> b) + slot - (e >> 16);
      val[f] = int32_t(s) + mn;
      const bool need = active && x < kL;
      const uint32_t hb = half_bits(__ballot(need), half);
      if (need) {
        const uint32_t idx = p + __popc(hb & ((1u << l) - 1u));
        if (idx < pend) x = (x << 16) | T.payload[idx];
        else err = EP_TILE_OVERRUN;
      }
      p += __popc(hb);
    }

    if (active) {
      // algebraic inverse: z8 = 2m + parity(z1..z7), x_i = z_i + c/2
      int32_t s7 = 0;
#pragma unroll
      for (int i = 1; i <= 7; ++i) s7 += val[i];
      int32_t z[8];
#pragma unroll
      for (int i = 0; i < 7; ++i) z[i] = val[i + 1];
      z[7] = 2 * val[8] + (s7 & 1);
      const uint64_t gv = g + uint64_t(k) * 32u;
      if (T.dtype == EP_OUT_LATTICE2X_I32) {
        int4* o = reinterpret_cast<int4*>(T.out) + 2 * gv;
        o[0] = make_int4(2 * z[0] + int(c), 2 * z[1] + int(c), 2 * z[2] + int(c), 2 * z[3] + int(c));
        o[1] = make_int4(2 * z[4] + int(c), 2 * z[5] + int(c), 2 * z[6] + int(c), 2 * z[7] + int(c));
      } else {
        const float gs = __fmul_rn(T.scale, T.row_scales[row]);
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xi = __fmul_rn(float(2 * z[i] + int(c)), 0.5f);   // exact half-integer
          y[i] = __fmul_rn(xi, gs);
        }
        if (T.dtype == EP_OUT_BF16) {
          uint4 w;
          w.x = bf16_rne(y[0]) | (bf16_rne(y[1]) << 16);
          w.y = bf16_rne(y[2]) | (bf16_rne(y[3]) << 16);
          w.z = bf16_rne(y[4]) | (bf16_rne(y[5]) << 16);
          w.w = bf16_rne(y[6]) | (bf16_rne(y[7]) << 16);
          reinterpret_cast<uint4*>(T.out)[gv] = w;
        } else if (T.dtype == EP_OUT_FP8_E4M3) {
          uint2 w;
          w.x = fp8_e4m3_rne(y[0]) | (fp8_e4m3_rne(y[1]) << 8) | (fp8_e4m3_rne(y[2]) << 16) |
                (fp8_e4m3_rne(y[3]) << 24);
          w.y = fp8_e4m3_rne(y[4]) | (fp8_e4m3_rne(y[5]) << 8) | (fp8_e4m3_rne(y[6]) << 16) |
                (fp8_e4m3_rne(y[7]) << 24);
          reinterpret_cast<uint2*>(T.out)[gv] = w;
        } else {
          uint2 w;
          w.x = int8_rne(y[0]) | (int8_rne(y[1]) << 8) | (int8_rne(y[2]) << 16) | (int8_rne(y[3]) << 24);
          w.y = int8_rne(y[4]) | (int8_rne(y[5]) << 8) | (int8_rne(y[6]) << 16) | (int8_rne(y[7]) << 24);
          reinterpret_cast<uint2*>(T.out)[gv] = w;
        }
      }
    }
    // advance this lane's vector by 32 positions
    col += 32u;
    while (col >= T.vpr && T.vpr) {
      col -= T.vpr;
      ++row;
    }
  }

  // end-of-tile invariants: every state back at 2^15 and every word consumed
  const uint32_t ov = half_bits(__ballot(err == EP_TILE_OVERRUN), half);
  const uint32_t et = half_bits(__ballot(err == EP_TILE_EMPTY_TABLE), half);
  const uint32_t bl = half_bits(__ballot(err == EP_TILE_BAD_LENGTH), half);
  const uint32_t bs = half_bits(__ballot(x != kL), half);
  if (tile_ok && l == 0 && T.status) {
    int st = EP_TILE_OK;
    if (ov) st = EP_TILE_OVERRUN;
    else if (et) st = EP_TILE_EMPTY_TABLE;
    else if (bl) st = EP_TILE_BAD_LENGTH;
    else if (bs) st = EP_TILE_BAD_STATE;
    else if (p != pend) st = EP_TILE_BAD_LENGTH;
    T.status[t] = st;
  }
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t tens_off, chunk_off, total;
  std::vector<size_t> lut_off, sym_off;
  std::vector<uint32_t> sym_count;
  size_t nchunks;
};

int validate(const ep_tensor_desc& d, int i) {
  auto bad = [&](const char* what) {
    return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": " + what);
  };
  if (d.rows < 0) return bad("rows < 0");
  if (d.cols <= 0 || d.cols % 8 != 0) return bad("cols must be a positive multiple of 8");
  if (d.vectors_per_tile < 32) return bad("vectors_per_tile < 32");
  if (d.prob_bits < 9 || d.prob_bits > 15) return bad("prob_bits outside [9, 15]");
  const unsigned __int128 nvec = (unsigned __int128)(uint64_t)d.rows * (uint64_t)d.cols / 8u;
  if (nvec >= ((unsigned __int128)1 << 32)) return bad("rows*cols/8 must be < 2^32");
  const uint64_t nv = uint64_t(nvec);
  const uint64_t T = (nv + d.vectors_per_tile - 1) / d.vectors_per_tile;
  if (T != d.num_tiles) return bad("num_tiles != ceil(rows*cols/8 / vectors_per_tile)");
  if (d.alphabet[0] != 2 || d.min_offset[0] != 0) return bad("table 0 must be the coset bit (alphabet 2, min 0)");
  for (int k = 1; k < kTables; ++k)
    if (d.alphabet[k] > (1u << d.prob_bits)) return bad("alphabet exceeds 2^prob_bits");
  if (d.num_tiles > 0) {
    if (!d.row_scales || !d.tile_states || !d.tile_offsets || !d.payload || !d.freqs)
      return bad("NULL device pointer");
  }
  return EP_OK;
}

int make_layout(const ep_tensor_desc* descs, int n, Layout& L) {
  if (n < 0 || (n > 0 && !descs)) return fail(EP_ERR_INVALID_ARG, "bad tensor count or NULL descriptors");
  size_t off = 0;
  L.tens_off = off;
  off = align256(off + sizeof(DevTensor) * size_t(n));
  L.nchunks = 0;
  for (int i = 0; i < n; ++i) {
    int rc = validate(descs[i], i);
    if (rc != EP_OK) return rc;
    L.nchunks += (descs[i].num_tiles + kTilesPerChunk - 1) / kTilesPerChunk;
  }
  if (L.nchunks >= (size_t(1) << 31)) return fail(EP_ERR_UNSUPPORTED, "too many tiles in one call");
  L.chunk_off = off;
  off = align256(off + sizeof(Chunk) * L.nchunks);
  L.lut_off.resize(n);
  L.sym_off.resize(n);
  L.sym_count.resize(n);
  for (int i = 0; i < n; ++i) {
    const ep_tensor_desc& d = descs[i];
    L.lut_off[i] = off;
    off = align256(off + sizeof(uint16_t) * (size_t(16) << d.prob_bits));
    uint32_t cnt = 0;
    for (int k = 1; k < kTables; ++k) cnt += std::max<uint32_t>(d.alphabet[k], 1u);
    L.sym_count[i] = cnt;
    L.sym_off[i] = off;
    off = align256(off + sizeof(uint32_t) * cnt);
  }
  L.total = std::max<size_t>(off, 256);
  return EP_OK;
}

struct PlanImpl {
  void* ws;
  uint64_t nchunks;
  uint64_t ntensors;
  uint64_t magic;
};
static_assert(sizeof(PlanImpl) <= sizeof(ep_batch_plan), "plan record too large");
constexpr uint64_t kPlanMagic = 0x45504c414e763031ull;

}  // namespace

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
  int rc = make_layout(descs, n, L);
  if (rc != EP_OK) return rc;
  *bytes = L.total;
  return EP_OK;
}

int ep_batch_prepare(const ep_tensor_desc* descs, const int* dtypes, void* const* outs,
                     int32_t* const* tile_status, int n, void* workspace, size_t ws_bytes,
                     void* stream, ep_batch_plan* plan) {
  if (!plan) return fail(EP_ERR_INVALID_ARG, "plan is NULL");
  std::memset(plan, 0, sizeof(*plan));
  Layout L;
  int rc = make_layout(descs, n, L);
  if (rc != EP_OK) return rc;
  if (n > 0 && (!dtypes || !outs)) return fail(EP_ERR_INVALID_ARG, "NULL dtypes or outs");
  if (!workspace || ws_bytes < L.total)
    return fail(EP_ERR_WORKSPACE, "workspace smaller than ep_workspace_size()");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(EP_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  std::vector<unsigned char> host(L.lut_off.empty() ? L.total : L.lut_off[0], 0);
  DevTensor* ht = reinterpret_cast<DevTensor*>(host.data() + L.tens_off);
  Chunk* hc = reinterpret_cast<Chunk*>(host.data() + L.chunk_off);
  char* wsb = static_cast<char*>(workspace);
  size_t ci = 0;
  for (int i = 0; i < n; ++i) {
    const ep_tensor_desc& d = descs[i];
    const int dt = dtypes[i];
    if (dt != EP_OUT_BF16 && dt != EP_OUT_FP8_E4M3 && dt != EP_OUT_INT8 && dt != EP_OUT_LATTICE2X_I32)
      return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": unknown output dtype");
    const size_t align = dt == EP_OUT_BF16 || dt == EP_OUT_LATTICE2X_I32 ? 16 : 8;
    if (d.num_tiles > 0 && (!outs[i] || reinterpret_cast<uintptr_t>(outs[i]) % align != 0))
      return fail(EP_ERR_INVALID_ARG, "tensor " + std::to_string(i) + ": output NULL or misaligned");
    DevTensor& D = ht[i];
    D.nvec = uint64_t(d.rows) * uint64_t(d.cols) / 8u;
    D.vpr = uint32_t(d.cols / 8);
    D.V = d.vectors_per_tile;
    D.T = d.num_tiles;
    D.b = d.prob_bits;
    D.scale = d.scale;
    D.dtype = dt;
    D.row_scales = d.row_scales;
    D.states = d.tile_states;
    D.offsets = d.tile_offsets;
    D.payload = d.payload;
    D.payload_words = d.payload_words;
    D.freqs = d.freqs;
    D.lut = reinterpret_cast<uint16_t*>(wsb + L.lut_off[i]);
    D.symtab = reinterpret_cast<uint32_t*>(wsb + L.sym_off[i]);
    D.out = outs[i];
    D.status = tile_status ? tile_status[i] : nullptr;
    uint32_t sb = 0, em = 0;
    for (int k = 0; k < kTables; ++k) {
      D.alphabet[k] = d.alphabet[k];
      D.freq_base[k] = d.freq_base[k];
      D.minv[k] = d.min_offset[k];
      if (k == 0) {
        D.sym_base[k] = 0;
        continue;
      }
      D.sym_base[k] = sb;
      sb += std::max<uint32_t>(d.alphabet[k], 1u);
      if (d.alphabet[k] == 0) em |= 1u << k;
    }
    D.empty_mask = em;
    for (uint32_t t0 = 0; t0 < d.num_tiles; t0 += kTilesPerChunk) hc[ci++] = Chunk{uint32_t(i), t0};
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(wsb, host.data(), host.size(), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
  if (n > 0) {
    hipLaunchKernelGGL(build_tables_kernel, dim3(16, n), dim3(256), 0, st,
                       reinterpret_cast<const DevTensor*>(wsb + L.tens_off));
    e = hipGetLastError();
    if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("table build launch: ") + hipGetErrorString(e));
  }
  PlanImpl* P = reinterpret_cast<PlanImpl*>(plan);
  P->ws = workspace;
  P->nchunks = L.nchunks;
  P->ntensors = uint64_t(n);
  P->magic = kPlanMagic;
  (void)ws_bytes;
  return EP_OK;
}

int ep_batch_launch(const ep_batch_plan* plan, void* stream) {
  if (!plan) return fail(EP_ERR_INVALID_ARG, "plan is NULL");
  const PlanImpl* P = reinterpret_cast<const PlanImpl*>(plan);
  if (P->magic != kPlanMagic) return fail(EP_ERR_INVALID_ARG, "plan was not filled by ep_batch_prepare");
  if (P->nchunks == 0) return EP_OK;
  char* wsb = static_cast<char*>(P->ws);
  const size_t chunk_off = align256(sizeof(DevTensor) * size_t(P->ntensors));
  hipLaunchKernelGGL(decode_kernel, dim3(uint32_t(P->nchunks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const DevTensor*>(wsb),
                     reinterpret_cast<const Chunk*>(wsb + chunk_off));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(EP_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
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

}  // extern "C"
