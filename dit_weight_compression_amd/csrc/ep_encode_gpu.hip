// EntroPack compressor on the MI355X (gfx950).
//
// Produces the same container as the host compressor (ep_encode.cpp), byte
// for byte, following "EntroPack: Fast and Accurate Entropy-Coded Weight
// Compression at Arbitrary Bitrates": Figure 2(a) and sections 3.1-3.6 (row
// normalisation, nearest-E8 quantisation, parity-reduced fields, 17
// coset-conditioned tables, sampled scale search, least-squares row scales,
// 32-lane interleaved rANS tiles), appendix C.1 (bisection, precision
// escalation, scale coarsening), appendix C.3 (state and word sizes) and
// appendix B.1 (row-scaled FP8 / INT8 pre-cast).
//
// Work split.  Everything that touches every weight runs in kernels: the
// route pre-cast, the per-row sums of squares, the E8 quantisation (with the
// per-table ranges), the symbol histograms, the row-scale refit, the tile
// encoder, the offset scan and the payload compaction.  The host keeps the
// decisions that need only small exact data: the row sample, the square root
// of each row mean, the rate estimate from the exact counts, the bisection,
// the escalation and the frequency normalisation (ep_encode_common.h, shared
// with the host compressor).  Floating-point results match the host because
// every operation is IEEE-754 correctly rounded (fp64 and fp32 division,
// conversions, rint), no multiply-add is contracted (-ffp-contract=off), and
// every order-dependent sum (row sums of squares, refit numerator and
// denominator, the two squared distances of the E8 search) keeps the host's
// sequential order: one lane owns one row or one vector.
//
// Tile encoder mapping: one wave64 encodes two tiles, one per half-wave; lane
// l of a half owns rANS state l.  Symbols are coded in the reverse of the
// decode order; the words a step pushes are placed with a ballot so that,
// written backwards from the end of the tile's scratch region, they appear in
// decode order (ascending lanes within a step), and a compaction pass moves
// each tile's words to its offset in the payload.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "entropack.h"
#include "entropack_device_encode.h"
#include "entropack_encode.h"
#include "ep_encode_common.h"

int ep_record_error(int code, const std::string& msg);

namespace {

using ep_common::kFields;
using ep_common::kStateLow;
using ep_common::kTables;

constexpr int kHistBins = 32768;       // LDS-privatised histogram capacity (128 KB)
constexpr int kRowBlock = 64;          // rows per block in the per-row passes
constexpr int kRowChunk = 128;         // columns staged per step in the per-row passes

struct HipFailure {
  int code;
  std::string msg;
};

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) throw HipFailure{EP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e)};
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- kernels
// Per-table value bounds and bases, passed by value.  Indices are always
// compile-time constants plus a select on the coset bit.
struct TableArgs {
  int32_t minv[kTables];
  uint32_t base[kTables];
};

__device__ __forceinline__ int32_t sel(int c, int32_t a0, int32_t a1) { return c ? a1 : a0; }

// OCP e4m3fn code of y: |y| clamped to 448, round to nearest even at the
// format's quantum (subnormal quantum 2^-9 below 2^-6).
__device__ uint32_t fp8_code(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  float a = fminf(fabsf(y), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = uint32_t(rintf(a * 512.0f));          // exact scaling, then ties to even
  } else {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFFu + ((u >> 20) & 1u);              // round the 20 dropped mantissa bits
    code = (u >> 20) - (120u << 3);
  }
  return sign | code;
}

__device__ float fp8_value(uint32_t code) {
  const int e = (code >> 3) & 0xF, m = code & 7;
  const float mag = e == 0 ? ldexpf(float(m), -9) : ldexpf(float(8 + m), e - 10);
  return (code & 0x80u) ? -mag : mag;
}

// Row-scaled pre-cast (appendix B.1): q_r = max|W_r| / 448 (FP8) or / 127
// (INT8); Wq = FP8 value of W/q_r, or rint(W/q_r) clamped to +-127.
__global__ __launch_bounds__(256) void precast_kernel(const float* __restrict__ W, int64_t rows, int64_t cols,
                                                     int route, float* __restrict__ Wq,
                                                     float* __restrict__ qscale) {
  __shared__ float red[4];
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* w = W + r * cols;
    float amax = 0.0f;
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) amax = fmaxf(amax, fabsf(w[c]));
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float qs = route == EP_ROUTE_FP8 ? amax / 448.0f : amax / 127.0f;
    if (threadIdx.x == 0) qscale[r] = qs;
    for (int64_t c = threadIdx.x; c < cols; c += blockDim.x) {
      float v = 0.0f;
      if (qs != 0.0f) {
        const float y = w[c] / qs;
        v = route == EP_ROUTE_FP8 ? fp8_value(fp8_code(y)) : fminf(127.0f, fmaxf(-127.0f, rintf(y)));
      }
      Wq[r * cols + c] = v;
    }
  }
}

// Nearest point of D8: round half to even, then fix an odd coordinate sum
// by moving the worst-rounded coordinate (first on ties) the other way.
__device__ __forceinline__ void nearest_d8(const double* v, double* y) {
  int32_t par = 0;
  int worst = 0;
  double werr = -1.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] = rint(v[i]);
    par ^= int32_t(y[i]);
    const double e = fabs(v[i] - y[i]);
    if (e > werr) {
      werr = e;
      worst = i;
    }
  }
  if (par & 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i == worst) y[i] += (v[i] >= y[i]) ? 1.0 : -1.0;
  }
}

// E8 quantisation of the vectors of `nrows` rows (rows idx[i], or i when idx
// is null) at scale s: u = w / n_row, v = u / s, nearest of D8 and D8 + 1/2
// (fp64 squared distances summed in coordinate order, ties to the integer
// coset), fields (c, z1..z7, floor(z8/2)) stored as 9 planes of `stride`.
// Also the per-table ranges: lo[k] = min, lo[17 + k] = -max (atomicMin).
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ Wq, int64_t cols,
                                                      const double* __restrict__ norms,
                                                      const int64_t* __restrict__ idx, uint64_t nq,
                                                      double s, int32_t* __restrict__ fields,
                                                      uint64_t stride, int32_t* __restrict__ ranges) {
  const uint64_t per_row = uint64_t(cols) / 8;
  int32_t lo[16], nhi[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo[k] = INT32_MAX;
    nhi[k] = INT32_MAX;
  }
  for (uint64_t g = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < nq;
       g += uint64_t(gridDim.x) * blockDim.x) {
    const uint64_t i = g / per_row, j = g - i * per_row;
    const int64_t r = idx ? idx[i] : int64_t(i);
    const double n = norms[r];
    const float4* src = reinterpret_cast<const float4*>(Wq + r * cols + 8 * int64_t(j));
    const float4 a = src[0], b = src[1];
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    double v[8], y0[8], h[8], y1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const double u = n > 0.0 ? double(w[q]) / n : 0.0;
      v[q] = u / s;
      h[q] = v[q] - 0.5;
    }
    nearest_d8(v, y0);
    nearest_d8(h, y1);
    double d0 = 0.0, d1 = 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const double p = y1[q] + 0.5;
      d0 += (v[q] - y0[q]) * (v[q] - y0[q]);
      d1 += (v[q] - p) * (v[q] - p);
    }
    const int c = d0 <= d1 ? 0 : 1;
    int32_t z[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) z[q] = int32_t(c ? y1[q] : y0[q]);
    int32_t fl[kFields];
    fl[0] = c;
#pragma unroll
    for (int q = 0; q < 7; ++q) fl[1 + q] = z[q];
    fl[8] = z[7] >> 1;
#pragma unroll
    for (int f = 0; f < kFields; ++f) fields[uint64_t(f) * stride + g] = fl[f];
#pragma unroll
    for (int f = 1; f < kFields; ++f) {
      const int k0 = 2 * (f - 1);   // table 1 + k0 + c, stored at index k0 + c
      if (c) {
        lo[k0 + 1] = min(lo[k0 + 1], fl[f]);
        nhi[k0 + 1] = min(nhi[k0 + 1], -fl[f]);
      } else {
        lo[k0] = min(lo[k0], fl[f]);
        nhi[k0] = min(nhi[k0], -fl[f]);
      }
    }
  }
  __shared__ int32_t red[4][32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int32_t a = lo[k], b = nhi[k];
    for (int o = 32; o > 0; o >>= 1) {
      a = min(a, __shfl_xor(a, o));
      b = min(b, __shfl_xor(b, o));
    }
    if (lane == 0) {
      red[wv][k] = a;
      red[wv][16 + k] = b;
    }
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    int32_t m = red[0][threadIdx.x];
    for (int w = 1; w < 4; ++w) m = min(m, red[w][threadIdx.x]);
    const int k = 1 + (threadIdx.x & 15);
    if (m != INT32_MAX) atomicMin(&ranges[threadIdx.x < 16 ? k : kTables + k], m);
  }
}

// Symbol counts over the first nq vectors of the bins [lo, hi) of the 17
// tables' concatenated histograms (counts[base[k] + value - min[k]]); fmask
// names the fields whose tables meet that range.  With lds, the block counts
// privately first (hi - lo <= kHistBins); otherwise it adds to global memory
// directly (one very wide table).
__global__ __launch_bounds__(1024) void histogram_kernel(const int32_t* __restrict__ fields, uint64_t stride,
                                                        uint64_t nq, TableArgs ta, uint32_t lo, uint32_t hi,
                                                        uint32_t fmask, int lds, uint32_t* __restrict__ counts) {
  __shared__ uint32_t h[kHistBins];
  const uint32_t nb = hi - lo;
  if (lds) {
    for (uint32_t i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0;
    __syncthreads();
  }
  for (uint64_t g = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < nq;
       g += uint64_t(gridDim.x) * blockDim.x) {
    const int c = fields[g];
#pragma unroll
    for (int f = 0; f < kFields; ++f) {
      if (!((fmask >> f) & 1u)) continue;
      uint32_t bin;
      if (f == 0) {
        bin = ta.base[0] + uint32_t(c);
      } else {
        const int k0 = 1 + 2 * (f - 1);
        const int32_t mn = sel(c, ta.minv[k0], ta.minv[k0 + 1]);
        const uint32_t bs = uint32_t(sel(c, int32_t(ta.base[k0]), int32_t(ta.base[k0 + 1])));
        bin = bs + uint32_t(fields[uint64_t(f) * stride + g] - mn);
      }
      const uint32_t rel = bin - lo;
      if (rel < nb) {
        if (lds) atomicAdd(&h[rel], 1u);
        else atomicAdd(&counts[bin], 1u);
      }
    }
  }
  if (lds) {
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nb; i += blockDim.x)
      if (h[i]) atomicAdd(&counts[lo + i], h[i]);
  }
}

// Direct-z8 coding (the Table 4 ablation): field 8 becomes z8 = 2 m +
// parity(z1..z7) in place, with its per-coset range: ranges[15 + c] = min,
// ranges[17 + 15 + c] = -max (atomicMin).
__global__ __launch_bounds__(256) void z8_kernel(int32_t* __restrict__ fields, uint64_t stride, uint64_t nq,
                                                int32_t* __restrict__ ranges) {
  int32_t lo[2] = {INT32_MAX, INT32_MAX}, nhi[2] = {INT32_MAX, INT32_MAX};
  for (uint64_t g = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < nq;
       g += uint64_t(gridDim.x) * blockDim.x) {
    const int c = fields[g];
    int32_t par = 0;
#pragma unroll
    for (int f = 1; f <= 7; ++f) par ^= fields[uint64_t(f) * stride + g];
    const int32_t z8 = 2 * fields[8 * stride + g] + (par & 1);
    fields[8 * stride + g] = z8;
    if (c) {
      lo[1] = min(lo[1], z8);
      nhi[1] = min(nhi[1], -z8);
    } else {
      lo[0] = min(lo[0], z8);
      nhi[0] = min(nhi[0], -z8);
    }
  }
  __shared__ int32_t red[4][4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int32_t v[4] = {lo[0], lo[1], nhi[0], nhi[1]};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    for (int o = 32; o > 0; o >>= 1) v[i] = min(v[i], __shfl_xor(v[i], o));
    if (lane == 0) red[wv][i] = v[i];
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    int32_t m = red[0][threadIdx.x];
    for (int w = 1; w < 4; ++w) m = min(m, red[w][threadIdx.x]);
    const int k = 15 + (threadIdx.x & 1);
    if (m != INT32_MAX) atomicMin(&ranges[threadIdx.x < 2 ? k : kTables + k], m);
  }
}

// Per-row sequential passes: lane l of wave 0 owns row r0 + l and adds in
// column order; all four waves stage the next chunk of kRowChunk columns of
// the block's 64 rows (and, with fields, their fields) through registers
// into the other half of a double buffer while wave 0 works on the current
// one.  kSumSq: sums[r] = sum of w^2.  kRefit: least-squares row scale
// <W_r, sX_r> / <sX_r, sX_r>, X_r rebuilt from the fields.  kDistortion:
// sums[r] = sum of (w - y)^2 with y = fp32(x * fp32(s * row_scales[r])), the
// decoded value.
enum RowPass : int { kSumSq = 0, kRefit = 1, kDistortion = 2 };
template <int kMode>
__global__ __launch_bounds__(256) void row_pass_kernel(const float* __restrict__ Wq, int64_t rows, int64_t cols,
                                                      const int32_t* __restrict__ fields, uint64_t stride,
                                                      double s, double* __restrict__ sums,
                                                      float* __restrict__ row_scales) {
  constexpr bool kFieldsIn = kMode != kSumSq;
  constexpr int kVec = kRowChunk / 8;                       // vectors per row per chunk
  constexpr int kW4 = kRowBlock * kRowChunk / 4 / 256;      // float4 loads per thread per chunk
  constexpr int kF = kFieldsIn ? kFields * kRowBlock * kVec / 256 : 1;   // field loads per thread
  __shared__ float wt[2][kRowBlock][kRowChunk + 1];
  __shared__ int32_t ft[2][kFieldsIn ? kFields : 1][kRowBlock][kFieldsIn ? kVec + 1 : 1];
  const int tid = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x) * kRowBlock;
  const int nrow = int(std::min<int64_t>(kRowBlock, rows - r0));
  const uint64_t per_row = uint64_t(cols) / 8;
  const int nchunks = int((cols + kRowChunk - 1) / kRowChunk);
  float4 wreg[kW4];
  int32_t freg[kF];

  auto gload = [&](int ch) {
    const int64_t c0 = int64_t(ch) * kRowChunk;
    const int nc = int(std::min<int64_t>(kRowChunk, cols - c0));
#pragma unroll
    for (int k = 0; k < kW4; ++k) {
      const int row = (tid >> 5) + 8 * k, c4 = tid & 31;
      if (row < nrow && 4 * c4 < nc)
        wreg[k] = *reinterpret_cast<const float4*>(Wq + (r0 + row) * cols + c0 + 4 * c4);
    }
    if (kFieldsIn) {
      const int nv = nc / 8;
      const uint64_t j0 = uint64_t(c0) / 8;
#pragma unroll
      for (int k = 0; k < kF; ++k) {
        const int f = k >> 2, rem = tid + 256 * (k & 3), row = rem >> 4, v = rem & 15;
        if (row < nrow && v < nv) freg[k] = fields[uint64_t(f) * stride + uint64_t(r0 + row) * per_row + j0 + v];
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kW4; ++k) {
      const int row = (tid >> 5) + 8 * k, c4 = tid & 31;
      wt[buf][row][4 * c4 + 0] = wreg[k].x;
      wt[buf][row][4 * c4 + 1] = wreg[k].y;
      wt[buf][row][4 * c4 + 2] = wreg[k].z;
      wt[buf][row][4 * c4 + 3] = wreg[k].w;
    }
    if (kFieldsIn) {
#pragma unroll
      for (int k = 0; k < kF; ++k) {
        const int f = k >> 2, rem = tid + 256 * (k & 3), row = rem >> 4, v = rem & 15;
        ft[buf][f][row][v] = freg[k];
      }
    }
  };

  double acc = 0.0, num = 0.0, den = 0.0;
  // the decoded multiplier fp32(s * r) of the row (distortion pass)
  const float gs = kMode == kDistortion && tid < nrow ? float(s) * row_scales[r0 + tid] : 0.0f;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    const int nc = int(std::min<int64_t>(kRowChunk, cols - int64_t(ch) * kRowChunk));
    if (ch + 1 < nchunks) gload(ch + 1);
    if (tid < nrow) {
      if (kMode == kSumSq) {
        for (int q = 0; q < nc; ++q) {
          const double w = double(wt[buf][tid][q]);
          acc += w * w;
        }
      } else {
        for (int v = 0; v < nc / 8; ++v) {
          const int64_t c = ft[buf][0][tid][v];
          int64_t s7 = 0, x2[8];
#pragma unroll
          for (int i = 1; i <= 7; ++i) {
            const int64_t z = ft[buf][i][tid][v];
            s7 += z;
            x2[i - 1] = 2 * z + c;
          }
          const int64_t z8 = 2 * int64_t(ft[buf][8][tid][v]) + (s7 & 1);
          x2[7] = 2 * z8 + c;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (kMode == kRefit) {
              const double sx = s * (double(x2[q]) * 0.5);
              num += double(wt[buf][tid][8 * v + q]) * sx;
              den += sx * sx;
            } else {
              const float y = float(x2[q]) * 0.5f * gs;
              const double e = double(wt[buf][tid][8 * v + q]) - double(y);
              acc += e * e;
            }
          }
        }
      }
    }
    if (ch + 1 < nchunks) lstore(buf ^ 1);
    __syncthreads();
  }
  if (tid < nrow) {
    if (kMode == kRefit) row_scales[r0 + tid] = den > 0.0 ? float(num / den) : 0.0f;
    else sums[r0 + tid] = acc;
  }
}

// Per-row rate of a set of candidate fields under a model (per-row
// refinement): block (r, k) adds the costs of row r's symbols in candidate k
// (planes of `stride` at cand + k * kFields * stride).  Costs are integers
// (units of 2^-16 bit), so the sum is exact in any order.  A value outside a
// table's range costs `miss`.
struct CostArgs {
  int32_t minv[kTables];
  uint32_t A[kTables];
  uint32_t base[kTables];
  int64_t miss;
};

__global__ __launch_bounds__(256) void rate_kernel(const int32_t* __restrict__ cand, uint64_t stride,
                                                  uint64_t per_row, CostArgs ca, const int64_t* __restrict__ cost,
                                                  uint32_t K, int64_t* __restrict__ rate) {
  const uint64_t r = blockIdx.x;
  const uint32_t k = blockIdx.y;
  const int32_t* f0 = cand + uint64_t(k) * kFields * stride;
  int64_t acc = 0;
  for (uint64_t j = threadIdx.x; j < per_row; j += blockDim.x) {
    const uint64_t g = r * per_row + j;
    const int c = f0[g];
    {
      const int64_t i = c;
      acc += cost[ca.base[0] + i];
    }
#pragma unroll
    for (int f = 1; f < kFields; ++f) {
      const int t = 1 + 2 * (f - 1);
      const int32_t mn = sel(c, ca.minv[t], ca.minv[t + 1]);
      const uint32_t A = c ? ca.A[t + 1] : ca.A[t];
      const uint32_t b0 = c ? ca.base[t + 1] : ca.base[t];
      const int64_t i = int64_t(f0[uint64_t(f) * stride + g]) - mn;
      acc += (i >= 0 && i < int64_t(A)) ? cost[b0 + i] : ca.miss;
    }
  }
  __shared__ int64_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (int(threadIdx.x) < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) rate[uint64_t(k) * gridDim.x + r] = red[0];
}

// Gather each row's selected candidate into `fields` and take the per-table
// ranges like quantize_kernel (lo[k] = min, lo[17 + k] = -max).
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ cand, uint64_t stride,
                                                    uint64_t nvec, uint64_t per_row,
                                                    const int32_t* __restrict__ choice,
                                                    int32_t* __restrict__ fields, int32_t* __restrict__ ranges) {
  int32_t lo[16], nhi[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo[k] = INT32_MAX;
    nhi[k] = INT32_MAX;
  }
  for (uint64_t g = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; g < nvec;
       g += uint64_t(gridDim.x) * blockDim.x) {
    const int32_t* src = cand + uint64_t(choice[g / per_row]) * kFields * stride;
    int32_t fl[kFields];
#pragma unroll
    for (int f = 0; f < kFields; ++f) {
      fl[f] = src[uint64_t(f) * stride + g];
      fields[uint64_t(f) * stride + g] = fl[f];
    }
    const int c = fl[0];
#pragma unroll
    for (int f = 1; f < kFields; ++f) {
      const int k0 = 2 * (f - 1);
      if (c) {
        lo[k0 + 1] = min(lo[k0 + 1], fl[f]);
        nhi[k0 + 1] = min(nhi[k0 + 1], -fl[f]);
      } else {
        lo[k0] = min(lo[k0], fl[f]);
        nhi[k0] = min(nhi[k0], -fl[f]);
      }
    }
  }
  __shared__ int32_t red[4][32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int32_t a = lo[k], b = nhi[k];
    for (int o = 32; o > 0; o >>= 1) {
      a = min(a, __shfl_xor(a, o));
      b = min(b, __shfl_xor(b, o));
    }
    if (lane == 0) {
      red[wv][k] = a;
      red[wv][16 + k] = b;
    }
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    int32_t m = red[0][threadIdx.x];
    for (int w = 1; w < 4; ++w) m = min(m, red[w][threadIdx.x]);
    const int k = 1 + (threadIdx.x & 15);
    if (m != INT32_MAX) atomicMin(&ranges[threadIdx.x < 16 ? k : kTables + k], m);
  }
}

// rANS encode of tiles of V vectors: one tile per half-wave, lane l owns
// state l and the tile's vectors l, l+32, ...  Coding runs in the reverse of
// the decode order (rounds descending, fields m..c, lanes descending); a
// lane whose state would leave [2^15, 2^31) pushes its low 16 bits first.
// Words are written backwards from the end of the tile's region of `cap`
// words so that they read in decode order.  tab[base[k] + i] = cum | f << 16.
__global__ __launch_bounds__(256) void rans_encode_kernel(const int32_t* __restrict__ fields, uint64_t stride,
                                                         uint64_t nvec, uint32_t V, uint32_t T, uint32_t b,
                                                         TableArgs ta, const uint32_t* __restrict__ tab,
                                                         uint32_t* __restrict__ states,
                                                         uint32_t* __restrict__ wcount,
                                                         uint16_t* __restrict__ scratch, uint64_t cap,
                                                         uint32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, l = lane & 31;
  const uint64_t t = (uint64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6)) * 2 + half;
  const bool live = t < T;
  const uint64_t first = t * V;
  const uint32_t n = live ? uint32_t(std::min<uint64_t>(V, nvec - first)) : 0u;
  uint16_t* region = scratch + (live ? t : 0) * cap;
  const uint32_t below = (1u << l) - 1u;
  const int rounds = int((V + 31) / 32);
  uint32_t x = kStateLow, pos = 0, bad = 0;
  for (int k = rounds - 1; k >= 0; --k) {
    const uint32_t v = uint32_t(k) * 32 + uint32_t(l);
    const bool active = v < n;
    int32_t fl[kFields];
#pragma unroll
    for (int f = 0; f < kFields; ++f) fl[f] = active ? fields[uint64_t(f) * stride + first + v] : 0;
    const int c = fl[0];
#pragma unroll
    for (int f = kFields - 1; f >= 0; --f) {
      uint32_t ent = 0;
      if (active) {
        if (f == 0) {
          ent = tab[ta.base[0] + uint32_t(c)];
        } else {
          const int k0 = 1 + 2 * (f - 1);
          const int32_t mn = sel(c, ta.minv[k0], ta.minv[k0 + 1]);
          const uint32_t bs = uint32_t(sel(c, int32_t(ta.base[k0]), int32_t(ta.base[k0 + 1])));
          ent = tab[bs + uint32_t(fl[f] - mn)];
        }
      }
      uint32_t fq = ent >> 16;
      const uint32_t cm = ent & 0xFFFFu;
      if (active && fq == 0) {
        bad = 1;
        fq = 1;
      }
      const bool push = active && x >= (fq << (31 - b));
      const uint32_t hm = uint32_t(__ballot(push) >> (32 * half));
      const uint32_t np = __popc(hm);
      if (push) {
        region[cap - pos - np + __popc(hm & below)] = uint16_t(x & 0xFFFFu);
        x >>= 16;
      }
      pos += np;
      if (active) x = ((x / fq) << b) + (x % fq) + cm;
    }
  }
  if (live) {
    states[t * 32 + l] = x;
    if (l == 0) wcount[t] = pos;
  }
  if (bad) atomicOr(err, 1u);
}

// offsets[t] = exclusive prefix sum of wcount (one block of 1024 threads);
// offsets[T] and *total get the sum (64-bit, so overflow is visible).
__global__ __launch_bounds__(1024) void offsets_kernel(const uint32_t* __restrict__ wcount, uint32_t T,
                                                      uint32_t* __restrict__ offsets,
                                                      unsigned long long* __restrict__ total) {
  __shared__ unsigned long long wsum[16];
  __shared__ unsigned long long running;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (threadIdx.x == 0) running = 0;
  __syncthreads();
  for (uint32_t base = 0; base < T; base += 1024) {
    const uint32_t t = base + threadIdx.x;
    const unsigned long long val = t < T ? wcount[t] : 0ull;
    unsigned long long inc = val;
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    unsigned long long before = running;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    if (t < T) offsets[t] = uint32_t(before + inc - val);
    __syncthreads();
    if (threadIdx.x == 1023) running = before + inc;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    offsets[T] = uint32_t(running);
    *total = running;
  }
}

// Moves each tile's words from the end of its scratch region to its offset.
__global__ __launch_bounds__(256) void compact_kernel(const uint16_t* __restrict__ scratch, uint64_t cap,
                                                     const uint32_t* __restrict__ wcount,
                                                     const uint32_t* __restrict__ offsets, uint32_t T,
                                                     uint16_t* __restrict__ payload) {
  for (uint64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const uint32_t n = wcount[t];
    const uint16_t* src = scratch + t * cap + (cap - n);
    uint16_t* dst = payload + offsets[t];
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
  }
}

// ---------------------------------------------------------------- host side
struct Shape {
  int64_t rows, cols, per_row;
  uint64_t nvec, T, cap;   // cap = 9 V words of scratch per tile
  uint32_t V;
  int route;
  uint32_t nbins;          // histogram capacity (all 17 tables)
  uint32_t ntab;           // table capacity (sum of alphabets <= 2 + 16 * 2^15)
};

struct Layout {
  size_t wq, qs, sums, norms, sample, fields, ranges, counts, tab, freqs, rscale, states, wcount, offsets,
      total, scratch, bytes;
};

// Largest |field| any scale of the search can produce: |u| <= sqrt(cols)
// after RMS normalisation, s >= 1e-3, and a coordinate moves by at most 1.5.
uint32_t bins_bound(int64_t cols) {
  const double vmax = std::ceil(std::sqrt(double(cols)) * 1000.01) + 4.0;
  return uint32_t(2 + 16 * (2 * uint64_t(vmax) + 1));
}

int make_shape(int64_t rows, int64_t cols, double target_bpp, uint32_t V, int route, Shape& S) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return EP_ERR_INVALID_ARG;
  if (route < EP_ROUTE_DIRECT || route > EP_ROUTE_INT8) return EP_ERR_INVALID_ARG;
  if (uint64_t(rows) * uint64_t(cols) / 8u > 0xFFFFFFFFull) return EP_ERR_INVALID_ARG;
  if (!(target_bpp > 0.0) || !std::isfinite(target_bpp)) return EP_ERR_INVALID_ARG;
  if (V == 0) V = ep_common::default_vectors_per_tile(target_bpp);
  if (V < 32) return EP_ERR_INVALID_ARG;
  if (cols > (int64_t(1) << 34)) return EP_ERR_UNSUPPORTED;
  S.rows = rows;
  S.cols = cols;
  S.per_row = cols / 8;
  S.nvec = uint64_t(rows) * uint64_t(S.per_row);
  S.V = V;
  S.T = (S.nvec + V - 1) / V;
  S.cap = uint64_t(kFields) * V;
  S.route = route;
  S.nbins = bins_bound(cols);
  S.ntab = std::min<uint32_t>(S.nbins, 2 + 16 * (1u << 15));
  return EP_OK;
}

Layout make_layout(const Shape& S) {
  Layout L;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t p = at;
    at += align256(std::max<size_t>(bytes, 1));
    return p;
  };
  const size_t R = size_t(std::max<int64_t>(S.rows, 1));
  const bool rt = S.route != EP_ROUTE_DIRECT;
  L.wq = take(rt ? size_t(S.rows) * size_t(S.cols) * 4 : 0);
  L.qs = take(rt ? R * 4 : 0);
  L.sums = take(R * 8);
  L.norms = take(R * 8);
  L.sample = take(R * 8);
  L.fields = take(size_t(kFields) * std::max<uint64_t>(S.nvec, 1) * 4);
  L.ranges = take(2 * kTables * 4);
  L.counts = take(size_t(S.nbins) * 4);
  L.tab = take(size_t(S.ntab) * 4);
  L.freqs = take(size_t(S.ntab) * 2);
  L.rscale = take(R * 4);
  L.states = take(size_t(S.T) * 32 * 4);
  L.wcount = take(size_t(S.T) * 4);
  L.offsets = take((size_t(S.T) + 1) * 4);
  L.total = take(16);
  L.scratch = take(size_t(S.T) * size_t(S.cap) * 2);
  L.bytes = at;
  return L;
}

int grid_for(uint64_t items, int block, int cap_blocks) {
  return int(std::max<uint64_t>(1, std::min<uint64_t>((items + block - 1) / block, uint64_t(cap_blocks))));
}

struct Stats {
  int32_t minv[kTables];
  uint32_t A[kTables];
  uint32_t base[kTables];
  uint32_t sum;
};

class DeviceEncoder {
 public:
  DeviceEncoder(const Shape& S, const Layout& L, char* ws, hipStream_t st) : S_(S), L_(L), ws_(ws), st_(st) {}

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws_ + off); }

  // Route pre-cast and row norms n_r = sqrt(mean w^2) (the square root of
  // the fp64 row mean is taken on the host, like the host compressor).
  void prepare(const float* W) {
    const float* Wq = W;
    if (S_.route != EP_ROUTE_DIRECT) {
      if (S_.rows > 0)
        precast_kernel<<<grid_for(uint64_t(S_.rows), 1, 1 << 16), 256, 0, st_>>>(
            W, S_.rows, S_.cols, S_.route, at<float>(L_.wq), at<float>(L_.qs));
      check(hipGetLastError(), "precast_kernel");
      Wq = at<const float>(L_.wq);
    }
    Wq_ = Wq;
    norms_.assign(size_t(std::max<int64_t>(S_.rows, 1)), 0.0);
    if (S_.rows > 0) {
      row_pass_kernel<kSumSq><<<int((S_.rows + kRowBlock - 1) / kRowBlock), 256, 0, st_>>>(
          Wq, S_.rows, S_.cols, nullptr, 0, 0.0, at<double>(L_.sums), nullptr);
      check(hipGetLastError(), "row_pass_kernel");
      check(hipMemcpyAsync(norms_.data(), at<double>(L_.sums), size_t(S_.rows) * 8, hipMemcpyDeviceToHost, st_),
            "copy row sums");
      check(hipStreamSynchronize(st_), "row sums");
      for (int64_t r = 0; r < S_.rows; ++r) norms_[size_t(r)] = std::sqrt(norms_[size_t(r)] / double(S_.cols));
      check(hipMemcpyAsync(at<double>(L_.norms), norms_.data(), size_t(S_.rows) * 8, hipMemcpyHostToDevice, st_),
            "upload norms");
    }
    sample_ = ep_common::sample_rows(S_.rows, S_.cols);
    if (!sample_.empty())
      check(hipMemcpyAsync(at<int64_t>(L_.sample), sample_.data(), sample_.size() * 8, hipMemcpyHostToDevice, st_),
            "upload sample");
  }

  // Quantise (sampled rows, or all rows) and read the table ranges back;
  // the fields go to `dst` (a K-candidate buffer) instead of the main planes
  // when given.
  Stats quantize(bool sampled, double s, int32_t* dst = nullptr) {
    const uint64_t nq = sampled ? uint64_t(sample_.size()) * uint64_t(S_.per_row) : S_.nvec;
    nq_ = nq;
    Stats st;
    if (nq == 0) {
      for (int k = 0; k < kTables; ++k) {
        st.minv[k] = 0;
        st.A[k] = 0;
      }
      st.A[0] = 2;
      bases(st);
      return st;
    }
    check(hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(at<int32_t>(L_.ranges)), INT32_MAX, 2 * kTables, st_),
          "clear ranges");
    quantize_kernel<<<grid_for(nq, 256, 2048), 256, 0, st_>>>(Wq_, S_.cols, at<double>(L_.norms),
                                                               sampled ? at<int64_t>(L_.sample) : nullptr, nq, s,
                                                               dst ? dst : at<int32_t>(L_.fields), fields_stride(),
                                                               at<int32_t>(L_.ranges));
    check(hipGetLastError(), "quantize_kernel");
    return read_ranges("quantize");
  }

  // Per-row refinement (paper section 3.5, appendix C.2): candidates at
  // rho_k * s, their row scales and distortions, then `sweeps` rounds of
  // model update and selection under the baseline's rate.  Leaves the
  // selected fields in the main planes and returns their ranges; raises b
  // if the selected fields need it, or keeps the baseline's fields if even
  // 2^15 does not hold them.
  Stats rdo(float s, uint32_t& b, uint32_t K, uint32_t sweeps, size_t ext) {
    rdo_ext_ = ext;
    const size_t R = size_t(S_.rows), N = size_t(S_.nvec);
    int32_t* cand = at<int32_t>(ext);
    const size_t cand_bytes = align256(size_t(K) * kFields * N * 4);
    float* rsc = at<float>(ext + cand_bytes);
    double* dist = at<double>(ext + cand_bytes + align256(size_t(K) * R * 4));
    int64_t* rate = at<int64_t>(ext + cand_bytes + align256(size_t(K) * R * 4) + align256(size_t(K) * R * 8));
    int32_t* choice = at<int32_t>(ext + cand_bytes + align256(size_t(K) * R * 4) + 2 * align256(size_t(K) * R * 8));
    int64_t* cost = at<int64_t>(ext + cand_bytes + align256(size_t(K) * R * 4) + 2 * align256(size_t(K) * R * 8) +
                                align256(R * 4));
    const std::vector<double> rho = rdo_ratios(K);
    const int row_blocks = int((S_.rows + kRowBlock - 1) / kRowBlock);
    for (uint32_t k = 0; k < K; ++k) {
      int32_t* fk = cand + size_t(k) * kFields * N;
      quantize(false, double(s) * rho[k], fk);
      row_pass_kernel<kRefit><<<row_blocks, 256, 0, st_>>>(Wq_, S_.rows, S_.cols, fk, fields_stride(), double(s),
                                                          nullptr, rsc + size_t(k) * R);
      row_pass_kernel<kDistortion><<<row_blocks, 256, 0, st_>>>(Wq_, S_.rows, S_.cols, fk, fields_stride(),
                                                               double(s), dist + size_t(k) * R,
                                                               rsc + size_t(k) * R);
      check(hipGetLastError(), "candidate row passes");
    }
    std::vector<double> dk(size_t(K) * R), D(size_t(K) * R);
    check(hipMemcpyAsync(dk.data(), dist, dk.size() * 8, hipMemcpyDeviceToHost, st_), "copy distortions");
    check(hipStreamSynchronize(st_), "candidates");
    for (size_t r = 0; r < R; ++r)
      for (uint32_t k = 0; k < K; ++k) D[r * K + k] = dk[size_t(k) * R + r];
    std::vector<int32_t> sel(R, 0);
    std::vector<int64_t> rk(size_t(K) * R), Rt(size_t(K) * R);
    int64_t budget = -1;
    for (uint32_t sw = 0; sw < sweeps; ++sw) {
      const Stats st = gather(sel, choice);
      // the model: the selected fields' tables at the smallest precision >= b holding them
      uint32_t bm = b;
      for (int k = 1; k < kTables; ++k)
        while (st.A[k] > (1u << bm) && bm < 15) ++bm;
      bool fits = true;
      for (int k = 1; k < kTables; ++k) fits = fits && st.A[k] <= (1u << bm);
      if (!fits) break;
      const std::vector<uint64_t> cnt = counts(st);
      std::vector<int64_t> ct(std::max<uint32_t>(st.sum, 1u), 0);
      CostArgs ca;
      ca.miss = int64_t(65536) * int64_t(bm);
      bool ok = true;
      for (int k = 0; k < kTables && ok; ++k) {
        ca.minv[k] = st.minv[k];
        ca.A[k] = st.A[k];
        ca.base[k] = st.base[k];
        if (st.A[k] == 0) continue;
        std::vector<uint16_t> f(st.A[k]);
        ok = ep_common::normalize_table(cnt.data() + st.base[k], st.A[k], bm, f.data()) == 0;
        for (uint32_t i = 0; ok && i < st.A[k]; ++i)
          ct[st.base[k] + i] = f[i] ? std::llround(65536.0 * (double(bm) - std::log2(double(f[i])))) : ca.miss;
      }
      if (!ok) break;
      check(hipMemcpyAsync(cost, ct.data(), ct.size() * 8, hipMemcpyHostToDevice, st_), "upload costs");
      rate_kernel<<<dim3(uint32_t(R), K), 256, 0, st_>>>(cand, fields_stride(), uint64_t(S_.per_row), ca, cost, K,
                                                         rate);
      check(hipGetLastError(), "rate_kernel");
      check(hipMemcpyAsync(rk.data(), rate, rk.size() * 8, hipMemcpyDeviceToHost, st_), "copy rates");
      check(hipStreamSynchronize(st_), "rates");
      for (size_t r = 0; r < R; ++r)
        for (uint32_t k = 0; k < K; ++k) Rt[r * K + k] = rk[size_t(k) * R + r];
      if (budget < 0) {
        budget = 0;
        for (size_t r = 0; r < R; ++r) budget += Rt[r * K + size_t(sel[r])];
      }
      const double lam = rdo_penalty(D, Rt, R, K, budget);
      rdo_select(D, Rt, R, K, lam, &sel);
    }
    Stats st = gather(sel, choice);
    uint32_t bf = b;
    uint32_t amax = max_alphabet(st);
    while (amax > (1u << bf) && bf < 15) ++bf;
    if (amax > (1u << bf)) {
      std::fill(sel.begin(), sel.end(), 0);
      return gather(sel, choice);
    }
    b = bf;
    return st;
  }

  // Exact symbol counts of the last quantisation, widened to 64 bits.
  std::vector<uint64_t> counts(const Stats& st) {
    if (st.sum > S_.nbins) throw HipFailure{EP_ERR_UNSUPPORTED, "alphabets exceed the histogram bound"};
    std::vector<uint64_t> out(st.sum, 0);
    if (nq_ == 0) return out;
    check(hipMemsetAsync(at<uint32_t>(L_.counts), 0, size_t(st.sum) * 4, st_), "clear counts");
    TableArgs ta;
    for (int k = 0; k < kTables; ++k) {
      ta.minv[k] = st.minv[k];
      ta.base[k] = st.base[k];
    }
    // tables are contiguous in bin space: group them so each pass fits in LDS
    const int blocks = grid_for(nq_, 8192, 256);
    for (int k0 = 0; k0 < kTables;) {
      uint32_t lo = st.base[k0], hi = lo, fmask = 0;
      int k1 = k0;
      while (k1 < kTables && (k1 == k0 || hi + st.A[k1] - lo <= uint32_t(kHistBins))) {
        hi += st.A[k1];
        fmask |= 1u << (k1 == 0 ? 0 : 1 + (k1 - 1) / 2);
        ++k1;
      }
      if (hi > lo)
        histogram_kernel<<<blocks, 1024, 0, st_>>>(at<int32_t>(L_.fields), fields_stride(), nq_, ta, lo, hi, fmask,
                                                   hi - lo <= uint32_t(kHistBins), at<uint32_t>(L_.counts));
      k0 = k1;
    }
    check(hipGetLastError(), "histogram_kernel");
    std::vector<uint32_t> c32(st.sum);
    check(hipMemcpyAsync(c32.data(), at<uint32_t>(L_.counts), size_t(st.sum) * 4, hipMemcpyDeviceToHost, st_),
          "copy counts");
    check(hipStreamSynchronize(st_), "histogram");
    for (uint32_t i = 0; i < st.sum; ++i) out[i] = c32[i];
    return out;
  }

  double estimate(double s, uint32_t b) {
    const int64_t nvec_s = int64_t(sample_.size()) * S_.per_row;
    if (nvec_s == 0) return 0.0;
    const Stats st = quantize(true, s);
    const std::vector<uint64_t> cnt = counts(st);
    const uint64_t* per[kTables];
    for (int k = 0; k < kTables; ++k) per[k] = cnt.data() + st.base[k];
    const double bits = ep_common::sample_bits(per, st.A, b);
    return ep_common::estimate_from_bits(bits, nvec_s, S_.rows, S_.cols, S_.V, st.A,
                                         S_.route != EP_ROUTE_DIRECT);
  }

  static uint32_t max_alphabet(const Stats& st) {
    uint32_t amax = 0;
    for (int k = 1; k < kTables; ++k) amax = std::max(amax, st.A[k]);
    return amax;
  }

  // Row refit, final tables (in the requested coding), tile encode and offsets.
  int finish(float s, uint32_t b, Stats st, int coding, ep_encoded_info& I) {
    I.scale = s;
    I.coding = coding;
    I.prob_bits = b;
    I.vectors_per_tile = S_.V;
    I.num_tiles = uint32_t(S_.T);
    if (S_.rows > 0) {
      row_pass_kernel<kRefit><<<int((S_.rows + kRowBlock - 1) / kRowBlock), 256, 0, st_>>>(
          Wq_, S_.rows, S_.cols, at<int32_t>(L_.fields), fields_stride(), double(s), nullptr, at<float>(L_.rscale));
      check(hipGetLastError(), "row_pass_kernel refit");
    }
    const bool pooled = coding == EP_CODING_POOLED;
    if (coding == EP_CODING_DIRECT_Z8 && S_.nvec > 0) {
      // field 8 becomes z8 (after the refit, which uses m); new ranges for tables 15, 16
      check(hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(at<int32_t>(L_.ranges)), INT32_MAX, 2 * kTables,
                              st_),
            "clear ranges");
      z8_kernel<<<grid_for(S_.nvec, 256, 2048), 256, 0, st_>>>(at<int32_t>(L_.fields), fields_stride(), S_.nvec,
                                                                at<int32_t>(L_.ranges));
      check(hipGetLastError(), "z8_kernel");
      int32_t rg[2 * kTables];
      check(hipMemcpyAsync(rg, at<int32_t>(L_.ranges), sizeof(rg), hipMemcpyDeviceToHost, st_), "copy ranges");
      check(hipStreamSynchronize(st_), "z8");
      for (int k = 15; k < kTables; ++k) {
        const int32_t mn = rg[k], mx = rg[kTables + k] == INT32_MAX ? INT32_MIN : -rg[kTables + k];
        const bool has = mn <= mx;
        st.minv[k] = has ? mn : 0;
        st.A[k] = has ? uint32_t(int64_t(mx) - int64_t(mn) + 1) : 0u;
      }
      bases(st);
    }
    if (pooled) {
      // one range per field over both cosets; the two slots keep separate count regions
      for (int f = 1; f < kFields; ++f) {
        const int k0 = 1 + 2 * (f - 1), k1 = k0 + 1;
        if (st.A[k0] && st.A[k1]) {
          const int64_t mn = std::min(st.minv[k0], st.minv[k1]);
          const int64_t mx = std::max(int64_t(st.minv[k0]) + st.A[k0], int64_t(st.minv[k1]) + st.A[k1]) - 1;
          st.minv[k0] = int32_t(mn);
          st.A[k0] = uint32_t(mx - mn + 1);
        } else if (st.A[k1]) {
          st.minv[k0] = st.minv[k1];
          st.A[k0] = st.A[k1];
        }
        st.minv[k1] = st.minv[k0];
        st.A[k1] = st.A[k0];
      }
      bases(st);
    }
    for (int k = 1; k < kTables; ++k)
      if (st.A[k] > (1u << b)) return EP_ERR_UNSUPPORTED;   // an ablation's alphabet outgrew 2^b
    std::vector<uint64_t> cnt = counts(st);
    uint32_t nf = 0;
    for (int k = 0; k < kTables; ++k) {
      I.alphabet[k] = st.A[k];
      I.min_offset[k] = st.minv[k];
      if (pooled && k > 0 && (k - 1) % 2 == 1) {   // the coset-1 slot shares the coset-0 table
        I.freq_base[k] = I.freq_base[k - 1];
        for (uint32_t i = 0; i < st.A[k]; ++i) cnt[st.base[k - 1] + i] += cnt[st.base[k] + i];
        continue;
      }
      I.freq_base[k] = nf;
      nf += st.A[k];
    }
    I.num_freqs = nf;
    if (nf > S_.ntab) return EP_ERR_UNSUPPORTED;
    freqs_.assign(std::max<uint32_t>(nf, 1u), 0);
    for (int k = 0; k < kTables; ++k) {
      if (pooled && k > 0 && (k - 1) % 2 == 1) continue;
      if (st.A[k] &&
          ep_common::normalize_table(cnt.data() + st.base[k], st.A[k], b, &freqs_[I.freq_base[k]]) != 0)
        return EP_ERR_UNSUPPORTED;
    }
    tab_.assign(std::max<uint32_t>(nf, 1u), 0);
    for (int k = 0; k < kTables; ++k) {
      if (pooled && k > 0 && (k - 1) % 2 == 1) continue;
      uint32_t cum = 0;
      for (uint32_t i = 0; i < st.A[k]; ++i) {
        const uint32_t f = freqs_[I.freq_base[k] + i];
        tab_[I.freq_base[k] + i] = cum | (f << 16);
        cum += f;
      }
    }
    check(hipMemcpyAsync(at<uint16_t>(L_.freqs), freqs_.data(), freqs_.size() * 2, hipMemcpyHostToDevice, st_),
          "upload freqs");
    check(hipMemcpyAsync(at<uint32_t>(L_.tab), tab_.data(), tab_.size() * 4, hipMemcpyHostToDevice, st_),
          "upload tables");
    check(hipMemsetAsync(at<uint32_t>(L_.total), 0, 16, st_), "clear flags");
    if (S_.T > 0) {
      TableArgs ta;
      for (int k = 0; k < kTables; ++k) {
        ta.minv[k] = st.minv[k];
        ta.base[k] = I.freq_base[k];
      }
      const uint64_t blocks = (S_.T + 7) / 8;   // 4 waves of 2 tiles
      rans_encode_kernel<<<int(blocks), 256, 0, st_>>>(
          at<int32_t>(L_.fields), fields_stride(), S_.nvec, S_.V, uint32_t(S_.T), b, ta, at<uint32_t>(L_.tab),
          at<uint32_t>(L_.states), at<uint32_t>(L_.wcount), at<uint16_t>(L_.scratch), S_.cap,
          at<uint32_t>(L_.total) + 2);
      check(hipGetLastError(), "rans_encode_kernel");
    }
    offsets_kernel<<<1, 1024, 0, st_>>>(at<uint32_t>(L_.wcount), uint32_t(S_.T), at<uint32_t>(L_.offsets),
                                       at<unsigned long long>(L_.total));
    check(hipGetLastError(), "offsets_kernel");
    uint32_t flags[4];
    check(hipMemcpyAsync(flags, at<uint32_t>(L_.total), 16, hipMemcpyDeviceToHost, st_), "copy totals");
    check(hipStreamSynchronize(st_), "encode");
    if (flags[2]) return EP_ERR_UNSUPPORTED;
    const uint64_t words = uint64_t(flags[0]) | (uint64_t(flags[1]) << 32);
    if (words > 0xFFFFFFFFull) return EP_ERR_UNSUPPORTED;
    I.payload_words = words;
    I.stored_bytes = ep_common::stored_bytes(S_.rows, S_.T, words, I.alphabet, S_.route != EP_ROUTE_DIRECT, pooled);
    return EP_OK;
  }

 private:
  uint64_t fields_stride() const { return std::max<uint64_t>(S_.nvec, 1); }

  Stats read_ranges(const char* what) {
    Stats st;
    int32_t rg[2 * kTables];
    check(hipMemcpyAsync(rg, at<int32_t>(L_.ranges), sizeof(rg), hipMemcpyDeviceToHost, st_), "copy ranges");
    check(hipStreamSynchronize(st_), what);
    for (int k = 1; k < kTables; ++k) {
      const int32_t mn = rg[k], mx = rg[kTables + k] == INT32_MAX ? INT32_MIN : -rg[kTables + k];
      const bool has = mn <= mx;
      st.minv[k] = has ? mn : 0;
      st.A[k] = has ? uint32_t(int64_t(mx) - int64_t(mn) + 1) : 0u;
    }
    st.minv[0] = 0;
    st.A[0] = 2;
    bases(st);
    return st;
  }

  // Copy every row's chosen candidate into the main planes.
  Stats gather(const std::vector<int32_t>& sel, int32_t* choice) {
    nq_ = S_.nvec;
    check(hipMemcpyAsync(choice, sel.data(), sel.size() * 4, hipMemcpyHostToDevice, st_), "upload choices");
    check(hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(at<int32_t>(L_.ranges)), INT32_MAX, 2 * kTables, st_),
          "clear ranges");
    gather_kernel<<<grid_for(S_.nvec, 256, 2048), 256, 0, st_>>>(
        at<int32_t>(rdo_ext_), fields_stride(), S_.nvec, uint64_t(S_.per_row), choice, at<int32_t>(L_.fields),
        at<int32_t>(L_.ranges));
    check(hipGetLastError(), "gather_kernel");
    return read_ranges("gather");
  }

  // Nested candidate ratios: start at 1 and repeatedly split the widest of
  // the log-scale intervals between 0.70, 1 and 1.45 at its midpoint
  // (ties: the lower interval).
  static std::vector<double> rdo_ratios(uint32_t K) {
    std::vector<std::pair<double, double>> iv = {{std::log(0.70), 0.0}, {0.0, std::log(1.45)}};
    std::vector<double> rho;
    if (K) rho.push_back(1.0);
    while (rho.size() < K) {
      size_t w = 0;
      for (size_t i = 1; i < iv.size(); ++i)
        if (iv[i].second - iv[i].first > iv[w].second - iv[w].first) w = i;
      const double mid = 0.5 * (iv[w].first + iv[w].second);
      rho.push_back(std::exp(mid));
      iv.insert(iv.begin() + long(w) + 1, {mid, iv[w].second});
      iv[w].second = mid;
    }
    return rho;
  }

  // Each row's argmin_k D + lam * R (R in 2^-16 bit; ties to the lower k); returns the total rate.
  static int64_t rdo_select(const std::vector<double>& D, const std::vector<int64_t>& R, size_t rows, uint32_t K,
                            double lam, std::vector<int32_t>* sel) {
    int64_t total = 0;
    for (size_t r = 0; r < rows; ++r) {
      uint32_t best = 0;
      double jb = D[r * K] + lam * (double(R[r * K]) / 65536.0);
      for (uint32_t k = 1; k < K; ++k) {
        const double j = D[r * K + k] + lam * (double(R[r * K + k]) / 65536.0);
        if (j < jb) {
          jb = j;
          best = k;
        }
      }
      if (sel) (*sel)[r] = int32_t(best);
      total += R[r * K + best];
    }
    return total;
  }

  // The smallest penalty (doubling from sum D / sum R, then 60 bisection
  // steps) whose choices fit the budget; 0 if the least-distortion choices fit.
  static double rdo_penalty(const std::vector<double>& D, const std::vector<int64_t>& R, size_t rows, uint32_t K,
                            int64_t budget) {
    if (rdo_select(D, R, rows, K, 0.0, nullptr) <= budget) return 0.0;
    double sd = 0.0, sr = 0.0;
    for (size_t r = 0; r < rows; ++r) {
      sd += D[r * K];
      sr += double(R[r * K]) / 65536.0;
    }
    double hi = (sd > 0.0 && sr > 0.0) ? sd / sr : 1e-30, lo = 0.0;
    for (int it = 0; it < 200 && rdo_select(D, R, rows, K, hi, nullptr) > budget; ++it) {
      lo = hi;
      hi *= 2.0;
    }
    for (int i = 0; i < 60; ++i) {
      const double mid = 0.5 * (lo + hi);
      if (rdo_select(D, R, rows, K, mid, nullptr) > budget) lo = mid;
      else hi = mid;
    }
    return hi;
  }

  static void bases(Stats& st) {
    uint32_t acc = 0;
    for (int k = 0; k < kTables; ++k) {
      st.base[k] = acc;
      acc += std::max<uint32_t>(st.A[k], k == 0 ? 2u : 0u);
    }
    st.sum = acc;
  }

  const Shape S_;
  const Layout L_;
  char* ws_;
  hipStream_t st_;
  const float* Wq_ = nullptr;
  uint64_t nq_ = 0;
  std::vector<double> norms_;
  std::vector<int64_t> sample_;
  std::vector<uint16_t> freqs_;
  std::vector<uint32_t> tab_;

 public:
  size_t rdo_ext_ = 0;      // workspace offset of the refinement's candidate fields
};

// Workspace beyond the compressor's own layout for the per-row refinement:
// K candidates' fields, row scales, distortions and rates, the choices and
// the model's cost table.
size_t rdo_extra_bytes(const Shape& S, uint32_t K) {
  const size_t R = size_t(std::max<int64_t>(S.rows, 1)), N = size_t(std::max<uint64_t>(S.nvec, 1));
  return align256(size_t(K) * kFields * N * 4) + align256(size_t(K) * R * 4) + 2 * align256(size_t(K) * R * 8) +
         align256(R * 4) + align256(size_t(S.nbins) * 8);
}

}  // namespace

extern "C" {

int ep_encode_device_workspace_size(int64_t rows, int64_t cols, double target_bpp, uint32_t vectors_per_tile,
                                    int route, size_t* bytes) {
  if (!bytes) return ep_record_error(EP_ERR_INVALID_ARG, "bytes is NULL");
  Shape S;
  const int rc = make_shape(rows, cols, target_bpp, vectors_per_tile, route, S);
  if (rc != EP_OK) return ep_record_error(rc, "invalid tensor shape, target, tile size or route");
  *bytes = make_layout(S).bytes;
  return EP_OK;
}

}  // extern "C"

namespace {

// The compressor: argument checks, Algorithm 1 with escalation, optionally
// the per-row refinement (K > 1 and sweeps > 0), then the container.
int encode_impl(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t vectors_per_tile,
                uint32_t prob_bits, int route, int coding, uint32_t K, uint32_t sweeps, void* workspace,
                size_t ws_bytes, void* stream, ep_encoded_info* info) {
  if (!info) return ep_record_error(EP_ERR_INVALID_ARG, "info is NULL");
  if (coding < EP_CODING_STANDARD || coding > EP_CODING_DIRECT_Z8)
    return ep_record_error(EP_ERR_INVALID_ARG, "coding must be an ep_coding");
  if (!W && rows > 0) return ep_record_error(EP_ERR_INVALID_ARG, "W is NULL");
  if (W && (reinterpret_cast<uintptr_t>(W) & 15))
    return ep_record_error(EP_ERR_INVALID_ARG, "W must be 16-byte aligned");
  Shape S;
  int rc = make_shape(rows, cols, target_bpp, vectors_per_tile, route, S);
  if (rc != EP_OK) return ep_record_error(rc, "invalid tensor shape, target, tile size or route");
  uint32_t b = prob_bits ? prob_bits : ep_common::default_prob_bits(target_bpp);
  if (b < 9 || b > 15) return ep_record_error(EP_ERR_INVALID_ARG, "prob_bits must be in [9, 15]");
  const bool refine = K > 1 && sweeps > 0 && S.nvec > 0;
  if (refine && rows > int64_t(INT32_MAX)) return ep_record_error(EP_ERR_UNSUPPORTED, "too many rows to refine");
  const Layout L = make_layout(S);
  const size_t need = L.bytes + (refine ? rdo_extra_bytes(S, K) : 0);
  if (!workspace || ws_bytes < need) return ep_record_error(EP_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return ep_record_error(EP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  ep_encoded_info I;
  std::memset(&I, 0, sizeof(I));
  I.rows = rows;
  I.cols = cols;
  I.route = route;
  try {
    DeviceEncoder E(S, L, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
    E.prepare(W);
    float s = 1.0f;
    Stats st;
    for (;;) {
      const double sd = ep_common::search_scale(target_bpp, [&](double sc) { return E.estimate(sc, b); });
      I.estimated_bpp = E.estimate(sd, b);
      s = float(sd);
      st = E.quantize(false, double(s));
      uint32_t amax = DeviceEncoder::max_alphabet(st);
      if (amax <= (1u << b)) break;
      if (b < 15) {
        ++b;
        continue;
      }
      while (amax > (1u << b)) {
        s = ep_common::coarsen_scale(s, amax, b);
        st = E.quantize(false, double(s));
        amax = DeviceEncoder::max_alphabet(st);
      }
      break;
    }
    if (refine) st = E.rdo(s, b, K, sweeps, L.bytes);
    rc = E.finish(s, b, st, coding, I);
    if (rc != EP_OK) return ep_record_error(rc, "a table could not be normalised or the payload is too long");
  } catch (const HipFailure& f) {
    return ep_record_error(f.code, f.msg);
  }
  *info = I;
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_encode_device(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t vectors_per_tile,
                     uint32_t prob_bits, int route, int coding, void* workspace, size_t ws_bytes, void* stream,
                     ep_encoded_info* info) {
  return encode_impl(W, rows, cols, target_bpp, vectors_per_tile, prob_bits, route, coding, 0, 0, workspace,
                     ws_bytes, stream, info);
}

int ep_encode_device_rdo_workspace_size(int64_t rows, int64_t cols, double target_bpp, uint32_t vectors_per_tile,
                                        int route, uint32_t candidates, size_t* bytes) {
  if (!bytes) return ep_record_error(EP_ERR_INVALID_ARG, "bytes is NULL");
  if (candidates < 1 || candidates > 32) return ep_record_error(EP_ERR_INVALID_ARG, "candidates must be in [1, 32]");
  Shape S;
  const int rc = make_shape(rows, cols, target_bpp, vectors_per_tile, route, S);
  if (rc != EP_OK) return ep_record_error(rc, "invalid tensor shape, target, tile size or route");
  *bytes = make_layout(S).bytes + rdo_extra_bytes(S, candidates);
  return EP_OK;
}

int ep_encode_device_rdo(const float* W, int64_t rows, int64_t cols, double target_bpp, uint32_t vectors_per_tile,
                         uint32_t prob_bits, int route, uint32_t candidates, uint32_t sweeps, void* workspace,
                         size_t ws_bytes, void* stream, ep_encoded_info* info) {
  if (candidates < 1 || candidates > 32) return ep_record_error(EP_ERR_INVALID_ARG, "candidates must be in [1, 32]");
  return encode_impl(W, rows, cols, target_bpp, vectors_per_tile, prob_bits, route, EP_CODING_STANDARD, candidates,
                     sweeps, workspace, ws_bytes, stream, info);
}

int ep_encode_device_emit(const void* workspace, const ep_encoded_info* info, float* row_scales,
                          float* route_scales, uint32_t* states, uint32_t* offsets, uint16_t* payload,
                          uint16_t* freqs, void* stream) {
  if (!workspace || !info) return ep_record_error(EP_ERR_INVALID_ARG, "workspace or info is NULL");
  Shape S;
  if (make_shape(info->rows, info->cols, 1.0, info->vectors_per_tile, info->route, S) != EP_OK ||
      S.T != info->num_tiles)
    return ep_record_error(EP_ERR_INVALID_ARG, "info does not describe an encoded tensor");
  const Layout L = make_layout(S);
  const char* ws = static_cast<const char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto copy = [&](void* dst, size_t off, size_t bytes, const char* what) {
    if (dst && bytes) check(hipMemcpyAsync(dst, ws + off, bytes, hipMemcpyDeviceToDevice, st), what);
  };
  try {
    copy(row_scales, L.rscale, size_t(S.rows) * 4, "copy row scales");
    if (S.route != EP_ROUTE_DIRECT) copy(route_scales, L.qs, size_t(S.rows) * 4, "copy route scales");
    copy(states, L.states, size_t(S.T) * 32 * 4, "copy states");
    copy(offsets, L.offsets, (size_t(S.T) + 1) * 4, "copy offsets");
    copy(freqs, L.freqs, size_t(info->num_freqs) * 2, "copy freqs");
    if (payload && S.T > 0 && info->payload_words > 0) {
      compact_kernel<<<grid_for(S.T, 1, 1 << 16), 256, 0, st>>>(
          reinterpret_cast<const uint16_t*>(ws + L.scratch), S.cap, reinterpret_cast<const uint32_t*>(ws + L.wcount),
          reinterpret_cast<const uint32_t*>(ws + L.offsets), uint32_t(S.T), payload);
      check(hipGetLastError(), "compact_kernel");
    }
  } catch (const HipFailure& f) {
    return ep_record_error(f.code, f.msg);
  }
  return EP_OK;
}

}  // extern "C"
