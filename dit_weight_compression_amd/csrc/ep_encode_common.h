// Host-side pieces shared by the two EntroPack compressors (ep_encode.cpp on
// host threads, ep_encode_gpu.hip on the MI355X).  Everything here is a
// decision both must take identically for their containers to match byte for
// byte: the row sample of the scale search, the rate estimate from exact
// symbol counts, the bisection, the probability-precision escalation, the
// frequency normalisation and the stored-size accounting.
//
// Follows "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
// Arbitrary Bitrates", section 3.4 and appendix C.1 (sampled scale search:
// twelve geometric bisection steps on [1e-3, 8] over about 2^18 vectors in
// complete rows, b starting at 11 or 12, raised up to 15, then the scale
// coarsened by 1.05 A_max / 2^b), section 3.5 (17 coset-conditioned static
// tables), appendix C.3 and Table 5 (tile size V = max(32, floor(S/9)),
// 132 bytes of metadata per tile plus one final offset).
#ifndef EP_ENCODE_COMMON_H
#define EP_ENCODE_COMMON_H

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

namespace ep_common {

constexpr int kTables = 17;
constexpr int kFields = 9;
constexpr uint32_t kStateLow = 1u << 15;

// Table of field f (0 = c, 1..7 = z1..z7, 8 = m) for a vector in coset c.
inline int table_of(int f, int c) { return f == 0 ? 0 : 1 + 2 * (f - 1) + c; }

// Default tile size for a target rate: the largest coordinate count S of
// Table 5 whose target does not exceed the request, V = max(32, floor(S/9)).
inline uint32_t default_vectors_per_tile(double target_bpp) {
  const uint32_t S = target_bpp >= 8.0 ? 4096 : target_bpp >= 7.0 ? 8192 : target_bpp >= 4.0 ? 16384 : 32768;
  return std::max<uint32_t>(32, S / kFields);
}

// Default starting probability precision: 11 bits up to 7 bpp, else 12.
inline uint32_t default_prob_bits(double target_bpp) { return target_bpp <= 7.0 ? 11u : 12u; }

// Frequencies summing to 2^b from symbol counts: f = max(1, n*M/N) for every
// observed symbol, a deficit goes to the most frequent symbol (lowest index
// on ties), an excess is removed one unit at a time from the currently
// largest frequency above one (lowest index on ties).  Returns -1 when more
// symbols are observed than 2^b can hold, 0 otherwise (all zero if N = 0).
inline int normalize_table(const uint64_t* counts, uint32_t A, uint32_t b, uint16_t* out) {
  const uint64_t M = uint64_t(1) << b;
  uint64_t N = 0, distinct = 0;
  for (uint32_t i = 0; i < A; ++i) {
    N += counts[i];
    distinct += counts[i] != 0;
  }
  std::fill(out, out + A, uint16_t(0));
  if (N == 0) return 0;
  if (distinct > M) return -1;
  std::vector<uint32_t> f(A);
  uint64_t sum = 0;
  for (uint32_t i = 0; i < A; ++i) {
    f[i] = counts[i] ? uint32_t(std::max<uint64_t>(1, counts[i] * M / N)) : 0u;
    sum += f[i];
  }
  if (sum < M) {
    uint32_t top = 0;
    for (uint32_t i = 1; i < A; ++i)
      if (counts[i] > counts[top]) top = i;
    f[top] += uint32_t(M - sum);
  } else if (sum > M) {
    // max-heap of (f, -index) over the frequencies above one: the top is the
    // largest frequency, lowest index first, exactly the unit a linear scan
    // for the first maximum would take
    std::vector<uint64_t> heap;
    for (uint32_t i = 0; i < A; ++i)
      if (f[i] > 1) heap.push_back((uint64_t(f[i]) << 32) | uint64_t(~i));
    std::make_heap(heap.begin(), heap.end());
    for (; sum > M; --sum) {
      std::pop_heap(heap.begin(), heap.end());
      const uint32_t i = ~uint32_t(heap.back());
      if (--f[i] == 1) {
        heap.pop_back();
      } else {
        heap.back() = (uint64_t(f[i]) << 32) | uint64_t(~i);
        std::push_heap(heap.begin(), heap.end());
      }
    }
  }
  for (uint32_t i = 0; i < A; ++i) out[i] = uint16_t(f[i]);
  return 0;
}

// Stored size: 32-byte header, the coset-bit table (4 bytes), per coordinate
// table a 4-byte minimum, a 2-byte alphabet size and 2 bytes per symbol, 4
// bytes per row scale (twice with a route pre-cast), 132 bytes per tile
// (32 states and one offset), the closing offset and the payload words.
// With pooled tables (the Table 4 ablation) only the coset-0 copy of each
// coordinate table is stored.
inline uint64_t stored_bytes(int64_t rows, uint64_t T, uint64_t words, const uint32_t* A, bool route,
                             bool pooled = false) {
  uint64_t bytes = 32 + 4;
  for (int k = 1; k < kTables; ++k)
    if (!(pooled && (k - 1) % 2 == 1)) bytes += 6 + 2ull * A[k];
  bytes += 4ull * uint64_t(rows);
  if (route) bytes += 4ull * uint64_t(rows);
  bytes += 132ull * T + 4 + 2ull * words;
  return bytes;
}

inline uint64_t splitmix64_next(uint64_t& st) {
  uint64_t z = (st += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Ascending indices of ceil(2^18 / (cols/8)) complete rows (at most all of
// them), drawn by a partial Fisher-Yates shuffle seeded with rows<<32 + cols.
inline std::vector<int64_t> sample_rows(int64_t rows, int64_t cols) {
  const int64_t per_row = cols / 8;
  int64_t want = per_row > 0 ? ((int64_t(1) << 18) + per_row - 1) / per_row : rows;
  want = std::max<int64_t>(1, std::min(want, rows));
  std::vector<int64_t> perm(size_t(std::max<int64_t>(rows, 1)));
  for (int64_t i = 0; i < rows; ++i) perm[size_t(i)] = i;
  uint64_t st = (uint64_t(rows) << 32) + uint64_t(cols);
  for (int64_t i = 0; i < want && i < rows; ++i) {
    const uint64_t j = uint64_t(i) + splitmix64_next(st) % uint64_t(rows - i);
    std::swap(perm[size_t(i)], perm[size_t(j)]);
  }
  if (rows == 0) return {};
  perm.resize(size_t(want));
  std::sort(perm.begin(), perm.end());
  return perm;
}

// Ideal code length of the sampled symbols, sum of count * (b - log2 f), with
// each table normalised from its own counts; +inf when a table cannot be
// normalised at this precision.  counts[k] holds A[k] entries.
inline double sample_bits(const uint64_t* const* counts, const uint32_t* A, uint32_t b) {
  double bits = 0.0;
  std::vector<uint16_t> f;
  std::vector<double> cost((size_t(1) << b) + 1, -1.0);   // b - log2(f), filled on first use
  for (int k = 0; k < kTables; ++k) {
    if (A[k] == 0) continue;
    f.assign(A[k], 0);
    if (normalize_table(counts[k], A[k], b, f.data()) != 0) return INFINITY;
    for (uint32_t i = 0; i < A[k]; ++i)
      if (counts[k][i]) {
        double& c = cost[f[i]];
        if (c < 0.0) c = double(b) - std::log2(double(f[i]));
        bits += double(counts[k][i]) * c;
      }
  }
  return bits;
}

// Sampled rate estimate in bits per weight: the sample's code length scaled
// to the whole tensor plus the exact side information (payload excluded).
inline double estimate_from_bits(double bits, int64_t sample_vectors, int64_t rows, int64_t cols,
                                 uint32_t V, const uint32_t* A, bool route) {
  if (sample_vectors == 0) return 0.0;
  const int64_t nvec = rows * (cols / 8);
  const uint64_t T = (uint64_t(nvec) + V - 1) / V;
  const double payload = bits * (double(nvec) / double(sample_vectors)) / 8.0;
  const double side = double(stored_bytes(rows, T, 0, A, route));
  return 8.0 * (payload + side) / (double(rows) * double(cols));
}

// Twelve geometric bisection steps on [1e-3, 8]: a scale whose estimate
// exceeds the target becomes the new lower end.  Returns sqrt(lo * hi).
template <class Estimate>
double search_scale(double target, Estimate&& estimate) {
  double lo = 1e-3, hi = 8.0;
  for (int it = 0; it < 12; ++it) {
    const double s = std::sqrt(lo * hi);
    if (estimate(s) > target) lo = s;
    else hi = s;
  }
  return std::sqrt(lo * hi);
}

// Scale coarsening once b = 15 still cannot hold the largest alphabet.
inline float coarsen_scale(float s, uint32_t amax, uint32_t b) {
  return float(1.05 * double(s) * double(amax) / double(1u << b));
}

}  // namespace ep_common

#endif  // EP_ENCODE_COMMON_H
