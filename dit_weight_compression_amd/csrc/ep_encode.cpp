// Host-side EntroPack compressor producing the decoder's stream format.
//
// Follows "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
// Arbitrary Bitrates": Figure 2(a) and sections 3.1-3.6 (row normalisation,
// E8 quantisation, parity-reduced fields, coset-conditioned tables, sampled
// scale search, row-scale refit, tiled rANS), appendix C.1 (twelve geometric
// bisection steps on [1e-3, 8], ~2^18 sampled vectors in complete rows, b from
// 11 or 12 up to 15, then s <- 1.05 s A_max / 2^b), appendix C.3 (32 states of
// 32 bits in [2^15, 2^31), 16-bit words, V = max(32, floor(S/9))) and appendix
// B.1 (row-scaled FP8 / INT8 pre-cast).  Where the pages leave a step open
// this file makes the same choices as the decoder's format documentation in
// include/entropack.h: row RMS as the normalising statistic, Conway-Sloane
// nearest points with ties to even and to the lower coordinate, m = floor(z8/2),
// least-squares row scales, frequency normalisation f = max(1, n*M/N) with the
// deficit on the most frequent symbol and the excess taken one unit at a time
// from the largest frequency, a SplitMix64 row sample, and a rate estimate of
// sum(-log2(f/M)) over the sample plus the exact side information.
//
// Work is split over host threads by rows (quantisation, refit), by vectors
// (histograms, summed as integers) and by tiles (rANS); every floating-point
// sum keeps its sequential order, so the result does not depend on the thread
// count.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <memory>
#include <thread>
#include <vector>

#include "entropack.h"
#include "entropack_encode.h"
#include "ep_encode_common.h"

struct ep_encoded {
  ep_encoded_info info;
  std::vector<float> row_scales, route_scales;
  std::vector<uint32_t> states, offsets;
  std::vector<uint16_t> payload, freqs;
};

namespace {

using ep_common::kFields;
using ep_common::kStateLow;
using ep_common::kTables;
using ep_common::normalize_table;
using ep_common::table_of;

// ------------------------------------------------------------------ threads
void parallel_for(int threads, int64_t n, const std::function<void(int64_t, int64_t)>& body) {
  if (n <= 0) return;
  int64_t nt = std::min<int64_t>(std::max(1, threads), n);
  if (nt == 1) {
    body(0, n);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(size_t(nt));
  for (int64_t t = 0; t < nt; ++t) {
    int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    pool.emplace_back([&body, lo, hi] { body(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

// ------------------------------------------------------------------ lattice
inline double round_even(double x) {
  const double f = std::floor(x);
  const double d = x - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return std::fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

// Nearest point of D8 (Conway & Sloane): round, then fix an odd sum by moving
// the worst-rounded coordinate (first on ties) the other way.
inline void nearest_d8(const double* v, double* y) {
  int64_t sum = 0;
  int worst = 0;
  double worst_err = -1.0;
  for (int i = 0; i < 8; ++i) {
    y[i] = round_even(v[i]);
    sum += int64_t(y[i]);
    const double e = std::fabs(v[i] - y[i]);
    if (e > worst_err) {
      worst_err = e;
      worst = i;
    }
  }
  if (sum % 2 != 0) y[worst] += (v[worst] >= y[worst]) ? 1.0 : -1.0;
}

// Nearest E8 point of v written as fields (c, z1..z7, m).
inline void quantize_e8(const double* v, int32_t* fields) {
  double y0[8], w[8], y1[8];
  nearest_d8(v, y0);
  for (int i = 0; i < 8; ++i) w[i] = v[i] - 0.5;
  nearest_d8(w, y1);               // D8 part of the half-integer candidate
  double d0 = 0.0, d1 = 0.0;
  for (int i = 0; i < 8; ++i) {
    const double h = y1[i] + 0.5;
    d0 += (v[i] - y0[i]) * (v[i] - y0[i]);
    d1 += (v[i] - h) * (v[i] - h);
  }
  const double* z = d0 <= d1 ? y0 : y1;
  fields[0] = d0 <= d1 ? 0 : 1;
  for (int i = 0; i < 7; ++i) fields[1 + i] = int32_t(z[i]);
  fields[8] = int32_t(z[7]) >> 1;  // floor(z8 / 2)
}

// x_i * 2 of the point encoded by the fields.
inline void point_twice(const int32_t* fl, int64_t* x2) {
  const int64_t c = fl[0];
  int64_t s7 = 0;
  for (int i = 1; i <= 7; ++i) {
    s7 += fl[i];
    x2[i - 1] = 2 * int64_t(fl[i]) + c;
  }
  const int64_t z8 = 2 * int64_t(fl[8]) + (s7 & 1);
  x2[7] = 2 * z8 + c;
}

// ------------------------------------------------------------------ route pre-cast
uint8_t fp8_e4m3_code(float y) {
  // OCP e4m3fn: clamp to +-448, round to nearest even at the format's quantum.
  uint32_t bits;
  std::memcpy(&bits, &y, 4);
  const uint8_t sign = uint8_t((bits >> 24) & 0x80u);
  float a = std::fabs(y);
  if (a > 448.0f) a = 448.0f;
  uint32_t code;
  if (a < 0.015625f) {
    code = uint32_t(round_even(double(a) * 512.0));
  } else {
    uint32_t u;
    std::memcpy(&u, &a, 4);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    code = (u >> 20) - (120u << 3);
  }
  return uint8_t(sign | code);
}

float fp8_e4m3_value(uint8_t code) {
  const int e = (code >> 3) & 0xF, m = code & 7;
  double v = e == 0 ? std::ldexp(double(m), -9) : std::ldexp(1.0 + m / 8.0, e - 7);
  return float((code & 0x80) ? -v : v);
}

void route_precast(const float* W, int64_t rows, int64_t cols, int route, float* Wq, float* q,
                   int threads) {
  parallel_for(threads, rows, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) {
      const float* w = W + r * cols;
      float amax = 0.0f;
      for (int64_t c = 0; c < cols; ++c) amax = std::max(amax, std::fabs(w[c]));
      const float qs = route == EP_ROUTE_FP8 ? amax / 448.0f : amax / 127.0f;
      q[r] = qs;
      for (int64_t c = 0; c < cols; ++c) {
        float v = 0.0f;
        if (qs != 0.0f) {
          const float y = w[c] / qs;
          if (route == EP_ROUTE_FP8) {
            v = fp8_e4m3_value(fp8_e4m3_code(y));
          } else {
            double t = round_even(double(y));
            v = float(std::min(127.0, std::max(-127.0, t)));
          }
        }
        Wq[r * cols + c] = v;
      }
    }
  });
}

// ------------------------------------------------------------------ tables
struct TableStats {
  int32_t minv[kTables];
  uint32_t A[kTables];
  std::vector<uint64_t> counts[kTables];
};

// Ranges then counts of the 17 tables over nvec vectors of fields.
void table_stats(const int32_t* fields, int64_t nvec, int threads, TableStats& ts) {
  const int nt = int(std::max<int64_t>(1, std::min<int64_t>(threads, (nvec + 65535) / 65536)));
  std::vector<int32_t> lo(size_t(nt) * kTables, INT32_MAX), hi(size_t(nt) * kTables, INT32_MIN);
  parallel_for(nt, nt, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t g0 = nvec * t / nt, g1 = nvec * (t + 1) / nt;
      int32_t* L = &lo[size_t(t) * kTables];
      int32_t* H = &hi[size_t(t) * kTables];
      for (int64_t g = g0; g < g1; ++g) {
        const int32_t* fl = fields + kFields * g;
        for (int f = 1; f < kFields; ++f) {
          const int k = table_of(f, fl[0]);
          L[k] = std::min(L[k], fl[f]);
          H[k] = std::max(H[k], fl[f]);
        }
      }
    }
  });
  for (int k = 0; k < kTables; ++k) {
    int32_t mn = INT32_MAX, mx = INT32_MIN;
    for (int t = 0; t < nt; ++t) {
      mn = std::min(mn, lo[size_t(t) * kTables + k]);
      mx = std::max(mx, hi[size_t(t) * kTables + k]);
    }
    const bool has = mn <= mx;
    ts.minv[k] = has ? mn : 0;
    ts.A[k] = has ? uint32_t(int64_t(mx) - int64_t(mn) + 1) : 0u;
  }
  ts.minv[0] = 0;
  ts.A[0] = 2;
  std::vector<std::vector<uint64_t>> part(size_t(nt) * kTables);
  parallel_for(nt, nt, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t) {
      std::vector<uint64_t>* P = &part[size_t(t) * kTables];
      for (int k = 0; k < kTables; ++k) P[k].assign(std::max<uint32_t>(ts.A[k], 1u), 0);
      const int64_t g0 = nvec * t / nt, g1 = nvec * (t + 1) / nt;
      for (int64_t g = g0; g < g1; ++g) {
        const int32_t* fl = fields + kFields * g;
        P[0][fl[0]] += 1;
        for (int f = 1; f < kFields; ++f) {
          const int k = table_of(f, fl[0]);
          P[k][size_t(fl[f] - ts.minv[k])] += 1;
        }
      }
    }
  });
  for (int k = 0; k < kTables; ++k) {
    ts.counts[k].assign(std::max<uint32_t>(ts.A[k], 1u), 0);
    for (int t = 0; t < nt; ++t) {
      const auto& P = part[size_t(t) * kTables + k];
      for (size_t i = 0; i < P.size(); ++i) ts.counts[k][i] += P[i];
    }
  }
}

// ------------------------------------------------------------------ encoder state
struct Job {
  const float* Wq;
  int64_t rows, cols, per_row, nvec;
  uint32_t V;
  int route;
  int threads;
  std::vector<double> norms;
  std::vector<int64_t> sample;
};

void quantize_rows(const Job& J, const int64_t* idx, int64_t nrows, double s, int32_t* fields) {
  parallel_for(J.threads, nrows, [&](int64_t i0, int64_t i1) {
    double v[8];
    for (int64_t i = i0; i < i1; ++i) {
      const int64_t r = idx ? idx[i] : i;
      const double n = J.norms[size_t(r)];
      const float* w = J.Wq + r * J.cols;
      for (int64_t j = 0; j < J.per_row; ++j) {
        for (int q = 0; q < 8; ++q) {
          const double u = n > 0.0 ? double(w[8 * j + q]) / n : 0.0;
          v[q] = u / s;
        }
        quantize_e8(v, fields + kFields * (i * J.per_row + j));
      }
    }
  });
}

double estimate_bpp(const Job& J, double s, uint32_t b) {
  const int64_t ns = int64_t(J.sample.size());
  const int64_t nvec_s = ns * J.per_row;
  if (nvec_s == 0) return 0.0;
  std::vector<int32_t> fields(size_t(nvec_s) * kFields);
  quantize_rows(J, J.sample.data(), ns, s, fields.data());
  TableStats ts;
  table_stats(fields.data(), nvec_s, J.threads, ts);
  const uint64_t* counts[kTables];
  for (int k = 0; k < kTables; ++k) counts[k] = ts.counts[k].data();
  const double bits = ep_common::sample_bits(counts, ts.A, b);
  return ep_common::estimate_from_bits(bits, nvec_s, J.rows, J.cols, J.V, ts.A,
                                       J.route != EP_ROUTE_DIRECT);
}

uint32_t max_coordinate_alphabet(const int32_t* fields, int64_t nvec, int threads) {
  TableStats ts;
  table_stats(fields, nvec, threads, ts);
  uint32_t amax = 0;
  for (int k = 1; k < kTables; ++k) amax = std::max(amax, ts.A[k]);
  return amax;
}

// rANS encode of one tile (reverse of the decode order); returns words written.
int encode_tile(uint32_t n, const int32_t* sym, const uint16_t* const* fr,
                const uint32_t* const* cum, uint32_t b, uint32_t* states,
                std::vector<uint16_t>& words) {
  uint32_t x[EP_LANES];
  for (int l = 0; l < EP_LANES; ++l) x[l] = kStateLow;
  words.clear();
  const uint32_t K = (n + EP_LANES - 1) / EP_LANES;
  const uint64_t xmax_unit = uint64_t(kStateLow >> b) << 16;   // 2^(31-b)
  for (int64_t k = int64_t(K) - 1; k >= 0; --k)
    for (int f = kFields - 1; f >= 0; --f)
      for (int l = EP_LANES - 1; l >= 0; --l) {
        const uint64_t v = uint64_t(k) * EP_LANES + uint64_t(l);
        if (v >= n) continue;
        const int32_t* s = sym + kFields * v;
        const int t = table_of(f, s[0]);
        const uint32_t fq = fr[t][s[f]], cm = cum[t][s[f]];
        if (fq == 0) return -1;
        if (uint64_t(x[l]) >= xmax_unit * fq) {
          words.push_back(uint16_t(x[l] & 0xFFFFu));
          x[l] >>= 16;
        }
        x[l] = ((x[l] / fq) << b) + (x[l] % fq) + cm;
      }
  std::reverse(words.begin(), words.end());
  for (int l = 0; l < EP_LANES; ++l) states[l] = x[l];
  return 0;
}

int finish(Job& J, float s, uint32_t b, const std::vector<int32_t>& fields, ep_encoded* E) {
  ep_encoded_info& I = E->info;
  I.scale = s;
  I.prob_bits = b;
  I.vectors_per_tile = J.V;
  const uint64_t T = (uint64_t(J.nvec) + J.V - 1) / J.V;
  I.num_tiles = uint32_t(T);

  // least-squares row scales: <W_r, s X_r> / <s X_r, s X_r>
  E->row_scales.assign(size_t(J.rows), 0.0f);
  parallel_for(J.threads, J.rows, [&](int64_t r0, int64_t r1) {
    int64_t x2[8];
    for (int64_t r = r0; r < r1; ++r) {
      double num = 0.0, den = 0.0;
      for (int64_t j = 0; j < J.per_row; ++j) {
        point_twice(&fields[size_t(kFields * (r * J.per_row + j))], x2);
        for (int q = 0; q < 8; ++q) {
          const double sx = double(s) * (double(x2[q]) * 0.5);
          num += double(J.Wq[r * J.cols + 8 * j + q]) * sx;
          den += sx * sx;
        }
      }
      E->row_scales[size_t(r)] = den > 0.0 ? float(num / den) : 0.0f;
    }
  });

  TableStats ts;
  table_stats(fields.data(), J.nvec, J.threads, ts);
  uint32_t nf = 0;
  for (int k = 0; k < kTables; ++k) {
    I.alphabet[k] = ts.A[k];
    I.min_offset[k] = ts.minv[k];
    I.freq_base[k] = nf;
    nf += ts.A[k];
  }
  I.num_freqs = nf;
  E->freqs.assign(std::max<uint32_t>(nf, 1u), 0);
  for (int k = 0; k < kTables; ++k)
    if (ts.A[k] && normalize_table(ts.counts[k].data(), ts.A[k], b, &E->freqs[I.freq_base[k]]) != 0)
      return EP_ERR_UNSUPPORTED;
  std::vector<std::vector<uint32_t>> cum(kTables);
  const uint16_t* fr[kTables];
  const uint32_t* cp[kTables];
  for (int k = 0; k < kTables; ++k) {
    cum[k].assign(ts.A[k] + 1, 0);
    for (uint32_t i = 0; i < ts.A[k]; ++i) cum[k][i + 1] = cum[k][i] + E->freqs[I.freq_base[k] + i];
    fr[k] = &E->freqs[I.freq_base[k]];
    cp[k] = cum[k].data();
  }

  // zero-based symbols, then tiles in parallel, then concatenation
  std::vector<int32_t> sym(fields.size());
  parallel_for(J.threads, J.nvec, [&](int64_t g0, int64_t g1) {
    for (int64_t g = g0; g < g1; ++g) {
      const int32_t* fl = &fields[size_t(kFields * g)];
      int32_t* sy = &sym[size_t(kFields * g)];
      sy[0] = fl[0];
      for (int f = 1; f < kFields; ++f) sy[f] = fl[f] - ts.minv[table_of(f, fl[0])];
    }
  });
  E->states.assign(size_t(T) * EP_LANES, 0);
  std::vector<std::vector<uint16_t>> tile_words(static_cast<size_t>(T));
  std::atomic<int> bad{0};
  parallel_for(J.threads, int64_t(T), [&](int64_t t0, int64_t t1) {
    std::vector<uint16_t> w;
    for (int64_t t = t0; t < t1; ++t) {
      const uint64_t first = uint64_t(t) * J.V;
      const uint32_t n = uint32_t(std::min<uint64_t>(J.V, uint64_t(J.nvec) - first));
      if (encode_tile(n, &sym[size_t(kFields * first)], fr, cp, b, &E->states[size_t(t) * EP_LANES], w))
        bad = 1;
      tile_words[size_t(t)] = w;
    }
  });
  if (bad) return EP_ERR_UNSUPPORTED;
  E->offsets.assign(size_t(T) + 1, 0);
  uint64_t pos = 0;
  for (uint64_t t = 0; t < T; ++t) {
    E->offsets[size_t(t)] = uint32_t(pos);
    pos += tile_words[size_t(t)].size();
  }
  if (pos > 0xFFFFFFFFull) return EP_ERR_UNSUPPORTED;
  E->offsets[size_t(T)] = uint32_t(pos);
  E->payload.resize(size_t(pos));
  parallel_for(J.threads, int64_t(T), [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t)
      std::copy(tile_words[size_t(t)].begin(), tile_words[size_t(t)].end(),
                E->payload.begin() + E->offsets[size_t(t)]);
  });
  I.payload_words = pos;
  I.stored_bytes = ep_common::stored_bytes(J.rows, T, pos, I.alphabet, J.route != EP_ROUTE_DIRECT);
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_encode_host(const float* W, int64_t rows, int64_t cols, double target_bpp,
                   uint32_t vectors_per_tile, uint32_t prob_bits, int route, int threads,
                   ep_encoded** out) {
  if (!out || (!W && rows > 0)) return EP_ERR_INVALID_ARG;
  *out = nullptr;
  if (rows < 0 || cols <= 0 || cols % 8 != 0) return EP_ERR_INVALID_ARG;
  if (route < EP_ROUTE_DIRECT || route > EP_ROUTE_INT8) return EP_ERR_INVALID_ARG;
  if (uint64_t(rows) * uint64_t(cols) / 8u > 0xFFFFFFFFull) return EP_ERR_INVALID_ARG;
  uint32_t V = vectors_per_tile;
  if (V == 0) V = ep_common::default_vectors_per_tile(target_bpp);
  if (V < 32) return EP_ERR_INVALID_ARG;
  uint32_t b = prob_bits ? prob_bits : ep_common::default_prob_bits(target_bpp);
  if (b < 9 || b > 15) return EP_ERR_INVALID_ARG;
  if (threads <= 0) threads = int(std::max(1u, std::thread::hardware_concurrency()));

  std::unique_ptr<ep_encoded> E(new ep_encoded());
  std::memset(&E->info, 0, sizeof(E->info));
  E->info.rows = rows;
  E->info.cols = cols;
  E->info.route = route;

  Job J;
  std::vector<float> pre;
  if (route == EP_ROUTE_DIRECT) {
    J.Wq = W;
  } else {
    pre.resize(size_t(rows * cols));
    E->route_scales.resize(size_t(rows));
    route_precast(W, rows, cols, route, pre.data(), E->route_scales.data(), threads);
    J.Wq = pre.data();
  }
  J.rows = rows;
  J.cols = cols;
  J.per_row = cols / 8;
  J.nvec = rows * J.per_row;
  J.V = V;
  J.route = route;
  J.threads = threads;
  J.norms.assign(size_t(std::max<int64_t>(rows, 1)), 0.0);
  parallel_for(threads, rows, [&](int64_t r0, int64_t r1) {
    for (int64_t r = r0; r < r1; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < cols; ++c) {
        const double w = double(J.Wq[r * cols + c]);
        acc += w * w;
      }
      J.norms[size_t(r)] = std::sqrt(acc / double(cols));
    }
  });
  J.sample = ep_common::sample_rows(rows, cols);

  std::vector<int32_t> fields(size_t(std::max<int64_t>(J.nvec, 1)) * kFields);
  float s = 1.0f;
  for (;;) {
    const double sd = ep_common::search_scale(target_bpp, [&](double sc) { return estimate_bpp(J, sc, b); });
    E->info.estimated_bpp = estimate_bpp(J, sd, b);
    s = float(sd);
    quantize_rows(J, nullptr, rows, double(s), fields.data());
    uint32_t amax = max_coordinate_alphabet(fields.data(), J.nvec, threads);
    if (amax <= (1u << b)) break;
    if (b < 15) {
      ++b;
      continue;
    }
    while (amax > (1u << b)) {
      s = ep_common::coarsen_scale(s, amax, b);
      quantize_rows(J, nullptr, rows, double(s), fields.data());
      amax = max_coordinate_alphabet(fields.data(), J.nvec, threads);
    }
    break;
  }
  fields.resize(size_t(J.nvec) * kFields);
  int rc = finish(J, s, b, fields, E.get());
  if (rc != EP_OK) return rc;
  *out = E.release();
  return EP_OK;
}

int ep_encoded_get_info(const ep_encoded* e, ep_encoded_info* info) {
  if (!e || !info) return EP_ERR_INVALID_ARG;
  *info = e->info;
  return EP_OK;
}

int ep_encoded_copy(const ep_encoded* e, float* row_scales, float* route_scales, uint32_t* states,
                    uint32_t* offsets, uint16_t* payload, uint16_t* freqs) {
  if (!e) return EP_ERR_INVALID_ARG;
  auto put = [](auto* dst, const auto& src) {
    if (dst && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(src[0]));
  };
  put(row_scales, e->row_scales);
  put(route_scales, e->route_scales);
  put(states, e->states);
  put(offsets, e->offsets);
  put(payload, e->payload);
  if (freqs && e->info.num_freqs) std::memcpy(freqs, e->freqs.data(), e->info.num_freqs * 2);
  return EP_OK;
}

void ep_encoded_free(ep_encoded* e) { delete e; }

}  // extern "C"
