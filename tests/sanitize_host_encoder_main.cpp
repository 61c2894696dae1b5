// Sanitizer driver for the multithreaded host compressor, built by
// tests/test_host_encoder_sanitized.py twice: with AddressSanitizer and
// UndefinedBehaviorSanitizer, and with ThreadSanitizer.  It compresses small
// seeded matrices with 1 and 4 worker threads and requires byte-identical
// containers (tables, states, offsets, payload, scales), so that a data race
// that changed the output would also be caught without the race detector.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "entropack_encode.h"

namespace {

uint64_t rng = 0x243F6A8885A308D3ull;

uint64_t next_u64() {   // splitmix64
  uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

double uniform() { return double(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

struct Blob {
  ep_encoded_info info{};
  std::vector<float> rs, qs;
  std::vector<uint32_t> states, offsets;
  std::vector<uint16_t> payload, freqs;
};

bool encode(const std::vector<float>& W, int64_t rows, int64_t cols, double target, int route,
            int threads, Blob* b) {
  ep_encoded* e = nullptr;
  if (ep_encode_host(W.data(), rows, cols, target, 0, 0, route, threads, &e) != 0 || !e) return false;
  ep_encoded_get_info(e, &b->info);
  const size_t R = size_t(rows), T = b->info.num_tiles;
  b->rs.assign(R, 0.0f);
  b->qs.assign(R, 0.0f);
  b->states.assign(32 * T, 0);
  b->offsets.assign(T + 1, 0);
  b->payload.assign(b->info.payload_words, 0);
  b->freqs.assign(b->info.num_freqs, 0);
  ep_encoded_copy(e, b->rs.data(), route ? b->qs.data() : nullptr, b->states.data(), b->offsets.data(),
                  b->payload.data(), b->freqs.data());
  ep_encoded_free(e);
  return true;
}

template <class V>
bool same(const V& a, const V& b) {
  return a.size() == b.size() && (a.empty() || std::memcmp(a.data(), b.data(), a.size() * sizeof(a[0])) == 0);
}

}  // namespace

int main() {
  struct Case { int64_t rows, cols; double target; int route; };
  const Case cases[] = {{96, 256, 4.0, EP_ROUTE_DIRECT}, {40, 512, 8.0, EP_ROUTE_DIRECT},
                        {64, 128, 2.0, EP_ROUTE_DIRECT}, {48, 256, 5.0, EP_ROUTE_FP8},
                        {48, 256, 2.0, EP_ROUTE_INT8},   {3, 8, 4.0, EP_ROUTE_DIRECT}};
  int failures = 0;
  for (const Case& c : cases) {
    std::vector<float> W(size_t(c.rows * c.cols));
    for (float& w : W) w = float(0.02 * (uniform() + uniform() + uniform() - 1.5) / (0.25 + uniform()));
    Blob one, four;
    if (!encode(W, c.rows, c.cols, c.target, c.route, 1, &one) ||
        !encode(W, c.rows, c.cols, c.target, c.route, 4, &four)) {
      std::fprintf(stderr, "encode failed: %lldx%lld at %.1f bpp\n", (long long)c.rows, (long long)c.cols, c.target);
      ++failures;
      continue;
    }
    const bool ok = std::memcmp(&one.info, &four.info, sizeof(one.info)) == 0 && same(one.rs, four.rs) &&
                    same(one.qs, four.qs) && same(one.states, four.states) && same(one.offsets, four.offsets) &&
                    same(one.payload, four.payload) && same(one.freqs, four.freqs);
    if (!ok) {
      std::fprintf(stderr, "1 and 4 threads differ: %lldx%lld at %.1f bpp\n", (long long)c.rows,
                   (long long)c.cols, c.target);
      ++failures;
    }
  }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
