// Host-side fuzz driver for the segment planner, built with AddressSanitizer and UBSan on the CPU
// (tests/test_planner_sanitized.py).  Random block-id layouts, including invalid ones, go
// through build_host_plan; valid plans are checked against the rule's consequences: limits are
// non-decreasing and at least i + 1, each tile's range brackets its rows, the order is a
// heavy-first permutation, and the prefix ends where the last run starts.  Batches of such
// layouts (some with gaps, overlaps or empty sequences) go through build_varlen_plan; valid batch
// plans must give every sequence its own tiles, with descriptors that stay inside the sequence.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "bca_plan.h"

#include <algorithm>

static int fail(const char* what, int64_t S) {
  std::fprintf(stderr, "FAIL %s (S=%lld)\n", what, (long long)S);
  return 1;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937_64 rng(12345);
  int valid = 0, rejected = 0;
  for (int it = 0; it < iters; ++it) {
    const int64_t S = 1 + (int64_t)(rng() % 1500);
    std::vector<int32_t> ids((size_t)S);
    int32_t next = 0;
    for (int64_t i = 0; i < S;) {
      const int64_t n = 1 + (int64_t)(rng() % 200);
      const bool text = rng() % 2;
      const int32_t id = text ? -1 : next++;
      for (int64_t k = 0; k < n && i < S; ++k, ++i) ids[(size_t)i] = id;
    }
    if (it % 7 == 3) ids[(size_t)(rng() % S)] = -2 - (int32_t)(rng() % 5);      // invalid id
    if (it % 11 == 5 && next > 0) ids[(size_t)(rng() % S)] = 0;                 // possible reuse
    const int block_m = (it % 3 == 0) ? 128 : (it % 3 == 1 ? 256 : 64);
    bca::HostPlan p;
    std::string err;
    const int rc = bca::build_host_plan(ids.data(), S, block_m, &p, &err);
    if (rc != bca::kPlanOk) {
      if (err.empty()) return fail("error without text", S);
      ++rejected;
      continue;
    }
    ++valid;
    if ((int64_t)p.row_limit.size() != S) return fail("row_limit size", S);
    for (int64_t i = 0; i < S; ++i) {
      if (p.row_limit[(size_t)i] < i + 1 || p.row_limit[(size_t)i] > S) return fail("limit range", S);
      if (i && p.row_limit[(size_t)i] < p.row_limit[(size_t)i - 1]) return fail("monotone", S);
    }
    const int64_t nt = (S + block_m - 1) / block_m;
    if ((int64_t)p.kv_full.size() != nt || (int64_t)p.order.size() != nt) return fail("tiles", S);
    std::vector<int> seen((size_t)nt, 0);
    int64_t next_row = 0;  // tiles cover rows [0, S) in order, each once; only the first is partial
    for (int64_t t = 0; t < nt; ++t) {
      const int32_t o = p.order[(size_t)t];
      if (o < 0 || o >= nt || seen[(size_t)o]++) return fail("order permutation", S);
      if (t && p.kv_end[(size_t)p.order[(size_t)t - 1]] < p.kv_end[(size_t)o]) return fail("heavy first", S);
      const int64_t first = p.tiles[(size_t)t * bca::kTileInts + 1];
      if (first + block_m <= 0 || (t > 0 && first < 0) || std::max<int64_t>(first, 0) != next_row)
        return fail("tile partition", S);
      next_row = first + block_m;
      for (int64_t r = std::max<int64_t>(first, 0); r < first + block_m; ++r)
        if (p.row_limit[(size_t)r] < p.kv_full[(size_t)t] || p.row_limit[(size_t)r] > p.kv_end[(size_t)t])
          return fail("tile range", S);
    }
    if (next_row != S) return fail("tile partition end", S);
    const size_t nseg = p.segments.size() / 3;
    if (p.prefix_len != p.segments[3 * (nseg - 1)] || p.prefix_len + p.target_len != S)
      return fail("prefix", S);
  }
  // batches of layouts
  int bvalid = 0, brejected = 0;
  for (int it = 0; it < iters / 4; ++it) {
    const int32_t batch = 1 + (int32_t)(rng() % 6);
    std::vector<int64_t> lens((size_t)batch), starts((size_t)batch);
    std::vector<int32_t> ids;
    int64_t row = (int64_t)(rng() % 50);
    for (int32_t b = 0; b < batch; ++b) {
      lens[(size_t)b] = (it % 13 == 7 && b == 0) ? 0 : 1 + (int64_t)(rng() % 700);
      starts[(size_t)b] = row;
      row += lens[(size_t)b] + (int64_t)(rng() % 40);
      int32_t next = 0;
      for (int64_t i = 0; i < lens[(size_t)b];) {
        const int64_t n = 1 + (int64_t)(rng() % 150);
        const int32_t id = (rng() % 2) ? -1 : next++;
        for (int64_t k = 0; k < n && i < lens[(size_t)b]; ++k, ++i) ids.push_back(id);
      }
    }
    if (it % 9 == 4 && batch > 1) starts[1] = starts[0];                  // overlap
    const bool packed = it % 2 == 0;
    bca::HostPlan p;
    std::string err;
    const int rc = bca::build_varlen_plan(ids.data(), lens.data(), packed ? nullptr : starts.data(),
                                          batch, 128, &p, &err);
    if (rc != bca::kPlanOk) {
      if (err.empty()) return fail("batch error without text", batch);
      ++brejected;
      continue;
    }
    ++bvalid;
    int64_t off = 0, tiles = 0, pairs = 0;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = lens[(size_t)b];
      const int64_t s0 = packed ? off : starts[(size_t)b];
      for (int64_t t = 0; t < (n + 127) / 128; ++t, ++tiles) {
        const int32_t* d = &p.tiles[(size_t)tiles * bca::kTileInts];
        const int64_t nt = (n + 127) / 128;
        if (d[0] != s0 || d[1] != n - (nt - t) * 128 || d[2] != n || d[3] != off)
          return fail("descriptor", n);
        if (d[4] < 1 || d[4] > d[5] || d[5] > n) return fail("descriptor bounds", n);
      }
      for (int64_t i = 0; i < n; ++i) {
        const int32_t lim = p.row_limit[(size_t)(off + i)];
        if (lim < i + 1 || lim > n) return fail("batch limit range", n);
        pairs += lim;
      }
      off += n;
    }
    if ((int64_t)p.order.size() != tiles || (int64_t)p.tiles.size() != tiles * bca::kTileInts)
      return fail("batch tiles", tiles);
    if (pairs != p.useful_pairs || p.n_sequences != batch) return fail("batch totals", batch);
  }
  std::printf("planner fuzz ok: %d valid, %d rejected; batches %d valid, %d rejected\n", valid,
              rejected, bvalid, brejected);
  return 0;
}
