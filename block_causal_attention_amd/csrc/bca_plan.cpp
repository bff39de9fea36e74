// Segment planner: block ids -> per-row key limits and per-query-tile key ranges.
// Pure C++ (no HIP), so it can also be built and sanitised on a machine without a GPU.
//
// The rule ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section
// "Block-causal attention is the cache-enabling boundary") lets a text row see every key at or
// before it and an image row see every key before its block plus its whole block.  So each mask
// row is a prefix [0, hi(i)) of the keys: hi(i) = i + 1 on text (the bottom-right aligned causal
// triangle of the 10100.com article's piecewise-attention part) and hi(i) = end of the block on
// image rows.  hi never decreases along the sequence, so a tile's smallest limit is its first
// row's and its largest is its last row's; the O(S^2) mask is never built.
#include "bca_plan.h"

#include <algorithm>
#include <numeric>
#include <unordered_set>

namespace bca {

int build_host_plan(const int32_t* ids, int64_t S, int block_m, HostPlan* out, std::string* err) {
  if (ids == nullptr) {
    *err = "block_ids is NULL";
    return kPlanErrArg;
  }
  if (S < 1 || S > INT32_MAX) {
    *err = "seq_len must be in [1, 2^31 - 1], got " + std::to_string(S);
    return kPlanErrArg;
  }
  if (block_m < 1) {
    *err = "block_m must be positive";
    return kPlanErrArg;
  }
  HostPlan p;
  p.seq_len = S;
  // maximal runs of equal id
  std::unordered_set<int32_t> seen;
  int64_t start = 0;
  for (int64_t i = 0; i <= S; ++i) {
    if (i < S && ids[i] < -1) {
      *err = "block id " + std::to_string(ids[i]) + " at position " + std::to_string(i) +
             " is below -1";
      return kPlanErrBlockIds;
    }
    if (i == S || ids[i] != ids[start]) {
      const int32_t id = ids[start];
      if (id >= 0 && !seen.insert(id).second) {
        *err = "image block id " + std::to_string(id) + " occupies more than one run (again at " +
               std::to_string(start) + ")";
        return kPlanErrBlockIds;
      }
      p.segments.push_back((int32_t)start);
      p.segments.push_back((int32_t)i);
      p.segments.push_back(id);
      start = i;
    }
  }
  // per-row key limits
  p.row_limit.resize((size_t)S);
  const size_t nseg = p.segments.size() / 3;
  for (size_t r = 0; r < nseg; ++r) {
    const int32_t a = p.segments[3 * r], e = p.segments[3 * r + 1], id = p.segments[3 * r + 2];
    for (int32_t i = a; i < e; ++i) p.row_limit[(size_t)i] = id < 0 ? i + 1 : e;
  }
  p.useful_pairs = 0;
  for (int32_t x : p.row_limit) p.useful_pairs += x;
  // Query tiles end at the sequence's end: tile t covers rows [S - (nt - t) block_m,
  // S - (nt - 1 - t) block_m), so a partial tile is the first one, whose rows see the fewest
  // keys (hi never decreases), and its rows below 0 are padding.  Per tile the first real row's
  // limit is the minimum and the last row's the maximum.
  const int64_t nt = (S + block_m - 1) / block_m;
  p.kv_full.resize((size_t)nt);
  p.kv_end.resize((size_t)nt);
  p.tiles.assign((size_t)nt * kTileInts, 0);
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t first = S - (nt - t) * block_m;
    const int64_t last = first + block_m - 1;
    p.kv_full[(size_t)t] = p.row_limit[(size_t)std::max<int64_t>(first, 0)];
    p.kv_end[(size_t)t] = p.row_limit[(size_t)last];
    int32_t* d = &p.tiles[(size_t)t * kTileInts];
    d[1] = (int32_t)first;
    d[2] = (int32_t)S;
    d[4] = p.kv_full[(size_t)t];
    d[5] = p.kv_end[(size_t)t];
  }
  // heavy-first: kv_end descending, ties by tile index ascending
  p.order.resize((size_t)nt);
  std::iota(p.order.begin(), p.order.end(), 0);
  std::stable_sort(p.order.begin(), p.order.end(),
                   [&](int32_t x, int32_t y) { return p.kv_end[(size_t)x] > p.kv_end[(size_t)y]; });
  // prefix = everything before the last block; decode needs that block to be an image
  p.prefix_len = p.segments[3 * (nseg - 1)];
  p.target_len = S - p.prefix_len;
  p.decode_ok = p.segments[3 * (nseg - 1) + 2] >= 0 ? 1 : 0;
  p.block_m = block_m;
  p.rows = S;
  for (int64_t t = 0; t < nt; ++t) p.tiles[(size_t)t * kTileInts + 6] = (int32_t)p.prefix_len;
  p.seqs = {0, (int32_t)S, (int32_t)p.prefix_len, (int32_t)p.target_len, 0, 0, p.decode_ok, 0};
  // The prefix rows [0, P) tiled on their own: rows of the prefix see only prefix keys (P is a
  // block boundary), so their limits are the sequence's.
  const int64_t P = p.prefix_len;
  if (p.decode_ok && P > 0) {
    const int64_t ntp = (P + block_m - 1) / block_m;
    p.prefix_tiles.assign((size_t)ntp * kTileInts, 0);
    std::vector<int32_t> end((size_t)ntp);
    for (int64_t t = 0; t < ntp; ++t) {
      const int64_t first = P - (ntp - t) * block_m;
      const int64_t last = first + block_m - 1;
      int32_t* d = &p.prefix_tiles[(size_t)t * kTileInts];
      d[1] = (int32_t)first;
      d[2] = (int32_t)P;
      d[4] = p.row_limit[(size_t)std::max<int64_t>(first, 0)];
      d[5] = end[(size_t)t] = p.row_limit[(size_t)last];
      d[6] = (int32_t)P;
    }
    p.prefix_order.resize((size_t)ntp);
    std::iota(p.prefix_order.begin(), p.prefix_order.end(), 0);
    std::stable_sort(p.prefix_order.begin(), p.prefix_order.end(),
                     [&](int32_t x, int32_t y) { return end[(size_t)x] > end[(size_t)y]; });
  }
  *out = std::move(p);
  return kPlanOk;
}

int build_varlen_plan(const int32_t* ids, const int64_t* lengths, const int64_t* row_start,
                      int32_t batch, int block_m, HostPlan* out, std::string* err) {
  if (ids == nullptr || lengths == nullptr) {
    *err = "block_ids or lengths is NULL";
    return kPlanErrArg;
  }
  if (batch < 1) {
    *err = "batch must be >= 1";
    return kPlanErrArg;
  }
  std::vector<int64_t> start((size_t)batch);
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    if (lengths[b] < 1 || lengths[b] > INT32_MAX) {
      *err = "sequence " + std::to_string(b) + " has length " + std::to_string(lengths[b]);
      return kPlanErrArg;
    }
    start[(size_t)b] = row_start ? row_start[b] : total;
    total += lengths[b];
    if (start[(size_t)b] < 0 || start[(size_t)b] + lengths[b] > INT32_MAX) {
      *err = "sequence " + std::to_string(b) + " starts at row " +
             std::to_string(start[(size_t)b]) + ", outside [0, 2^31 - length]";
      return kPlanErrArg;
    }
  }
  if (total > INT32_MAX) {
    *err = "the sequences hold more than 2^31 - 1 positions";
    return kPlanErrArg;
  }
  // rows of different sequences must not overlap
  std::vector<int32_t> by_start((size_t)batch);
  std::iota(by_start.begin(), by_start.end(), 0);
  std::sort(by_start.begin(), by_start.end(),
            [&](int32_t x, int32_t y) { return start[(size_t)x] < start[(size_t)y]; });
  for (int32_t i = 1; i < batch; ++i) {
    const int32_t x = by_start[(size_t)i - 1], y = by_start[(size_t)i];
    if (start[(size_t)x] + lengths[x] > start[(size_t)y]) {
      *err = "sequences " + std::to_string(x) + " and " + std::to_string(y) + " overlap";
      return kPlanErrArg;
    }
  }
  HostPlan p;
  p.block_m = block_m;
  p.n_sequences = batch;
  p.decode_ok = 1;
  int64_t off = 0;
  for (int32_t b = 0; b < batch; ++b) {
    HostPlan one;
    const int rc = build_host_plan(ids + off, lengths[b], block_m, &one, err);
    if (rc != kPlanOk) {
      *err = "sequence " + std::to_string(b) + ": " + *err;
      return rc;
    }
    for (size_t r = 0; r < one.segments.size(); ++r) p.segments.push_back(one.segments[r]);
    p.row_limit.insert(p.row_limit.end(), one.row_limit.begin(), one.row_limit.end());
    // this sequence's cache rows and target rows follow those of the sequences before it
    const int32_t cache_row = (int32_t)p.prefix_len, target_row = (int32_t)p.target_len;
    const size_t nt = one.kv_end.size();
    for (size_t t = 0; t < nt; ++t) {
      p.kv_full.push_back(one.kv_full[t]);
      p.kv_end.push_back(one.kv_end[t]);
      const int32_t d[kTileInts] = {(int32_t)start[(size_t)b], one.tiles[t * kTileInts + 1],
                                    (int32_t)lengths[b], (int32_t)off, one.kv_full[t],
                                    one.kv_end[t], (int32_t)one.prefix_len, cache_row};
      p.tiles.insert(p.tiles.end(), d, d + kTileInts);
    }
    const int32_t sd[kSeqInts] = {(int32_t)start[(size_t)b], (int32_t)lengths[b],
                                  (int32_t)one.prefix_len, (int32_t)one.target_len, cache_row,
                                  target_row, one.decode_ok, 0};
    p.seqs.insert(p.seqs.end(), sd, sd + kSeqInts);
    p.prefix_len += one.prefix_len;
    p.target_len += one.target_len;
    p.decode_ok &= one.decode_ok;
    p.useful_pairs += one.useful_pairs;
    p.seq_len += lengths[b];
    p.rows = std::max<int64_t>(p.rows, start[(size_t)b] + lengths[b]);
    off += lengths[b];
  }
  // heavy-first over the whole batch: kv_end descending, ties by tile index ascending
  p.order.resize(p.kv_end.size());
  std::iota(p.order.begin(), p.order.end(), 0);
  std::stable_sort(p.order.begin(), p.order.end(),
                   [&](int32_t x, int32_t y) { return p.kv_end[(size_t)x] > p.kv_end[(size_t)y]; });
  *out = std::move(p);
  return kPlanOk;
}

}  // namespace bca
