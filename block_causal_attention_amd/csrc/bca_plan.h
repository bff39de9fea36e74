// Host-side segment planner (no HIP dependency).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace bca {

enum { kPlanOk = 0, kPlanErrArg = 1, kPlanErrBlockIds = 2 };

struct HostPlan {
  int64_t seq_len = 0;
  int64_t prefix_len = 0;
  int64_t target_len = 0;
  int64_t useful_pairs = 0;
  int32_t decode_ok = 0;
  int32_t block_m = 0;
  std::vector<int32_t> segments;   // (start, end, id) per maximal run
  std::vector<int32_t> row_limit;  // hi(i): row i sees keys [0, hi(i))
  std::vector<int32_t> kv_full;    // per query tile: min hi over its rows
  std::vector<int32_t> kv_end;     // per query tile: max hi over its rows
  std::vector<int32_t> order;      // query tiles by kv_end descending, ties by index
  // Per query tile, kTileInts ints: tensor row of its sequence's first position, first local row
  // of the tile, positions of the sequence, offset of the sequence's limits in row_limit,
  // kv_full, kv_end (local key indices), the sequence's prefix length and the cache row where its
  // prefix is stored.
  std::vector<int32_t> tiles;
  // Per sequence, kSeqInts ints: tensor row of its first position, length, prefix length P_b
  // (start of its last block), target length N_b, first cache row (sum of the earlier P),
  // first target row (sum of the earlier N), 1 when its last block is an image block, 0.
  std::vector<int32_t> seqs;
  // Single sequence whose last block is an image block after a non-empty prefix: query tiles of
  // the prefix rows alone (ending at row P, tile layout and order as above, n_rows = P and the
  // whole prefix stored to the cache), for a prefill that hands the target rows to the decode.
  std::vector<int32_t> prefix_tiles;
  std::vector<int32_t> prefix_order;
  int32_t n_sequences = 1;
  int64_t rows = 0;                // tensor rows spanned: max(row_start + length)
};

constexpr int kTileInts = 8;
constexpr int kSeqInts = 8;

// Returns kPlanOk, kPlanErrArg or kPlanErrBlockIds (with *err set).
int build_host_plan(const int32_t* ids, int64_t S, int block_m, HostPlan* out, std::string* err);

// A batch of independent sequences: ids holds the sequences' id vectors one after another,
// lengths[b] their lengths and row_start[b] (NULL: packed) the tensor row where sequence b
// starts.  Rows of different sequences must not overlap.  Tiles never cross a sequence.  The
// plan's prefix_len and target_len are the sums over the sequences (rows of the packed prefix
// cache and of the packed decode tensors), decode_ok is 1 when every sequence ends in an image.
int build_varlen_plan(const int32_t* ids, const int64_t* lengths, const int64_t* row_start,
                      int32_t batch, int block_m, HostPlan* out, std::string* err);

}  // namespace bca
