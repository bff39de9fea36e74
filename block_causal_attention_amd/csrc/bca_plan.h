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
};

// Returns kPlanOk, kPlanErrArg or kPlanErrBlockIds (with *err set).
int build_host_plan(const int32_t* ids, int64_t S, int block_m, HostPlan* out, std::string* err);

}  // namespace bca
