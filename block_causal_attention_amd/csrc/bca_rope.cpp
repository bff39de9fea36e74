// Host helpers of the Q/K prologue: three-axis RoPE positions and the cos/sin table.
//
// "Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section "Three-axis RoPE
// preserves image geometry": a head's 128 dims are split (16, 56, 56) over frame, height and
// width with base 10,000; text positions advance one coordinate shared by all three axes; an
// image block keeps the frame coordinate reached by the preceding text while its height and
// width coordinates form a grid centred on zero.  Where the section is silent this follows the
// plainest reading: a shared counter c starts at 0, a text token takes (c, c, c) and advances c,
// an H x W image block (row-major) takes (c, h - H/2, w - W/2) and then advances c by one;
// rotation pairs are adjacent dims, and pair k of an axis of width d turns by
// pos * base^(-2k/d).  Angles, cos and sin are computed in double and rounded to float once.
#include <cmath>
#include <string>

#include "bca.h"
#include "bca_plan.h"

namespace bca {
bca_status set_error(bca_status s, const std::string& msg);  // bca_api.cpp
}

namespace {

constexpr int kSections[3] = {16, 56, 56};
constexpr int kPairs = 64;  // 128 dims / 2

// Integer square root of n if n is a perfect square, else -1.
int64_t exact_sqrt(int64_t n) {
  int64_t r = (int64_t)std::llround(std::sqrt((double)n));
  for (int64_t c = r > 1 ? r - 1 : 0; c <= r + 1; ++c)
    if (c * c == n) return c;
  return -1;
}

}  // namespace

extern "C" {

bca_status bca_rope_positions(const int32_t* block_ids, int64_t seq_len, const int32_t* image_hw,
                              int32_t n_images, int32_t* pos_out) {
  if (pos_out == nullptr) return bca::set_error(BCA_ERR_ARG, "pos_out is NULL");
  bca::HostPlan plan;
  std::string err;
  const int rc = bca::build_host_plan(block_ids, seq_len, 1, &plan, &err);
  if (rc != bca::kPlanOk)
    return bca::set_error(rc == bca::kPlanErrBlockIds ? BCA_ERR_BLOCK_IDS : BCA_ERR_ARG, err);
  int64_t images = 0;
  for (size_t r = 0; r < plan.segments.size(); r += 3)
    if (plan.segments[r + 2] >= 0) ++images;
  if (image_hw != nullptr && n_images != images)
    return bca::set_error(BCA_ERR_ARG, "image_hw lists " + std::to_string(n_images) +
                                           " images but the layout has " +
                                           std::to_string(images));
  int64_t c = 0, img = 0;
  for (size_t r = 0; r < plan.segments.size(); r += 3) {
    const int64_t a = plan.segments[r], e = plan.segments[r + 1];
    if (plan.segments[r + 2] < 0) {
      for (int64_t i = a; i < e; ++i, ++c)
        for (int ax = 0; ax < 3; ++ax) pos_out[3 * i + ax] = (int32_t)c;
      continue;
    }
    const int64_t n = e - a;
    int64_t H, W;
    if (image_hw != nullptr) {
      H = image_hw[2 * img];
      W = image_hw[2 * img + 1];
    } else {
      H = W = exact_sqrt(n);
    }
    if (H < 1 || W < 1 || H * W != n)
      return bca::set_error(BCA_ERR_ARG, "image block " + std::to_string(img) + " has " +
                                             std::to_string(n) + " positions, not H x W" +
                                             (image_hw ? "" : " with H = W"));
    for (int64_t t = 0; t < n; ++t) {
      pos_out[3 * (a + t)] = (int32_t)c;
      pos_out[3 * (a + t) + 1] = (int32_t)(t / W - H / 2);
      pos_out[3 * (a + t) + 2] = (int32_t)(t % W - W / 2);
    }
    ++c;
    ++img;
  }
  return BCA_OK;
}

bca_status bca_rope_table(const int32_t* pos, int64_t n, double base, float* table_out) {
  if (pos == nullptr || table_out == nullptr)
    return bca::set_error(BCA_ERR_ARG, "pos or table_out is NULL");
  if (n < 0) return bca::set_error(BCA_ERR_ARG, "n must be >= 0");
  if (!(base > 1.0) || std::isinf(base))
    return bca::set_error(BCA_ERR_ARG, "base must be finite and > 1");
  double inv[kPairs];
  int axis[kPairs];
  for (int ax = 0, p = 0; ax < 3; ++ax)
    for (int k = 0; k < kSections[ax] / 2; ++k, ++p) {
      inv[p] = std::pow(base, -2.0 * k / kSections[ax]);
      axis[p] = ax;
    }
  for (int64_t i = 0; i < n; ++i)
    for (int p = 0; p < kPairs; ++p) {
      const double ang = (double)pos[3 * i + axis[p]] * inv[p];
      table_out[(i * kPairs + p) * 2] = (float)std::cos(ang);
      table_out[(i * kPairs + p) * 2 + 1] = (float)std::sin(ang);
    }
  return BCA_OK;
}

}  // extern "C"
