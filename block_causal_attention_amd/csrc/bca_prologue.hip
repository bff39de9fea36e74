// Q/K prologue for gfx950: per-head RMS normalisation followed by three-axis RoPE, one pass over
// Q and K in HBM ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo": section
// "One stream for text, reference images, and the target" normalises Q and K per head before
// RoPE; section "Three-axis RoPE preserves image geometry" gives the rotation).
//
// Sixteen consecutive lanes own one 128-value head row, lane l holding dims 8l .. 8l + 7, which
// are the adjacent rotation pairs 4l .. 4l + 3.  The mean square is a 16-lane reduction; the
// rotation needs no exchange.  Arithmetic is fp32 (correctly rounded sqrt and divide), the
// result is rounded to bf16 (RNE).  The work is one read and one write of Q and K: HBM-bound.
#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerBlock = 16;  // 256 threads, 16 lanes per head row

// Normalises and rotates this lane's 8 values x of one head row.  w: the lane's 8 weights;
// cs: {cos, sin} of its 4 pairs.  Every lane of the row must call it (16-lane reduction).
__device__ inline u32x4 norm_rope8(u32x4 raw, const float* w, const float* cs, float eps) {
  const bf16x8 xb = __builtin_bit_cast(bf16x8, raw);
  float x[8];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (float)xb[i];
    ss = __builtin_fmaf(x[i], x[i], ss);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
  bf16x8 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float y0 = x[2 * p] * inv * w[2 * p];
    const float y1 = x[2 * p + 1] * inv * w[2 * p + 1];
    const float c = cs[2 * p], s = cs[2 * p + 1];
    out[2 * p] = (__bf16)(y0 * c - y1 * s);
    out[2 * p + 1] = (__bf16)(y0 * s + y1 * c);
  }
  return __builtin_bit_cast(u32x4, out);
}

__global__ __launch_bounds__(256) void qk_prologue(const PrologueArgs a) {
  const int lane16 = threadIdx.x & 15;
  const int64_t row_raw = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const bool live = row_raw < a.rows;        // uniform over the row's 16 lanes
  const int64_t row = live ? row_raw : a.rows - 1;
  const int h = (int)(row % a.heads);
  const int64_t bs = row / a.heads;
  const int s = (int)(bs % a.seq);
  const int64_t b = bs / a.seq;
  const int d0 = 8 * lane16;

  float cs[8], wq[8], wk[8];
  const f32x4* tp = reinterpret_cast<const f32x4*>(a.table + ((int64_t)s * 64 + 4 * lane16) * 2);
  const f32x4* wqp = reinterpret_cast<const f32x4*>(a.wq + d0);
  const f32x4* wkp = reinterpret_cast<const f32x4*>(a.wk + d0);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const f32x4 t = tp[j], u = wqp[j], v = wkp[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cs[4 * j + i] = t[i];
      wq[4 * j + i] = u[i];
      wk[4 * j + i] = v[i];
    }
  }
  const u32x4 qraw = *reinterpret_cast<const u32x4*>(a.q + b * a.q_sb + s * a.q_ss + h * a.q_sh + d0);
  const u32x4 kraw = *reinterpret_cast<const u32x4*>(a.k + b * a.k_sb + s * a.k_ss + h * a.k_sh + d0);
  const u32x4 qn = norm_rope8(qraw, wq, cs, a.eps);
  const u32x4 kn = norm_rope8(kraw, wk, cs, a.eps);
  if (live) {
    *reinterpret_cast<u32x4*>(a.qo + b * a.qo_sb + s * a.qo_ss + h * a.qo_sh + d0) = qn;
    *reinterpret_cast<u32x4*>(a.ko + b * a.ko_sb + s * a.ko_ss + h * a.ko_sh + d0) = kn;
  }
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(qk_prologue, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bca
