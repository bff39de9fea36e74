// Prefix-cache format conversions for gfx950.  The FP8 cache stores E4M3 codes with one fp32
// scale per (token, head) (the 10100.com Qwen-Image 2.1 article, FP8 part).
//   cache_quantize: the prefill's prefix K/V rows written as codes and scales.  The prefill
//     kernel itself stores only the cache's bf16 tensors: quantising inside its key-tile loop
//     cost the loop registers it needs for its operand reads.
//   cache_dequant: a cache written back as bf16, once per layer, so that the cached step can run
//     the bf16 decode.  The value of a code is its E4M3 value times the row scale, a power of two,
//     which v_cvt_scalef32_pk_bf16_fp8 forms exactly (rounded to nearest even only below bf16's
//     normal range): the instruction the decode uses when it turns the codes into its bf16 tiles
//     in LDS, so both paths see bitwise the same K and V.
// Sixteen lanes per 128-value row, eight values per lane.  HBM-bound.
#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline u32x4 expand8(u32x2 c, float sc) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], sc, false);  // bytes 0, 1
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], sc, true);   // bytes 2, 3
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], sc, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// One tensor's chunk of row (b, p, h): 8 values at dims d0 .. d0 + 7.
__device__ inline u32x4 load8(const void* base, int64_t sb, int64_t ss, int64_t sh,
                              const float* sbase, int64_t ssb, int64_t sss, int64_t ssh, bool q,
                              int64_t b, int64_t p, int64_t h, int d0) {
  if (q) {
    const uint8_t* src = static_cast<const uint8_t*>(base) + b * sb + p * ss + h * sh + d0;
    const float sc = sbase[b * ssb + p * sss + h * ssh];
    return expand8(*reinterpret_cast<const u32x2*>(src), sc);
  }
  const uint16_t* src = static_cast<const uint16_t*>(base) + b * sb + p * ss + h * sh + d0;
  return *reinterpret_cast<const u32x4*>(src);
}

// Quantises this lane's 8 bf16 values of a 128-wide row held by 16 consecutive lanes (8 values
// each): the row's amax comes from a 16-lane max; the scale is 2^k, the smallest power of two
// with amax <= 448 * 2^k and k >= -126 (1 if amax is 0), and codes = E4M3(x * 2^-k), the product
// exact and the conversion round-to-nearest-even.  Returns the 8 codes; *scale_out gets the row
// scale.
__device__ inline u32x2 quantize_row8(u32x4 x, float* scale_out) {
  const bf16x8 xb = __builtin_bit_cast(bf16x8, x);
  float f[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i] = (float)xb[i];
    amax = fmaxf(amax, fabsf(f[i]));
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  // amax = 1.m * 2^e: 448 = 1.75 * 2^8, so k = e - 8, or e - 7 when 1.m > 1.75 (a subnormal
  // amax, exponent field 0, takes the floor)
  const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
  const int e = (int)(bits >> 23) - 127;
  int k = e - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  k = (bits >> 23) == 0 ? -126 : max(k, -126);
  const float scale = amax > 0.0f ? __builtin_bit_cast(float, (uint32_t)(k + 127) << 23) : 1.0f;
  const float inv = amax > 0.0f ? __builtin_bit_cast(float, (uint32_t)(127 - k) << 23) : 1.0f;
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv, f[1] * inv, 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv, f[3] * inv, w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * inv, f[5] * inv, 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * inv, f[7] * inv, w1, true);
  *scale_out = scale;
  return u32x2{(uint32_t)w0, (uint32_t)w1};
}

// One tensor's row chunk (b, p, h, d0 .. d0 + 7) quantised: codes to `out`, the row scale (from
// the row's first lane) to `sout`.
__device__ inline void quantize8(const uint16_t* src, int64_t sb, int64_t ss, int64_t sh,
                                 uint8_t* out, int64_t ob, int64_t os, int64_t oh, float* sout,
                                 int64_t sob, int64_t sos, int64_t soh, int64_t b, int64_t p,
                                 int64_t h, int d0, bool first_lane) {
  const u32x4 x = *reinterpret_cast<const u32x4*>(src + b * sb + p * ss + h * sh + d0);
  float sc;
  const u32x2 c = quantize_row8(x, &sc);
  *reinterpret_cast<u32x2*>(out + b * ob + p * os + h * oh + d0) = c;
  if (first_lane) sout[b * sob + p * sos + h * soh] = sc;
}

__global__ __launch_bounds__(256) void cache_quantize(const QuantArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= a.rows) return;  // whole 16-lane groups: the row max stays inside one group
  const int d0 = 8 * (threadIdx.x & 15);
  const bool first = (threadIdx.x & 15) == 0;
  const int64_t h = row % a.heads;
  const int64_t bp = row / a.heads;
  const int64_t p = bp % a.prefix;
  const int64_t b = bp / a.prefix;
  if (a.ko != nullptr)
    quantize8(a.k, a.k_sb, a.k_ss, a.k_sh, a.ko, a.ko_sb, a.ko_ss, a.ko_sh, a.ks, a.ks_sb,
              a.ks_ss, a.ks_sh, b, p, h, d0, first);
  if (a.vo != nullptr)
    quantize8(a.v, a.v_sb, a.v_ss, a.v_sh, a.vo, a.vo_sb, a.vo_ss, a.vo_sh, a.vs, a.vs_sb,
              a.vs_ss, a.vs_sh, b, p, h, d0, first);
}

__global__ __launch_bounds__(256) void cache_dequant(const DequantArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= a.rows) return;  // whole 16-lane groups; no cross-lane exchange
  const int d0 = 8 * (threadIdx.x & 15);
  const int64_t h = row % a.heads;
  const int64_t bp = row / a.heads;
  const int64_t p = bp % a.prefix;
  const int64_t b = bp / a.prefix;
  const bool kq = a.fmt == kCacheFp8KV, vq = a.fmt != kCacheBf16;
  const u32x4 kx = load8(a.k, a.k_sb, a.k_ss, a.k_sh, a.ks, a.ks_sb, a.ks_ss, a.ks_sh, kq, b, p, h, d0);
  const u32x4 vx = load8(a.v, a.v_sb, a.v_ss, a.v_sh, a.vs, a.vs_sb, a.vs_ss, a.vs_sh, vq, b, p, h, d0);
  *reinterpret_cast<u32x4*>(a.ko + b * a.ko_sb + p * a.ko_ss + h * a.ko_sh + d0) = kx;
  *reinterpret_cast<u32x4*>(a.vo + b * a.vo_sb + p * a.vo_ss + h * a.vo_sh + d0) = vx;
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 15) / 16;
  hipLaunchKernelGGL(cache_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 15) / 16;
  hipLaunchKernelGGL(cache_dequant, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bca
