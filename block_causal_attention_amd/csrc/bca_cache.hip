// Prefix-cache expansion for gfx950: a cache stored as FP8 E4M3 codes with one fp32 scale per
// (token, head) (the 10100.com Qwen-Image 2.1 article, FP8 part) written back as bf16, once per
// layer, so that the cached step can run the bf16 decode.  The value of a code is its E4M3 value
// times the row scale, formed in fp32 and rounded to bf16 (RNE): the same rule the decode applies
// when it dequantises while staging, so both paths see bitwise the same K and V.
//
// Sixteen lanes per 128-value row, eight values per lane: 8 code bytes (or 16 bf16 bytes) in,
// 16 bytes out.  HBM-bound.
#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline u32x4 expand8(u32x2 c, float sc) {
  const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[0], false);  // bytes 0, 1
  const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[0], true);   // bytes 2, 3
  const auto p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[1], false);
  const auto p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[1], true);
  const bf16x8 r = {(__bf16)(p0[0] * sc), (__bf16)(p0[1] * sc), (__bf16)(p1[0] * sc),
                    (__bf16)(p1[1] * sc), (__bf16)(p2[0] * sc), (__bf16)(p2[1] * sc),
                    (__bf16)(p3[0] * sc), (__bf16)(p3[1] * sc)};
  return __builtin_bit_cast(u32x4, r);
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

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.rows + 15) / 16;
  hipLaunchKernelGGL(cache_dequant, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bca
