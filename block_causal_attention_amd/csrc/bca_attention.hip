// Block-causal flash attention for gfx950 (MI355X): prefill (plan-driven) and prefix-cached
// decode (mask-free over [cache ; target]), plus the prefix-K/V copy.
//
// The rule ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section
// "Block-causal attention is the cache-enabling boundary") makes every mask row a prefix of the
// keys: row i sees exactly keys [0, hi(i)).  The planner turns that into, per tile of 128 query
// rows, a key bound below which no mask is needed (kv_full) and one past which no key is visible
// (kv_end); this kernel walks key tiles [0, kv_end), masks only the tiles that cross a row limit,
// and never loads the rest.  Decode is the same kernel with no mask except the sequence tail.
//
// Work decomposition.  One workgroup = 4 waves = one tile of 128 query rows of one (batch, head);
// wave w owns rows [32w, 32w + 32).  Per key tile of 64 keys:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q rows held in VGPRs.
//                 The accumulator layout gives each lane ONE query (lane % 32) and 16 keys, so the
//                 row max and row sum are in-lane reductions plus one swap of the two lane halves.
//   online softmax in base 2 with scale*log2(e) folded into one FMA per score; the running max is
//                 only raised (and O, l rescaled) when it grows by more than 8 (p <= 2^8 stays
//                 exact in fp32 and in bf16's exponent range), so most tiles skip the rescale.
//   O^T += V^T P^T  on the same MFMA: B = P^T straight from the score registers (bf16, RNE), A =
//                 V^T read from the row-major LDS tile with ds_read_b64_tr_b16, which hands each
//                 lane four consecutive keys of one column.  The key order inside one MFMA step
//                 is permuted identically in A and B, which leaves the sum unchanged.
// The O^T accumulator again has one query per lane, so the final 1/l is per lane.
#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKStride = kHeadDim + 8;   // bf16 per LDS K row: 272 B, rows 4 banks apart
constexpr int kVStride = kHeadDim + 16;  // bf16 per LDS V row: 288 B, rows 8 banks apart
constexpr int kChunksPerThread = kBlockN * kHeadDim / 8 / kThreads;  // 16-byte chunks per tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units
static_assert(kBlockM == 32 * kWaves, "one 32-row query block per wave");
static_assert(kBlockN == 64, "two 32-key MFMA blocks per key tile");

// Reduce across the two 32-lane halves of the wave: after v_permlane32_swap(x, x) every lane
// holds {x[lane % 32], x[lane % 32 + 32]} in the same order, so both halves get identical bits.
__device__ inline float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)s[0]), __builtin_bit_cast(float, (unsigned)s[1]));
}
__device__ inline float halves_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
}

template <bool kDecode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kBlockN * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[kBlockN * kVStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane holds
  const int qn = lane & 31;    // query column of this lane in the 32x32 accumulator

  // Workgroup -> (batch, head, query tile).  Workgroups are handed to the 8 XCDs round-robin
  // (id % 8), and each XCD has its own L2.  Re-index so that XCD x receives a contiguous run of
  // the (batch, head)-major work list: all query tiles of one head then run on one XCD at about
  // the same time and share that head's K/V tiles in its L2.  Within a head, tiles run in the
  // plan's heavy-first order.  (A remainder of fewer than 8 workgroups keeps its own index.)
  const int bh_count = a.batch * a.heads;
  const int total = a.n_qtiles * bh_count;
  const int full8 = total & ~7;
  int work = blockIdx.x;
  if (work < full8) work = (work & 7) * (full8 >> 3) + (work >> 3);
  const int bh = work / a.n_qtiles;
  const int slot = work - bh * a.n_qtiles;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int tile = kDecode ? slot : a.order[slot];
  const int kv_end = kDecode ? a.kv_len : a.kv_end[tile];
  const int kv_full = kDecode ? a.kv_len : a.kv_full[tile];

  // This lane's query row, its key limit, and its Q slice as eight MFMA B operands.
  const int row = tile * kBlockM + wave * 32 + qn;
  const bool row_ok = row < a.n_q;
  const int lim = kDecode ? a.kv_len : a.row_limit[row_ok ? row : a.n_q - 1];
  bf16x8 qreg[8];
  {
    const uint16_t* qp = a.q + b * a.q_sb + (int64_t)(row_ok ? row : 0) * a.q_ss + h * a.q_sh +
                         8 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 x = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * c) : u32x4{0, 0, 0, 0};
      qreg[c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> register staging of one K/V tile (keys >= kv_end are zero: never visible).
  u32x4 kst[kChunksPerThread], vst[kChunksPerThread];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r) {
      const int c = tid + r * kThreads;
      const int key = n0 + (c >> 4);
      const int col = (c & 15) * 8;
      if (key < kv_end) {
        const uint16_t* kp;
        const uint16_t* vp;
        if (!kDecode || key < a.split) {
          kp = a.k + b * a.k_sb + (int64_t)key * a.k_ss + h * a.k_sh + col;
          vp = a.v + b * a.v_sb + (int64_t)key * a.v_ss + h * a.v_sh + col;
        } else {
          const int64_t kk = key - a.split;
          kp = a.k2 + b * a.k2_sb + kk * a.k2_ss + h * a.k2_sh + col;
          vp = a.v2 + b * a.v2_sb + kk * a.v2_ss + h * a.v2_sh + col;
        }
        kst[r] = *reinterpret_cast<const u32x4*>(kp);
        vst[r] = *reinterpret_cast<const u32x4*>(vp);
      } else {
        kst[r] = u32x4{0, 0, 0, 0};
        vst[r] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r) {
      const int c = tid + r * kThreads;
      const int key = c >> 4;
      const int col = (c & 15) * 8;
      *reinterpret_cast<u32x4*>(&k_lds[key * kKStride + col]) = kst[r];
      *reinterpret_cast<u32x4*>(&v_lds[key * kVStride + col]) = vst[r];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x16{};
  float m_run = -__builtin_inff();  // running max of scale*log2(e)*s, same in both halves
  float l_part = 0.0f;              // this lane's share of the row sum (its 16 keys per block)
  const float c2 = a.scale_log2;

  // ds_read_b64_tr_b16 addressing: lane t of each 16-lane group points at row (t / 4) and
  // column 4 * (t % 4) of a 4 x 16 block; it receives that block's column t (4 rows).
  const int g = lane >> 4;
  const int tq = lane & 15;
  const int tr_row = 4 * half + (tq >> 2);
  const int tr_col = 16 * (g & 1) + 4 * (tq & 3);

  load_tile(0);
  for (int n0 = 0; n0 < kv_end; n0 += kBlockN) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (n0 + kBlockN < kv_end) load_tile(n0 + kBlockN);  // in flight during this tile's math

    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&k_lds[(32 * kb + qn) * kKStride + 16 * c + 8 * half]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], s[kb], 0, 0, 0);
      }
    }

    // ---- mask (only tiles that cross a row limit), row max
    // accumulator element i of block kb holds key n0 + 32 kb + 8 (i / 4) + 4 half + i % 4
    if (n0 + kBlockN > kv_full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = n0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key >= lim) s[kb][i] = -__builtin_inff();
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = halves_max(mx);

    // Each row raises its own max only when it grew by more than the threshold, so a row's
    // arithmetic depends on its own visible scores alone; the wave-uniform branch merely skips
    // the O rescale when no row of the wave needs one (rows that don't get alpha = 1 exactly).
    const float m_cand = fmaxf(m_run, mx * c2);
    const bool raise = m_cand > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_cand) : 1.0f;  // 0 at first
      m_run = raise ? m_cand : m_run;
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] *= alpha;
    }

    // ---- p = 2^(s * c2 - m), row sum, bf16 P^T operands (4 chunks of 16 keys)
    bf16x8 pb[4];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c2, -m_run));
        lsum += p;
        pb[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
      }
    l_part += lsum;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const __bf16* base = &v_lds[(16 * kc + tr_row) * kVStride + 32 * d + tr_col];
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * kVStride));
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], o[d], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O_acc / l; lane holds dims 32 d + 8 j + 4 half + (0..3) of its query
  const float inv = 1.0f / halves_sum(l_part);
  if (row_ok) {
    float* op = a.o + b * a.o_sb + (int64_t)row * a.o_ss + h * a.o_sh + 4 * half;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 val = {o[d][4 * j] * inv, o[d][4 * j + 1] * inv, o[d][4 * j + 2] * inv,
                           o[d][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(op + 32 * d + 8 * j) = val;
      }
  }
}

// Prefix-K/V store: dst[b, j, h, :] = src[b, j, h, :] for j < rows, both K and V, 16 B per thread.
__global__ __launch_bounds__(256) void prefix_copy(const CopyArgs k, const CopyArgs v) {
  const int64_t per_row = (int64_t)k.heads * (kHeadDim / 8);
  const int64_t total = (int64_t)k.batch * k.rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)(i % (kHeadDim / 8)) * 8;
    const int64_t r = i / (kHeadDim / 8);
    const int hh = (int)(r % k.heads);
    const int64_t bj = r / k.heads;
    const int64_t j = bj % k.rows;
    const int64_t bb = bj / k.rows;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(k.src + bb * k.s_sb + j * k.s_ss + hh * k.s_sh + col);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(v.src + bb * v.s_sb + j * v.s_ss + hh * v.s_sh + col);
    *reinterpret_cast<u32x4*>(k.dst + bb * k.d_sb + j * k.d_ss + hh * k.d_sh + col) = kx;
    *reinterpret_cast<u32x4*>(v.dst + bb * v.d_sb + j * v.d_ss + hh * v.d_sh + col) = vx;
  }
}

}  // namespace

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.n_qtiles * a.batch * a.heads);
  hipLaunchKernelGGL(attn_fwd<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.n_qtiles * a.batch * a.heads);
  hipLaunchKernelGGL(attn_fwd<true>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefix_copy(const CopyArgs& k, const CopyArgs& v, hipStream_t stream) {
  const int64_t total = (int64_t)k.batch * k.rows * k.heads * (kHeadDim / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(prefix_copy, dim3((unsigned)blocks), dim3(256), 0, stream, k, v);
  return hipGetLastError();
}

}  // namespace bca
