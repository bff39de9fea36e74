// Block-causal flash attention for gfx950 (MI355X): prefill (plan-driven) and prefix-cached
// decode (mask-free over [cache ; target]); the prefill also writes the prefix-K/V cache.
//
// The rule ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section
// "Block-causal attention is the cache-enabling boundary") makes every mask row a prefix of the
// keys: row i sees exactly keys [0, hi(i)).  The planner turns that into, per tile of kBlockM
// query rows, a key bound below which no mask is needed (kv_full) and one past which no key is
// visible (kv_end); this kernel walks key tiles [0, kv_end), masks only the tiles that cross a
// row limit, and never loads the rest.  Decode is the same kernel with no mask except the tail.
//
// Work decomposition.  One workgroup = kWaves waves = one tile of kBlockM query rows of one
// (batch, head); a wave owns kQueryBlocks blocks of 32 rows.  Per key tile of kBlockN keys:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q rows held in VGPRs.
//                 The accumulator gives each lane ONE query (lane % 32) and 16 keys, so the row
//                 max is an in-lane reduction plus one swap of the two 32-lane halves.
//   online softmax in base 2 with scale*log2(e) folded into one FMA per score; a row's running
//                 max is raised (and its O and l rescaled) only when it grew by more than 8
//                 (p <= 2^8 is exact in fp32 and within bf16's range), so most tiles skip it.
//                 The row sum accumulates the bf16-rounded p (the values PV uses) two at a time
//                 with v_dot2_f32_bf16 against (1, 1).
//   O^T += V^T P^T  on the same MFMA: B = P^T straight from the score registers (bf16, RNE), A =
//                 V^T read from the row-major LDS tile with ds_read_b64_tr_b16, which hands each
//                 lane four consecutive keys of one column.  The key order inside one MFMA step
//                 is permuted identically in A and B, which leaves the sum unchanged.
// Pipeline.  K runs one tile ahead of V in a two-buffer LDS ring: while a wave turns tile j's
// scores into P and multiplies by V(j), it already issues the MFMAs for tile j+1's scores, so
// matrix and vector work of the same wave can overlap.  Global loads for the tiles after that
// are in flight during the whole iteration (register staging); one barrier per tile.
#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

#ifndef BCA_WAVES_PER_SIMD
#define BCA_WAVES_PER_SIMD (kQueryBlocks == 1 ? 2 : 1)
#endif
constexpr int kThreads = 64 * kWaves;
constexpr int kOccupancy = BCA_WAVES_PER_SIMD;
constexpr int kKStride = kHeadDim + 8;   // bf16 per LDS K row: 272 B, rows 4 banks apart
#ifndef BCA_V_PAD
#define BCA_V_PAD 16
#endif
constexpr int kVStride = kHeadDim + BCA_V_PAD;  // bf16 per LDS V row
constexpr int kChunks = kBlockN * kHeadDim / 8;  // 16-byte chunks per K (or V) tile
constexpr int kChunksPerThread = kChunks / kThreads;
constexpr int kRowsPerPass = kThreads / 16;      // tile rows covered by one pass of the group
constexpr float kRescaleThreshold = 8.0f;        // log2 units
// With one 32-row block per wave, the next tile's scores are computed while this tile's softmax
// runs (K one tile ahead of V).  With two blocks there are not enough registers for a second
// score tile, and the tiles run one after the other through a plain double buffer.
#ifndef BCA_SCHED_INTERLEAVE
#define BCA_SCHED_INTERLEAVE 0
#endif
#ifndef BCA_SCORES_AHEAD
#define BCA_SCORES_AHEAD (kQueryBlocks == 1)
#endif
constexpr bool kScoresAhead = BCA_SCORES_AHEAD;
constexpr int kKeyBlocks = kBlockN / 32;  // 32-key MFMA blocks per key tile
static_assert(kBlockN == 32 || kBlockN == 64, "one or two 32-key MFMA blocks per key tile");
static_assert(kChunks % kThreads == 0, "whole 16-byte chunks per thread");

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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kOccupancy, kOccupancy)))
void attn_fwd(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kBlockN * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kBlockN * kVStride];

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
  const int ntiles = (kv_end + kBlockN - 1) / kBlockN;

  // This lane's query rows, their key limits, and their Q slices as MFMA B operands.
  int lim[kQueryBlocks];
  bool row_ok[kQueryBlocks];
  bf16x8 qreg[kQueryBlocks][8];
#pragma unroll
  for (int qb = 0; qb < kQueryBlocks; ++qb) {
    const int row = tile * kBlockM + (wave * kQueryBlocks + qb) * 32 + qn;
    row_ok[qb] = row < a.n_q;
    lim[qb] = kDecode ? a.kv_len : a.row_limit[row_ok[qb] ? row : a.n_q - 1];
    const uint16_t* qp =
        a.q + b * a.q_sb + (int64_t)(row_ok[qb] ? row : 0) * a.q_ss + h * a.q_sh + 8 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 x =
          row_ok[qb] ? *reinterpret_cast<const u32x4*>(qp + 16 * c) : u32x4{0, 0, 0, 0};
      qreg[qb][c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- global -> register staging of K or V tiles ------------------------------------------
  // Thread t moves the 16-byte chunk at column 8 (t % 16) of tile rows t / 16 + kRowsPerPass r.
  const int ld_row = tid >> 4;
  const int ld_col = (tid & 15) * 8;
  const uint16_t* k_base = a.k + b * a.k_sb + h * a.k_sh + ld_col;
  const uint16_t* v_base = a.v + b * a.v_sb + h * a.v_sh + ld_col;
  const uint16_t* k2_base = a.k2 + b * a.k2_sb + h * a.k2_sh + ld_col;
  const uint16_t* v2_base = a.v2 + b * a.v2_sb + h * a.v2_sh + ld_col;
  const int64_t k_row_off = (int64_t)ld_row * a.k_ss;
  const int64_t v_row_off = (int64_t)ld_row * a.v_ss;
  const int64_t k2_row_off = (int64_t)ld_row * a.k2_ss;
  const int64_t v2_row_off = (int64_t)ld_row * a.v2_ss;

  // Loads one tile (K or V) starting at key n0; keys >= kv_end read as zero.  The common case
  // (whole tile from one source, nothing past kv_end) uses a tile-uniform base plus a per-thread
  // offset; only a tile that straddles the cache/target split or the end resolves each row.
  auto load_tile = [&](int n0, u32x4 (&st)[kChunksPerThread], const uint16_t* base1,
                       int64_t ss1, int64_t off1, const uint16_t* base2, int64_t ss2,
                       int64_t off2) {
    const bool in_end = n0 + kBlockN <= kv_end;
    if (in_end && (!kDecode || n0 + kBlockN <= a.split)) {
      const uint16_t* t = base1 + (int64_t)n0 * ss1 + off1;
#pragma unroll
      for (int r = 0; r < kChunksPerThread; ++r)
        st[r] = *reinterpret_cast<const u32x4*>(t + (int64_t)(kRowsPerPass * r) * ss1);
    } else if (kDecode && in_end && n0 >= a.split) {
      const uint16_t* t = base2 + (int64_t)(n0 - a.split) * ss2 + off2;
#pragma unroll
      for (int r = 0; r < kChunksPerThread; ++r)
        st[r] = *reinterpret_cast<const u32x4*>(t + (int64_t)(kRowsPerPass * r) * ss2);
    } else {
#pragma unroll
      for (int r = 0; r < kChunksPerThread; ++r) {
        const int key = n0 + ld_row + kRowsPerPass * r;
        const bool valid = key < kv_end;
        const int kc = valid ? key : kv_end - 1;
        const bool first = !kDecode || kc < a.split;
        const uint16_t* p =
            first ? base1 + (int64_t)kc * ss1 : base2 + (int64_t)(kc - a.split) * ss2;
        const u32x4 x = *reinterpret_cast<const u32x4*>(p);
        st[r] = valid ? x : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto load_k = [&](int n0, u32x4 (&st)[kChunksPerThread]) {
    load_tile(n0, st, k_base, a.k_ss, k_row_off, k2_base, a.k2_ss, k2_row_off);
  };
  auto load_v = [&](int n0, u32x4 (&st)[kChunksPerThread]) {
    load_tile(n0, st, v_base, a.v_ss, v_row_off, v2_base, a.v2_ss, v2_row_off);
  };
  // Prefix-K/V cache (prefill only): this workgroup owns cache rows [cache_lo, cache_hi), which
  // lie inside its own diagonal key tiles, so they are stored from the staging registers as
  // those tiles pass through; no K/V row is read twice for the cache.
  const int cache_lo = tile * kBlockM;
  const int cache_hi = kDecode || a.kc == nullptr ? 0 : min(cache_lo + kBlockM, a.cache_len);
  auto store_cache = [&](int n0, const u32x4 (&st)[kChunksPerThread], uint16_t* base,
                         int64_t sb, int64_t ss, int64_t sh) {
    if (kDecode || n0 >= cache_hi || n0 + kBlockN <= cache_lo) return;
    uint16_t* p = base + b * sb + h * sh + ld_col;
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r) {
      const int key = n0 + ld_row + kRowsPerPass * r;
      if (key >= cache_lo && key < cache_hi)
        *reinterpret_cast<u32x4*>(p + (int64_t)key * ss) = st[r];
    }
  };
  auto store_k = [&](int buf, int n0, const u32x4 (&st)[kChunksPerThread]) {
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r)
      *reinterpret_cast<u32x4*>(&k_lds[buf][(ld_row + kRowsPerPass * r) * kKStride + ld_col]) =
          st[r];
    store_cache(n0, st, a.kc, a.kc_sb, a.kc_ss, a.kc_sh);
  };
  auto store_v = [&](int buf, int n0, const u32x4 (&st)[kChunksPerThread]) {
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r)
      *reinterpret_cast<u32x4*>(&v_lds[buf][(ld_row + kRowsPerPass * r) * kVStride + ld_col]) =
          st[r];
    store_cache(n0, st, a.vc, a.vc_sb, a.vc_ss, a.vc_sh);
  };

  // ---- S^T = K Q^T for the 32-key blocks of the K tile in buffer buf ------------------
  auto scores = [&](int buf, f32x16 (&s)[kQueryBlocks][kKeyBlocks]) {
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb) {
#pragma unroll
      for (int qb = 0; qb < kQueryBlocks; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
            &k_lds[buf][(32 * kb + qn) * kKStride + 16 * c + 8 * half]);
#pragma unroll
        for (int qb = 0; qb < kQueryBlocks; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], s[qb][kb], 0, 0, 0);
      }
    }
  };

  f32x16 o[kQueryBlocks][4];
  float m_run[kQueryBlocks];   // running max of scale*log2(e)*s (same in both lane halves)
  float l_part[kQueryBlocks];  // this lane's share of the row sum
#pragma unroll
  for (int qb = 0; qb < kQueryBlocks; ++qb) {
#pragma unroll
    for (int d = 0; d < 4; ++d) o[qb][d] = f32x16{};
    m_run[qb] = -__builtin_inff();
    l_part[qb] = 0.0f;
  }
  const float c2 = a.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ds_read_b64_tr_b16 addressing: lane t of each 16-lane group points at row (t / 4) and
  // column 4 * (t % 4) of a 4 x 16 block; it receives that block's column t (4 rows).
  const int g = lane >> 4;
  const int tq = lane & 15;
  const int tr_row = 4 * half + (tq >> 2);
  const int tr_col = 16 * (g & 1) + 4 * (tq & 3);

  // ---- prologue --------------------------------------------------------------------------
  u32x4 kst[kChunksPerThread], vst[kChunksPerThread];
  f32x16 s_cur[kQueryBlocks][kKeyBlocks];
  if constexpr (kScoresAhead) {
    // K(0), V(0), K(1) into LDS; K(2) and V(1) in flight; scores of tile 0
    load_k(0, kst);
    load_v(0, vst);
    store_k(0, 0, kst);
    store_v(0, 0, vst);
    if (ntiles > 1) {
      load_k(kBlockN, kst);
      store_k(1, kBlockN, kst);
    }
    if (ntiles > 2) load_k(2 * kBlockN, kst);
    if (ntiles > 1) load_v(kBlockN, vst);
    __syncthreads();
    scores(0, s_cur);
    __syncthreads();  // every wave has read K(0) before its buffer is refilled
  } else {
    // tile 0 into LDS buffer 0; tile 1 in flight
    load_k(0, kst);
    load_v(0, vst);
    store_k(0, 0, kst);
    store_v(0, 0, vst);
    if (ntiles > 1) {
      load_k(kBlockN, kst);
      load_v(kBlockN, vst);
    }
    __syncthreads();
  }

  for (int j = 0; j < ntiles; ++j) {
    const int n0 = j * kBlockN;
    if constexpr (!kScoresAhead) scores(j & 1, s_cur);


    // mask: only tiles that cross some row's limit.  Accumulator element i of key block kb
    // holds key n0 + 32 kb + 8 (i / 4) + 4 half + i % 4.
    if (n0 + kBlockN > kv_full) {
#pragma unroll
      for (int qb = 0; qb < kQueryBlocks; ++qb)
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = n0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key >= lim[qb]) s_cur[qb][kb][i] = -__builtin_inff();
          }
    }

    // row max; each row raises its own running max only when it grew by more than the
    // threshold, so a row's arithmetic depends on its own visible scores alone.  The branch is
    // wave-uniform and merely skips the O rescale when no row of the wave needs one.
#pragma unroll
    for (int qb = 0; qb < kQueryBlocks; ++qb) {
      float mx = s_cur[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[qb][kb][i]);
      mx = halves_max(mx);
      const float m_cand = fmaxf(m_run[qb], mx * c2);
      const bool raise = m_cand > m_run[qb] + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[qb] - m_cand) : 1.0f;  // 0 at first
        m_run[qb] = raise ? m_cand : m_run[qb];
        l_part[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d) o[qb][d] *= alpha;
      }
    }

    // scores of the next tile (its K is already in LDS); independent of the softmax below.
    // On the last tile this reads a stale buffer and the result is discarded.
    f32x16 s_nxt[kQueryBlocks][kKeyBlocks];
    if constexpr (kScoresAhead) scores((j + 1) & 1, s_nxt);

    // p = 2^(s c2 - m) as bf16 P^T operands (chunks of 16 keys), row sums
    bf16x8 pb[kQueryBlocks][2 * kKeyBlocks];
#pragma unroll
    for (int qb = 0; qb < kQueryBlocks; ++qb) {
      const float mneg = -m_run[qb];
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[qb][kb][i], c2, mneg));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[qb][kb][i + 1], c2, mneg));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          pb[qb][2 * kb + (i >> 3)][i & 7] = pp[0];
          pb[qb][2 * kb + (i >> 3)][(i & 7) + 1] = pp[1];
          if (i & 2)
            acc1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc1, false);
          else
            acc0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc0, false);
        }
      l_part[qb] += acc0 + acc1;
    }

    // O^T += V^T P^T with V(j) from buffer j & 1
    const int vb = j & 1;
#pragma unroll
    for (int kc = 0; kc < 2 * kKeyBlocks; ++kc) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const __bf16* base = &v_lds[vb][(16 * kc + tr_row) * kVStride + 32 * d + tr_col];
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * kVStride));
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int qb = 0; qb < kQueryBlocks; ++qb)
          o[qb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb][kc], o[qb][d], 0, 0, 0);
      }
    }

#if BCA_SCHED_INTERLEAVE
    if constexpr (kScoresAhead && kQueryBlocks == 1 && kBlockN == 64) {
      // Interleave, within this wave, the next tile's K reads and QK^T MFMAs with this tile's
      // softmax arithmetic, then the V reads with the PV MFMAs (masks: 0x100 LDS read,
      // 0x008 MFMA, 0x002 VALU).
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 14; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
    }
#endif
    if constexpr (kScoresAhead) {
      // refill: K(j+2) replaces K(j), V(j+1) replaces V(j-1); then start the next loads
      if (j + 2 < ntiles) store_k(j & 1, (j + 2) * kBlockN, kst);
      if (j + 1 < ntiles) store_v((j + 1) & 1, (j + 1) * kBlockN, vst);
      if (j + 3 < ntiles) load_k((j + 3) * kBlockN, kst);
      if (j + 2 < ntiles) load_v((j + 2) * kBlockN, vst);
    } else {
      // refill: tile j+1 replaces tile j-1; then start loading tile j+2
      if (j + 1 < ntiles) {
        store_k((j + 1) & 1, (j + 1) * kBlockN, kst);
        store_v((j + 1) & 1, (j + 1) * kBlockN, vst);
      }
      if (j + 2 < ntiles) {
        load_k((j + 2) * kBlockN, kst);
        load_v((j + 2) * kBlockN, vst);
      }
    }
    __syncthreads();
    if constexpr (kScoresAhead) {
#pragma unroll
      for (int qb = 0; qb < kQueryBlocks; ++qb)
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb) s_cur[qb][kb] = s_nxt[qb][kb];
    }
  }

  // ---- epilogue: O = O_acc / l; lane holds dims 32 d + 8 jj + 4 half + (0..3) of its query
#pragma unroll
  for (int qb = 0; qb < kQueryBlocks; ++qb) {
    const float inv = 1.0f / halves_sum(l_part[qb]);
    if (row_ok[qb]) {
      const int row = tile * kBlockM + (wave * kQueryBlocks + qb) * 32 + qn;
      float* op = a.o + b * a.o_sb + (int64_t)row * a.o_ss + h * a.o_sh + 4 * half;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 val = {o[qb][d][4 * jj] * inv, o[qb][d][4 * jj + 1] * inv,
                             o[qb][d][4 * jj + 2] * inv, o[qb][d][4 * jj + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * d + 8 * jj) = val;
        }
    }
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

}  // namespace bca
