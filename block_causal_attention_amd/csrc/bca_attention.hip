// Block-causal flash attention for gfx950 (MI355X): prefill (plan-driven) and prefix-cached
// decode (mask-free over [cache ; target]); the prefill also writes the prefix-K/V cache's bf16
// tensors (an FP8 cache's quantised ones come from cache_quantize, bca_cache.hip).
//
// The rule ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section
// "Block-causal attention is the cache-enabling boundary") makes every mask row a prefix of the
// keys: row i sees exactly keys [0, hi(i)).  The planner turns that into, per query tile (the
// prefill's workgroup), a key bound below which no mask is needed (kv_full) and one past which
// no key is visible (kv_end); this kernel walks key tiles [0, kv_end), masks only the tiles that
// cross a row limit, and never loads the rest.  Decode is the same kernel with no mask except
// the tail.
//
// Work decomposition.  One workgroup = kW waves = one tile of 32 kW query rows of one (batch,
// head); a wave owns kQueryBlocks blocks of 32 rows.  The prefill and the decode run 12 waves
// (384 rows, one workgroup per CU at 3 waves per SIMD, so each K/V tile in LDS serves 384 rows;
// a small decode grid runs 4).  Per key tile of kBlockN = 32 keys:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = Q rows held in VGPRs.
//                 The accumulator gives each lane ONE query (lane % 32) and 16 keys, so the row
//                 max is an in-lane reduction plus one swap of the two 32-lane halves.
//   online softmax in base 2 with scale*log2(e) folded into one FMA per score.  p is computed
//                 against the running max of earlier tiles; a row's max is raised (and its O, l
//                 rescaled) only when its scores grew by more than 16, which shows up as a lane's
//                 tile sum above 2^16 and sends the wave through an exact recompute.  So the
//                 common tile needs no max reduction at all.  The row sum accumulates the
//                 bf16-rounded p (the values PV uses) two at a time with v_dot2_f32_bf16.
//   O^T += V^T P^T  on the same MFMA: B = P^T straight from the score registers (bf16, RNE), A =
//                 V^T read from the row-major LDS tile with ds_read_b64_tr_b16, which hands each
//                 lane four consecutive keys of one column.  The key order inside one MFMA step
//                 is permuted identically in A and B, which leaves the sum unchanged.
// K/V tiles go through a two-buffer LDS ring with one barrier per tile: tile j+1 is in flight
// while tile j is computed.  The ring is filled by direct loads: buffer_load_dwordx4 ... lds
// writes 1 KB (4 rows) straight into LDS per instruction, the tile's fills dealt round-robin over
// the waves, with a fixed per-lane offset and the tile's position in the descriptor.  Rows are
// unpadded, with an XOR swizzle of their 16-byte chunks (below) that keeps the K reads and the
// transposed V reads free of bank conflicts.  An FP8 prefix cache's code bytes and row scales
// come in the same way, two tiles ahead, and are turned into the bf16 tile in LDS.
#include <atomic>
#include <mutex>
#include <queue>
#include <vector>
#include <algorithm>
#include <type_traits>

#include "bca_internal.h"

namespace bca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// While a wave issues its score or PV MFMAs it runs at raised priority, so the SIMD's arbiter
// prefers waves that can feed the matrix core and the others fill the gaps with softmax work.
// Measured per kernel (interleaved A/B): +2% for the prefill; the decode's 12-wave kernel runs 4%
// faster without it, and its 8-wave tail kernel 2%.
constexpr int kMfmaPrio = 1;
constexpr int kDecodeDirectMfmaPrio = 0;
// Reads kept in flight ahead of the MFMAs (in steps of one MFMA) in the score and PV phases.
// Measured (interleaved A/B, 12-wave kernels): 3 and 4 give the prefill +2.7% and the decode
// +0.5% over the compiler's own order; 2 and 2 or 2 and 4 the same within noise; 4 and 6 less on
// the prefill.
constexpr int kSchedKDepth = 3;
constexpr int kSchedVDepth = 4;

// A row's running max is raised only when its scores grew by more than kRescaleThreshold (log2
// units), so p <= 2^16: exact in fp32, within bf16's exponent range, and l, O stay far below
// fp32 overflow.  A lane's tile sum above kRescaleBound is what sends a wave to the exact path.
constexpr float kRescaleThreshold = 16.0f;
constexpr float kRescaleBound = 65536.0f;
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format; range-checked
// against num_records with stride 0).
constexpr int kBufferWord3 = 0x00020000;

// Swizzle of direct-load tiles: the 16-byte chunk c of tile row r sits at chunk c ^ swz(r).
// swz is a bijection on each 16 consecutive rows (K reads: 16 lanes, 16 rows, one logical chunk
// -> 16 distinct chunks) and sends the 4-chunk group of one 32-column block in 4 aligned rows to
// 4 distinct groups (transposed V reads: 32 lanes read 4 rows x 64 B).
__device__ inline int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Scheduling of one MFMA phase: kSteps steps, each kReads LDS operand reads feeding kMfmas
// MFMAs.  With kDepth > 0 the reads of step i + kDepth are issued right after step i's MFMAs,
// so kDepth steps' reads are always in flight ahead of their MFMAs (instead of the order the
// compiler's scheduler picks, which in some loop shapes waits for each read right before its
// MFMA).  Placed after the phase's code, in the same basic block.
template <int kSteps, int kReads, int kMfmas, int kDepth>
__device__ __forceinline__ void pipeline_reads() {
  if constexpr (kDepth > 0) {
    constexpr int kMfmaMask = 0x008, kDsReadMask = 0x100;
    constexpr int kLead = kDepth < kSteps ? kDepth : kSteps;
    __builtin_amdgcn_sched_group_barrier(kDsReadMask, kReads * kLead, 0);
#pragma unroll
    for (int i = 0; i + kLead < kSteps; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfmaMask, kMfmas, 0);
      __builtin_amdgcn_sched_group_barrier(kDsReadMask, kReads, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfmaMask, kMfmas * kLead, 0);
  }
}

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

// FP8 prefix cache (E4M3, one fp32 scale per (token, head) row, a power of two; the exact rule is
// in bca.h).  dequant turns {8 code bytes of a row, its scale bits, 0} into the 8 bf16 values
// E4M3(code) * scale that the LDS tile holds: v_cvt_scalef32_pk_bf16_fp8 forms each pair exactly
// (a power-of-two scale only moves the exponent).
__device__ inline u32x4 dequant(u32x4 x) {
  // (the element goes through a scalar first: hipcc lowers a bit_cast of an ext_vector element
  // operand to a cast of element 0)
  const uint32_t sc_bits = x[2];
  const float sc = __builtin_bit_cast(float, sc_bits);
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[0], sc, false);  // bytes 0, 1
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[0], sc, true);   // bytes 2, 3
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[1], sc, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[1], sc, true);
  return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
               __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// The body of all the kernels.  kBlockN keys per key tile and kW waves per workgroup are chosen
// per kernel, and so is the occupancy (set on the kernels below).
template <bool kDecode, int kFmt, int kBlockN, int kW>
__device__ __forceinline__ void attn_fwd(const AttnArgs& a) {
  constexpr int kThreads = 64 * kW;
  constexpr int kRows = 32 * kQueryBlocks * kW;  // query rows per workgroup
  constexpr int kRowsPerPass = kThreads / 16;    // cache copy: rows per pass
  constexpr int kKeyBlocks = kBlockN / 32;       // 32-key MFMA blocks
  // cache copy: 16-byte chunks per thread (the last pass may be partial)
  constexpr int kChunksPerThread = (kBlockN * kHeadDim / 8 + kThreads - 1) / kThreads;
  static_assert(kBlockN == 32 || kBlockN == 64, "one or two 32-key MFMA blocks per key tile");
  // cache-copy passes past the tile's rows (a partial last pass) store nothing
  constexpr bool kPartialPass = kBlockN * kHeadDim / 8 % kThreads != 0;
  // The decode may read a quantised cache (its first key source); the prefill stores bf16 only.
  static_assert(kDecode || kFmt == kCacheBf16, "the prefill stores the cache's bf16 tensors");
  // wave priority while issuing MFMAs (0: never raised)
  constexpr int kPrioLevel =
      kDecode && (kW == kDecodeDirectWaves || kW == kDecodeTailWaves) ? kDecodeDirectMfmaPrio
                                                                      : kMfmaPrio;
  constexpr bool kPrio = kPrioLevel > 0;
  constexpr bool kKqSrc = kDecode && kFmt == kCacheFp8KV;
  constexpr bool kVqSrc = kDecode && kFmt != kCacheBf16;
  // A decode over a quantised cache brings the code bytes and row scales of the cache rows into
  // LDS as they are and turns them into the bf16 tile in LDS (convert below).
  constexpr bool kDirectQ = kKqSrc || kVqSrc;
  // LDS rows: unpadded (256 B) with their 16-byte chunks swizzled.
  constexpr int kKStride = kHeadDim;
  constexpr int kVStride = kHeadDim;
  // The two ring buffers, in separate arrays named by a constant (the tile loop is unrolled by
  // two below): reads of one are then provably independent of the direct loads in flight into the
  // other, so the compiler adds no vmcnt wait before them (the ring's own waits and barrier order
  // the buffers).  `buf` is a std::integral_constant.
  __shared__ __attribute__((aligned(16))) __bf16 k_lds0[kBlockN * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 k_lds1[kBlockN * kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds0[kBlockN * kVStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds1[kBlockN * kVStride];
  auto k_lds = [](auto buf) -> __bf16* { return decltype(buf)::value ? k_lds1 : k_lds0; };
  auto v_lds = [](auto buf) -> __bf16* { return decltype(buf)::value ? v_lds1 : v_lds0; };
  // Decode over a quantised cache: a two-tile ring of code bytes (row-major, 128 B a row) and
  // row scales per quantised tensor, next to the bf16 ring the MFMAs read.
  constexpr int kCodeBytes = kDirectQ ? kBlockN * kHeadDim : 16;
  __shared__ __attribute__((aligned(16))) uint8_t kcode0[kKqSrc ? kCodeBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t kcode1[kKqSrc ? kCodeBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t vcode0[kCodeBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vcode1[kCodeBytes];
  __shared__ __attribute__((aligned(16))) float kscl0[64], kscl1[64], vscl0[64], vscl1[64];
  auto code_lds = [](bool v, auto buf) -> uint8_t* {
    return decltype(buf)::value ? (v ? vcode1 : kcode1) : (v ? vcode0 : kcode0);
  };
  auto scl_lds = [](bool v, auto buf) -> float* {
    return decltype(buf)::value ? (v ? vscl1 : kscl1) : (v ? vscl0 : kscl0);
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane holds
  const int qn = lane & 31;    // query column of this lane in the 32x32 accumulator

  // Workgroup -> (batch, head, query tile).  Workgroups are handed to the 8 XCDs round-robin
  // (id % 8), and each XCD has its own L2.  Re-index so that XCD x receives a contiguous run of
  // the (batch, head)-major work list: all query tiles of one head then run on one XCD at about
  // the same time and share that head's K/V tiles in its L2.  Within a head, tiles run in the
  // plan's heavy-first order.  (A remainder of fewer than 8 workgroups keeps its own index.)
  // A split decode adds a key-range index inside each (batch, head): workgroups of one (batch,
  // head, key range) stay contiguous, so they share that range's K/V tiles in one L2.
  const int n_split = kDecode && a.n_split > 1 ? a.n_split : 1;
  const int bh_count = a.batch * a.heads * n_split;
  const int total = a.n_qtiles * bh_count;
  const int full8 = total & ~7;
  int work = blockIdx.x;
  if (work < full8) work = (work & 7) * (full8 >> 3) + (work >> 3);
  int bhs = work / a.n_qtiles;
  int slot = work - bhs * a.n_qtiles;
  // The 12-wave decode may instead take query tiles of three heights (AttnArgs::mix): a round of
  // 256-row tiles (two waves per SIMD with rows) after the 384-row ones fills a grid whose
  // 384-row tiles would leave the last round part empty.
  constexpr bool kMix = kDecode && kW == kDecodeDirectWaves;
  static_assert(!kMix || kRows == 384, "tile heights 384, 256, 128");
  int mix_row0 = 0, tile_rows = kRows;
  if constexpr (kMix) {
    mix_row0 = slot * kRows;
    if ((a.mix[0] | a.mix[1] | a.mix[2]) != 0) {
      // this XCD's bh_count / 8 (batch, head) entries (bh_count % 8 == 0 here)
      const int nb = bh_count >> 3;
      int l = blockIdx.x >> 3, hl;
      if (l < nb * a.mix[0]) {
        hl = l / a.mix[0];
        mix_row0 = 384 * (l - hl * a.mix[0]);
      } else if ((l -= nb * a.mix[0]) < nb * a.mix[1]) {
        hl = l / a.mix[1];
        mix_row0 = 384 * a.mix[0] + 256 * (l - hl * a.mix[1]);
        tile_rows = 256;
      } else {
        l -= nb * a.mix[1];
        hl = l / a.mix[2];
        mix_row0 = 384 * a.mix[0] + 256 * a.mix[1] + 128 * (l - hl * a.mix[2]);
        tile_rows = 128;
      }
      bhs = (blockIdx.x & 7) * nb + hl;
      slot = 0;
    }
  }
  const int bh = kDecode ? bhs / n_split : bhs;
  const int split = kDecode ? bhs - bh * n_split : 0;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int tile = kDecode ? slot : a.order[slot];
  // The tile's sequence (prefill plans may hold several): its first tensor row, the tile's first
  // local row, its length and where its row limits start.  Rows, keys and limits below are local
  // to the sequence; the decode has one sequence of n_q query rows over kv_len keys.
  // Keys below kv_split come from the first source, the rest from the second; kv_len in all.
  // cache_row0: first cache row of the sequence's prefix (stored by the prefill, read by a
  // decode over a batch of sequences, whose targets start at tensor row seq_row0).
  // (the decode's tail launch starts its tiles at row_base)
  constexpr bool kTail = kDecode && kW == kDecodeTailWaves;
  int seq_row0 = 0, row0 = tile * kRows + (kTail ? a.row_base : 0), n_rows = a.n_q, rl_off = 0;
  if constexpr (kMix) row0 = mix_row0;
  int kv_len = a.kv_len, kv_split = a.split, kv_end = a.kv_len, kv_full = a.kv_len;
  int cache_len = 0, cache_row0 = 0;
  if constexpr (!kDecode) {
    const int32_t* td = a.tiles + tile * kTileInts;
    seq_row0 = td[0];
    row0 = td[1];
    n_rows = td[2];
    rl_off = td[3];
    kv_full = td[4];
    kv_end = td[5];
    cache_len = td[6];
    cache_row0 = td[7];
  } else if (a.seqs != nullptr) {
    const int32_t* sd = a.seqs + b * kSeqInts;
    kv_split = sd[2];
    n_rows = sd[3];
    cache_row0 = sd[4];
    seq_row0 = sd[5];
    kv_len = kv_end = kv_full = kv_split + n_rows;
    // the grid spans the longest target: this sequence may have no rows in this tile (the whole
    // workgroup leaves before any barrier)
    if (row0 >= n_rows) return;
  }
  // this tile's real rows end here
  const int row_end = kMix ? min(n_rows, row0 + tile_rows) : n_rows;
  const int ntiles = (kv_end + kBlockN - 1) / kBlockN;
  // key tiles this workgroup visits: all of them, or its split's range
  const int split_tiles = a.split_units * (kSplitUnit / kBlockN);
  const int j_begin = n_split > 1 ? split * split_tiles : 0;
  const int j_end = n_split > 1 ? min(ntiles, j_begin + split_tiles) : ntiles;

  // does any of this wave's query rows exist (wave-uniform)
  const int wave_row0 = row0 + wave * 32 * kQueryBlocks;
  const bool live = wave_row0 + 32 * kQueryBlocks > 0 && wave_row0 < row_end;
  // Prefill: the largest key limit among this wave's real rows (wave-uniform: limits never
  // decrease along a sequence, so it is the last real row's).  A key tile starting at or past it
  // is invisible to the whole wave, whose part of that tile then adds exact zeros.
  int wave_lim = kv_len;
  if constexpr (!kDecode) {
    const int last = min(wave_row0 + 32 * kQueryBlocks - 1, n_rows - 1);
    wave_lim = __builtin_amdgcn_readfirstlane(last < 0 ? 0 : a.row_limit[rl_off + last]);
  }
  // In the 4-wave decode, a wave whose rows all lie past the end skips its compute inside the
  // tile loop (measured 5% faster there than a loop of its own, from the code generation).
  constexpr bool kSkipDead = kDecode && kW == kDecodeDirectSmallWaves;

  // This lane's query rows, their key limits, and their Q slices as MFMA B operands.
  int lim[kQueryBlocks];
  bool row_ok[kQueryBlocks];
  bf16x8 qreg[kQueryBlocks][8];
#pragma unroll
  for (int qb = 0; qb < kQueryBlocks; ++qb) {
    const int row = row0 + (wave * kQueryBlocks + qb) * 32 + qn;
    row_ok[qb] = row >= 0 && row < row_end;  // a prefill tile's first rows may be padding
    lim[qb] = kDecode ? kv_len : a.row_limit[rl_off + (row_ok[qb] ? row : n_rows - 1)];
    const uint16_t* qp = a.q + b * a.q_sb + (int64_t)(seq_row0 + (row_ok[qb] ? row : 0)) * a.q_ss +
                         h * a.q_sh + 8 * half;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 x =
          row_ok[qb] ? *reinterpret_cast<const u32x4*>(qp + 16 * c) : u32x4{0, 0, 0, 0};
      qreg[qb][c] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // first key source: bf16, or (decode over a quantised cache) code bytes plus row scales
  // (prefill: the sequence's own rows; decode: its cache rows, then its target rows)
  const int64_t src1_row = kDecode ? cache_row0 : seq_row0;
  const uint16_t* k_base =
      static_cast<const uint16_t*>(a.k) + b * a.k_sb + h * a.k_sh + src1_row * a.k_ss;
  const uint16_t* v_base =
      static_cast<const uint16_t*>(a.v) + b * a.v_sb + h * a.v_sh + src1_row * a.v_ss;
  const uint8_t* k8_base =
      static_cast<const uint8_t*>(a.k) + b * a.k_sb + h * a.k_sh + src1_row * a.k_ss;
  const uint8_t* v8_base =
      static_cast<const uint8_t*>(a.v) + b * a.v_sb + h * a.v_sh + src1_row * a.v_ss;
  const float* ks_base =
      kKqSrc ? a.kcs + b * a.kcs_sb + h * a.kcs_sh + src1_row * a.kcs_ss : nullptr;
  const float* vs_base =
      kVqSrc ? a.vcs + b * a.vcs_sb + h * a.vcs_sh + src1_row * a.vcs_ss : nullptr;
  const uint16_t* k2_base = a.k2 + b * a.k2_sb + h * a.k2_sh + (int64_t)seq_row0 * a.k2_ss;
  const uint16_t* v2_base = a.v2 + b * a.v2_sb + h * a.v2_sh + (int64_t)seq_row0 * a.v2_ss;

  // Descriptor of one whole tile from one source: its first row, 32-bit offsets inside it.
  auto tile_rsrc = [&](const void* first_row, int64_t row_bytes) {
    const int64_t bytes = (int64_t)(kBlockN - 1) * row_bytes + kHeadDim * 2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(first_row), (short)0,
                                             (int)(uint32_t)bytes, kBufferWord3);
  };

  // ---- filling the ring: direct loads ----------------------------------------------------------
  // A tile is kFills load instructions of one 4-row group (4 x 256 bytes): K's kGroups groups,
  // then V's.  Instruction n is issued by wave n % kW as that wave's fill n / kW.  Lane L writes
  // LDS chunk L % 16 of row L / 16 of the group, so it fetches logical chunk (L % 16) ^ swz(row)
  // of that key.  With kW a multiple of 4 every group a wave fills is congruent to the wave mod 4,
  // so all its fills share one swizzle phase and the lane's offset inside a group is one VGPR per
  // source stride.  The group's first row is added to it (prefill: its descriptor ends at the
  // sequence's last row, and rows past it load as zero, which takes the whole offset inside the
  // range check) or goes in the scalar offset (decode whole tiles, all in range; the scalar
  // offset is outside the range check).
  // The common case (whole tile from one source, nothing past kv_end) goes through a tile-wide
  // descriptor; a decode tile straddling the cache/target split or the end resolves each row.
  constexpr int kGroups = kBlockN / 4;
  constexpr int kFills = 2 * kGroups;
  constexpr int kFillsPerWave = (kFills + kW - 1) / kW;
  static_assert(kW % 4 == 0 && kGroups % 4 == 0, "one swizzle phase per wave");
  const int dma_r = lane >> 4;
  const int dma_p = lane & 15;
  auto fill_n = [&](int i) { return wave + kW * i; };  // wave-uniform
  auto fill_is_v = [&](int i) { return fill_n(i) >= kGroups; };
  auto fill_g = [&](int i) { return fill_is_v(i) ? fill_n(i) - kGroups : fill_n(i); };
  auto fill_row = [&](int i) { return 4 * fill_g(i) + dma_r; };
  // swz(row) = ((row & 3) << 2) | ((row >> 2) & 3) with row & 3 = dma_r and row >> 2 = the group
  const int fill_col = 8 * (dma_p ^ ((dma_r << 2) | (wave & 3)));
  // byte offset of this lane inside a 4-row group with row stride ss (elements)
  auto lane_off = [&](int64_t ss) {
    uint32_t off = ((uint32_t)dma_r * (uint32_t)ss + (uint32_t)fill_col) * 2u;
    asm volatile("" : "+v"(off));
    return off;
  };
  // This wave's fills of a whole tile from descriptors kr and vr (row strides kss, vss; lane
  // offsets koff, voff).
  // (do_k, do_v: std::bool_constant; a tensor whose rows come from codes is not filled here)
  auto fill_whole = [&](__amdgpu_buffer_rsrc_t kr, int64_t kss, uint32_t koff,
                        __amdgpu_buffer_rsrc_t vr, int64_t vss, uint32_t voff, auto buf,
                        auto do_k, auto do_v) {
#pragma unroll
    for (int i = 0; i < kFillsPerWave; ++i) {
      if (kFills % kW != 0 && fill_n(i) >= kFills) break;
      const int r0 = 4 * fill_g(i);
      const bool v = fill_is_v(i);
      if (v ? !decltype(do_v)::value : !decltype(do_k)::value) continue;
      const uint32_t rows_off = (uint32_t)(r0 * (v ? vss : kss) * 2);
      const uint32_t vo = kDecode ? (v ? voff : koff) : (v ? voff : koff) + rows_off;
      const uint32_t so = kDecode ? rows_off : 0u;
      __bf16* dst = (v ? v_lds(buf) : k_lds(buf)) + r0 * kHeadDim;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? vr : kr, (lds_void*)dst, 16, vo, so, 0, 0);
    }
  };
  auto dma_rsrc = [&](const uint16_t* base, int64_t ss, int n0) {
    const int64_t bytes = ((int64_t)(n_rows - 1 - n0) * ss + kHeadDim) * 2;  // to the sequence end
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)n0 * ss), (short)0,
                                             (int)(uint32_t)bytes, kBufferWord3);
  };
  const uint32_t dma_k = lane_off(a.k_ss), dma_v = lane_off(a.v_ss);
  const uint32_t dma_k2 = kDecode ? lane_off(a.k2_ss) : 0u;
  const uint32_t dma_v2 = kDecode ? lane_off(a.v2_ss) : 0u;
  auto dma_tile = [&](int n0, auto buf) {
    if constexpr (!kDecode) {
      fill_whole(dma_rsrc(k_base, a.k_ss, n0), a.k_ss, dma_k, dma_rsrc(v_base, a.v_ss, n0), a.v_ss,
                 dma_v, buf, std::true_type{}, std::true_type{});
      return;
    }
    const bool in_end = n0 + kBlockN <= kv_end;
    const bool src1 = n0 + kBlockN <= kv_split;
    const bool src2 = n0 >= kv_split;
    // decode: whole tiles from one source through buffer loads, the rest row by row below
    if (in_end && src1) {
      if constexpr (!kKqSrc || !kVqSrc)
        fill_whole(tile_rsrc(k_base + (int64_t)n0 * a.k_ss, a.k_ss * 2), a.k_ss, dma_k,
                   tile_rsrc(v_base + (int64_t)n0 * a.v_ss, a.v_ss * 2), a.v_ss, dma_v, buf,
                   std::bool_constant<!kKqSrc>{}, std::bool_constant<!kVqSrc>{});
      return;
    }
    if (in_end && src2) {
      fill_whole(tile_rsrc(k2_base + (int64_t)(n0 - kv_split) * a.k2_ss, a.k2_ss * 2), a.k2_ss,
                 dma_k2, tile_rsrc(v2_base + (int64_t)(n0 - kv_split) * a.v2_ss, a.v2_ss * 2),
                 a.v2_ss, dma_v2, buf, std::true_type{}, std::true_type{});
      return;
    }
#pragma unroll
    for (int i = 0; i < kFillsPerWave; ++i) {
      if (kFills % kW != 0 && fill_n(i) >= kFills) break;
      const bool v = fill_is_v(i);
      // keys past the end fetch row kv_end - 1 (masked, finite)
      const int key = min(n0 + fill_row(i), kv_end - 1);
      const bool first = key < kv_split;
      // a quantised tensor's cache rows come from its codes (convert): those lanes load nothing
      if ((v ? kVqSrc : kKqSrc) && first) continue;
      const uint16_t* p = v ? (first ? v_base + (int64_t)key * a.v_ss
                                     : v2_base + (int64_t)(key - kv_split) * a.v2_ss)
                            : (first ? k_base + (int64_t)key * a.k_ss
                                     : k2_base + (int64_t)(key - kv_split) * a.k2_ss);
      const int dst = 4 * fill_g(i) * kHeadDim;
      __builtin_amdgcn_global_load_lds((const void*)(p + fill_col),
                                       (lds_void*)&(v ? v_lds(buf) : k_lds(buf))[dst], 16, 0, 0);
    }
  };

  // ---- quantised cache rows (direct-fill decode over an FP8 cache) ------------------------------
  // code_fill: the code bytes and scales of tile n0's cache rows (rows past the split repeat the
  // last cache row; convert skips them) into code buffer cb.  Per quantised tensor five loads:
  // four of 8 rows x 128 B (lane L: row L / 8, bytes 16 (L % 8) ..) and one of the 32 row scales
  // (lane L: row L % 32); load i goes to wave i % kW.  Buffer loads from a descriptor at the
  // tile's first row, with 32-bit lane offsets.
  constexpr int kCodeLoads = (kVqSrc ? 5 : 0) + (kKqSrc ? 5 : 0);
  auto code_fill = [&](int n0, auto cb) {
    if constexpr (kDirectQ) {
      if (n0 >= kv_split) return;
      const int last = min(kBlockN, kv_split - n0) - 1;  // last cache row of the tile
      for (int i = wave; i < kCodeLoads; i += kW) {
        const bool v = kVqSrc && i < 5;
        const int g = i % 5;
        if (g < 4) {
          const int64_t ss = v ? a.v_ss : a.k_ss;
          const uint8_t* base = (v ? v8_base : k8_base) + (int64_t)n0 * ss;
          const auto rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)base, (short)0, (int)(uint32_t)(last * ss + kHeadDim), kBufferWord3);
          const uint32_t off =
              (uint32_t)min(8 * g + (lane >> 3), last) * (uint32_t)ss + 16u * (lane & 7);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(code_lds(v, cb) + 8 * g * kHeadDim),
                                                   16, off, 0, 0, 0);
        } else {
          const int64_t ss = v ? a.vcs_ss : a.kcs_ss;
          const float* base = (v ? vs_base : ks_base) + (int64_t)n0 * ss;
          const auto rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)base, (short)0, (int)(uint32_t)((last * ss + 1) * 4), kBufferWord3);
          const uint32_t off = (uint32_t)min(lane & 31, last) * (uint32_t)ss * 4u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)scl_lds(v, cb), 4, off, 0, 0, 0);
        }
      }
    }
  };
  // convert: the cache rows of tile n0 from code buffer `buf` into the bf16 tile of the same
  // index, value = E4M3(code) * scale rounded to bf16 (dequant), in the tile's swizzled layout.
  // Work items of 8 values, 512 per quantised tensor (V first): item c is row (c % 512) / 16,
  // columns 8 (c % 16) .. + 7, taken by thread c % kThreads.
  auto convert = [&](int n0, auto buf) {
    if constexpr (kDirectQ) {
      if (n0 >= kv_split) return;
      constexpr int kItems = 512 * ((kVqSrc ? 1 : 0) + (kKqSrc ? 1 : 0));
#pragma unroll
      for (int c0 = 0; c0 < kItems; c0 += kThreads) {
        const int c = c0 + tid;
        if (kItems % kThreads != 0 && c >= kItems) break;
        const bool v = kVqSrc && c < 512;
        const int row = (c & 511) >> 4, col8 = c & 15;
        if (n0 + row >= kv_split) continue;
        const uint2 codes =
            *reinterpret_cast<const uint2*>(code_lds(v, buf) + row * kHeadDim + 8 * col8);
        const float sc = scl_lds(v, buf)[row];
        const u32x4 x = {codes.x, codes.y, __builtin_bit_cast(uint32_t, sc), 0u};
        __bf16* dst = (v ? v_lds(buf) : k_lds(buf)) + row * kHeadDim + 8 * (col8 ^ swz(row));
        *reinterpret_cast<u32x4*>(dst) = dequant(x);
      }
    }
  };

  // ---- prefix-K/V cache (prefill only) ----------------------------------------------------------
  // This workgroup owns cache rows [cache_lo, cache_hi), which lie inside its own diagonal key
  // tiles; they are copied out of the LDS tile while it is resident, so no K/V row is fetched
  // twice.  Either tensor may be absent (NULL): a quantised one is written by its own pass.
  const int cache_lo = row0;
  const int cache_hi =
      kDecode || (a.kc == nullptr && a.vc == nullptr) ? 0 : min(cache_lo + kRows, cache_len);
  // Chunk tid + kThreads r of the tile: row (tid >> 4) + kRowsPerPass r, chunk tid % 16 (a
  // partial last pass stores nothing past the tile).
  const int ld_row = tid >> 4;
  const int ld_col = (tid & 15) * 8;
  auto store_row = [&](int n0, auto buf, int r) {
    const int row = ld_row + kRowsPerPass * r;
    const int key = n0 + row;
    if (row >= kBlockN || key < cache_lo || key >= cache_hi) return;
    const int col = 8 * ((ld_col >> 3) ^ swz(row));
    const int64_t at = (int64_t)cache_row0 + key;
    if (a.kc != nullptr)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.kc) + b * a.kc_sb + at * a.kc_ss +
                                h * a.kc_sh + ld_col) =
          *reinterpret_cast<const u32x4*>(&k_lds(buf)[row * kKStride + col]);
    if (a.vc != nullptr)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.vc) + b * a.vc_sb + at * a.vc_ss +
                                h * a.vc_sh + ld_col) =
          *reinterpret_cast<const u32x4*>(&v_lds(buf)[row * kVStride + col]);
  };
  auto store_cache = [&](int n0, auto buf) {
    if (kDecode || n0 >= cache_hi || n0 + kBlockN <= cache_lo) return;
    // n0 made opaque: otherwise the compiler keeps this rare store's row pointers live across
    // the whole loop and advances them every tile
    asm volatile("" : "+s"(n0));
#pragma unroll
    for (int r = 0; r < kChunksPerThread; ++r) store_row(n0, buf, r);
  };

  // ---- per-lane LDS read addresses (byte offsets inside one buffer) ------------------------------
  // K operand of MFMA step c, key block kb: row 32 kb + qn, d = 16 c + 8 half .. + 7.
  // V^T operand (ds_read_b64_tr_b16): lane t of each 16-lane group points at row t / 4 and
  // column 4 (t % 4) of a 4 x 16 block and receives that block's column t (4 rows).
  const int g = lane >> 4;
  const int tq = lane & 15;
  const int tr_row = 4 * half + (tq >> 2);
  const int tr_col = 16 * (g & 1) + 4 * (tq & 3);
  auto k_addr = [&](int kb, int c) {
    const int row = 32 * kb + qn;
    const int chunk = 2 * c + half;
    return row * kKStride + 8 * (chunk ^ swz(row));
  };
  auto v_addr = [&](int kc, int d, int hi) {
    const int row = 16 * kc + tr_row + 8 * hi;
    const int col = 32 * d + tr_col;
    return row * kVStride + 8 * ((col >> 3) ^ swz(row)) + (col & 7);
  };
  // The same offsets computed once, in bytes.  Key block kb (K) and 16-row group kc (V) only add
  // constants (swz(row) depends on row bits 0..3, and those do not change with kb or kc), and so
  // does the buffer where the loop below names it by a constant; all of these fold into the
  // reads' immediate offsets.  In a swizzled tile the chunk index is not additive, so each MFMA
  // step c (K) and each (row half hi, column block d) pair (V) keeps its own offset; the asm
  // barrier stops the compiler from re-deriving them inside the loop.
  int koff[8], voff[2][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    koff[c] = 2 * k_addr(0, c);
    asm volatile("" : "+v"(koff[c]));
  }
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      voff[hi][d] = 2 * v_addr(0, d, hi);
      asm volatile("" : "+v"(voff[hi][d]));
    }
  // Operand reads from buffer `cur`: an int, or a std::integral_constant where the loop is
  // unrolled by two tiles, which leaves no address arithmetic in the loop at all.
  auto k_read = [&](auto cur, int c, int kb) {
    const char* p = reinterpret_cast<const char*>(&k_lds(cur)[0]) + koff[c] + 64 * kb * kKStride;
    return *reinterpret_cast<const bf16x8*>(p);
  };
  auto v_read = [&](auto cur, int hi, int d, int kc) {
    const char* p = reinterpret_cast<const char*>(&v_lds(cur)[0]) + voff[hi][d] + 32 * kc * kVStride;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
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

  // ---- prologue ----------------------------------------------------------------------------------
  // Tile j lives in buffer (j - j_begin) % 2; the first two tiles resident.
  using Buf0 = std::integral_constant<int, 0>;
  using Buf1 = std::integral_constant<int, 1>;
  if (j_begin < j_end) dma_tile(j_begin * kBlockN, Buf0{});
  if (j_begin + 1 < j_end) dma_tile((j_begin + 1) * kBlockN, Buf1{});
  if constexpr (kDirectQ) {
    // the codes of the first two tiles, converted once they are all in; the third tile's codes
    // go into code buffer 0 only after every wave has converted from it
    if (j_begin < j_end) code_fill(j_begin * kBlockN, Buf0{});
    if (j_begin + 1 < j_end) code_fill((j_begin + 1) * kBlockN, Buf1{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j_begin < j_end) convert(j_begin * kBlockN, Buf0{});
    if (j_begin + 1 < j_end) convert((j_begin + 1) * kBlockN, Buf1{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j_begin + 2 < j_end) code_fill((j_begin + 2) * kBlockN, Buf0{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One key tile j from buffer cur.  kMasked: the tile crosses some row's key limit.  Full tiles
  // run in a loop of their own, with no mask code between the score MFMAs and the softmax, so the
  // compiler can overlap the two inside one wave.
  auto tile_step = [&](auto masked_c, int j, auto cur) {
    constexpr bool kMasked = decltype(masked_c)::value;
    const int n0 = j * kBlockN;
    store_cache(n0, cur);
    // A wave that sees no key of a masked tile, or (4-wave bf16 decode) whose query rows all lie
    // past the end, only fills and synchronises: its share of the tile is exactly zero.
    // A 64-key tile is computed as two 32-key halves in key order, exactly as two 32-key tiles.
#pragma unroll
    for (int kh = 0; kh < kKeyBlocks; ++kh) {
      const int nh = n0 + 32 * kh;
      if ((!kSkipDead || live) && !(kMasked && !kDecode && nh >= wave_lim)) {
        constexpr int kKB = 1;

        // ---- S^T = K Q^T
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(kPrioLevel);
        f32x16 s[kQueryBlocks][kKB];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
          for (int qb = 0; qb < kQueryBlocks; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const bf16x8 ka = k_read(cur, c, kh + kb);
#pragma unroll
            for (int qb = 0; qb < kQueryBlocks; ++qb)
              s[qb][kb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], s[qb][kb], 0, 0, 0);
          }
        }
        pipeline_reads<8 * kKB, 1, kQueryBlocks, kSchedKDepth>();

        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        // ---- mask: only tiles that cross some row's limit.  Accumulator element i of key block kb
        // holds key n0 + 32 kb + 8 (i / 4) + 4 half + i % 4.
        if (kMasked) {
#pragma unroll
          for (int qb = 0; qb < kQueryBlocks; ++qb)
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key = nh + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
                if (key >= lim[qb]) s[qb][kb][i] = -__builtin_inff();
              }
        }

        // ---- p = 2^(s c2 - m) against the running max m of earlier tiles, as bf16 P^T
        // operands (chunks of 16 keys), plus this tile's row-sum share.  A row whose scores grew
        // past m + kRescaleThreshold (or any row on its first tile, where m = -inf) shows a lane
        // sum above 2^threshold (or inf); only then does the wave take the exact path: per-row
        // max, raise and rescale for rows that grew by more than the threshold, and p recomputed.
        // Rows that do not raise recompute the same values, so each row still depends on its own
        // scores alone.
        bf16x8 pb[kQueryBlocks][2 * kKB];
        float tsum[kQueryBlocks];
        auto exp_tile = [&](int qb) {
          const float mneg = -m_run[qb];
          float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
              const float x0 = __builtin_fmaf(s[qb][kb][i], c2, mneg);
              const float x1 = __builtin_fmaf(s[qb][kb][i + 1], c2, mneg);
              const float p0 = __builtin_amdgcn_exp2f(x0);
              const float p1 = __builtin_amdgcn_exp2f(x1);
              const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
              pb[qb][2 * kb + (i >> 3)][i & 7] = pp[0];
              pb[qb][2 * kb + (i >> 3)][(i & 7) + 1] = pp[1];
              if (i & 2)
                acc1 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc1, false);
              else
                acc0 = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc0, false);
            }
          tsum[qb] = acc0 + acc1;
        };
        bool redo = false;
#pragma unroll
        for (int qb = 0; qb < kQueryBlocks; ++qb) {
          exp_tile(qb);
          redo = redo || !(tsum[qb] <= kRescaleBound);
        }
        if (__builtin_amdgcn_ballot_w64(redo)) {
#pragma unroll
          for (int qb = 0; qb < kQueryBlocks; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb][kb][i]);
            mx = halves_max(mx);
            const float m_cand = fmaxf(m_run[qb], mx * c2);
            const bool raise = m_cand > m_run[qb] + kRescaleThreshold;
            // (0 on the first tile)
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run[qb] - m_cand) : 1.0f;
            m_run[qb] = raise ? m_cand : m_run[qb];
            l_part[qb] *= alpha;
#pragma unroll
            for (int d = 0; d < 4; ++d) o[qb][d] *= alpha;
            exp_tile(qb);
          }
        }
#pragma unroll
        for (int qb = 0; qb < kQueryBlocks; ++qb) l_part[qb] += tsum[qb];

        // ---- O^T += V^T P^T
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(kPrioLevel);
#pragma unroll
        for (int kc = 0; kc < 2 * kKB; ++kc) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const bf16x4 lo = v_read(cur, 0, d, 2 * kh + kc);
            const bf16x4 hi = v_read(cur, 1, d, 2 * kh + kc);
            const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int qb = 0; qb < kQueryBlocks; ++qb)
              o[qb][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[qb][kc], o[qb][d], 0, 0, 0);
          }
        }
        pipeline_reads<8 * kKB, 2, kQueryBlocks, kSchedVDepth>();

        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      }
    }

    // ---- refill: tile j+1 was issued one iteration ago; wait for it, then after the barrier
    // reuse this buffer for tile j+2
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < j_end) {
      // quantised cache rows of tile j+2: their codes (code buffer cur, fetched one tile ago)
      // into this buffer; then the codes of tile j+3 into the other code buffer, which every
      // wave finished converting from before this barrier
      convert((j + 2) * kBlockN, cur);
      dma_tile((j + 2) * kBlockN, cur);
      if constexpr (kDirectQ) {
        if (j + 3 < j_end)
          code_fill((j + 3) * kBlockN, std::integral_constant<int, 1 - decltype(cur)::value>{});
      }
    }
  };
  // The share of tile j of a wave without query rows: the same fills and barrier.
  auto idle_step = [&](int j, auto cur) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < j_end) {
      convert((j + 2) * kBlockN, cur);
      dma_tile((j + 2) * kBlockN, cur);
      if constexpr (kDirectQ) {
        if (j + 3 < j_end)
          code_fill((j + 3) * kBlockN, std::integral_constant<int, 1 - decltype(cur)::value>{});
      }
    }
  };
  // tiles [0, n_full) lie entirely below every row's limit; the rest need the mask
  const int n_full = min(j_end, kv_full / kBlockN);
  // two tiles per trip, buffer 0 then buffer 1, so that each copy names its buffer by a constant
  auto run = [&](auto masked_c, int lo, int hi) {
    int j = lo;
    if (j < hi && ((j - j_begin) & 1)) tile_step(masked_c, j++, Buf1{});
    for (; j + 1 < hi; j += 2) {
      tile_step(masked_c, j, Buf0{});
      tile_step(masked_c, j + 1, Buf1{});
    }
    if (j < hi) tile_step(masked_c, j, Buf0{});
  };
  // 12-wave decode: a wave without query rows (a 256- or 128-row tile, or past the end) runs the
  // tile loop's barriers in a loop of its own, which leaves the compute loop free of any test for
  // it.  (The prefill's padding waves, in a sequence's first tile only, compute zeros.)
  if constexpr (kMix) {
    if (!live) {
      int j = j_begin;
      if (j < j_end && ((j - j_begin) & 1)) idle_step(j++, Buf1{});
      for (; j + 1 < j_end; j += 2) {
        idle_step(j, Buf0{});
        idle_step(j + 1, Buf1{});
      }
      if (j < j_end) idle_step(j, Buf0{});
      return;
    }
  }
  run(std::false_type{}, j_begin, n_full);
  run(std::true_type{}, max(j_begin, n_full), j_end);

  // ---- split epilogue: this key range's unnormalised O, running max m (scaled, base 2) and row
  // sum l, to be merged by split_combine.  Layout [split][b][row][h] (x 128 for O).
  if (n_split > 1) {
#pragma unroll
    for (int qb = 0; qb < kQueryBlocks; ++qb) {
      const float l = halves_sum(l_part[qb]);
      if (row_ok[qb]) {
        const int row = row0 + (wave * kQueryBlocks + qb) * 32 + qn;
        const int64_t r = (((int64_t)split * a.batch + b) * a.n_q + row) * a.heads + h;
        float* op = a.part_o + r * kHeadDim + 4 * half;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 val = {o[qb][d][4 * jj], o[qb][d][4 * jj + 1], o[qb][d][4 * jj + 2],
                               o[qb][d][4 * jj + 3]};
            *reinterpret_cast<f32x4*>(op + 32 * d + 8 * jj) = val;
          }
        if (half == 0) {
          a.part_ml[2 * r] = m_run[qb];
          a.part_ml[2 * r + 1] = l;
        }
      }
    }
    return;
  }

  // ---- epilogue: O = O_acc / l; lane holds dims 32 d + 8 jj + 4 half + (0..3) of its query
#pragma unroll
  for (int qb = 0; qb < kQueryBlocks; ++qb) {
    const float inv = 1.0f / halves_sum(l_part[qb]);
    if (row_ok[qb]) {
      const int row = row0 + (wave * kQueryBlocks + qb) * 32 + qn;
      float* op = a.o + b * a.o_sb + (int64_t)(seq_row0 + row) * a.o_ss + h * a.o_sh + 4 * half;
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

// Merges the key ranges of a split decode: per (b, row, h), M = max m_c, w_c = 2^(m_c - M),
// O = sum_c w_c O_c / sum_c w_c l_c.  Sixteen lanes per row, eight dims per lane.
__global__ __launch_bounds__(256) void split_combine(const AttnArgs a) {
  const int64_t rows = (int64_t)a.batch * a.n_q * a.heads;
  const int64_t r_raw = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (r_raw >= rows) return;  // whole 16-lane groups; no cross-lane exchange below
  const int d0 = 8 * (threadIdx.x & 15);
  const int h = (int)(r_raw % a.heads);
  const int64_t bn = r_raw / a.heads;
  const int row = (int)(bn % a.n_q);
  const int b = (int)(bn / a.n_q);
  float mx = -__builtin_inff();
  for (int c = 0; c < a.n_split; ++c) mx = fmaxf(mx, a.part_ml[2 * (c * rows + r_raw)]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float l = 0.0f;
  for (int c = 0; c < a.n_split; ++c) {
    const int64_t r = c * rows + r_raw;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * r] - mx);
    l = __builtin_fmaf(w, a.part_ml[2 * r + 1], l);
    const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + r * kHeadDim + d0);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = __builtin_fmaf(w, x0[i], acc[i]);
      acc[4 + i] = __builtin_fmaf(w, x1[i], acc[4 + i]);
    }
  }
  const float inv = 1.0f / l;
  float* op = a.o + b * a.o_sb + (int64_t)row * a.o_ss + h * a.o_sh + d0;
  *reinterpret_cast<f32x4*>(op) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  *reinterpret_cast<f32x4*>(op + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
}

// Prefill: block-causal, direct-to-LDS fills, optional store of the prefix cache's bf16 tensors.
__global__ __launch_bounds__(64 * kPrefillWaves)
__attribute__((amdgpu_waves_per_eu(kPrefillWavesPerSimd, kPrefillWavesPerSimd)))
void attn_prefill(const AttnArgs a) {
  attn_fwd<false, kCacheBf16, kPrefillBlockN, kPrefillWaves>(a);
}

// Decode over [prefix cache in format kFmt ; target]: direct-to-LDS fills like the prefill's
// (an FP8 cache's codes and scales too, turned into bf16 in LDS), 32-key tiles at 3 waves per
// SIMD, kW waves per workgroup.
template <int kFmt, int kW>
__global__ __launch_bounds__(64 * kW)
__attribute__((amdgpu_waves_per_eu(kDecodeDirectWavesPerSimd, kDecodeDirectWavesPerSimd)))
void attn_decode_direct(const AttnArgs a) {
  attn_fwd<true, kFmt, kDecodeDirectBlockN, kW>(a);
}

// Decode tail: the query tiles past the 12-wave launch's 384-row ones, as 256-row workgroups of 8
// waves at 2 waves per SIMD (the register budget of two waves allows 64-key fills, half the
// barriers) over a bf16 cache.  Each 64-key tile is computed as two 32-key halves, so every row
// gets bitwise the arithmetic of the 12-wave kernel.
__global__ __launch_bounds__(64 * kDecodeTailWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_decode_tail(const AttnArgs a) {
  attn_fwd<true, kCacheBf16, kDecodeTailBlockN, kDecodeTailWaves>(a);
}

// Library-owned device scratch for the allocation-free split decode (bca_decode_split_noalloc):
// the partial O, m and l of its key ranges.  One copy per GPU the library runs on, held until the
// process ends; every call on a GPU shares it.  In host code the array's name is only a
// stand-in: its device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) static unsigned char scratch[kScratchBytes];

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

hipError_t scratch_memory(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  std::lock_guard<std::mutex> lock(mu);
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  if (dev >= 0 && dev < kMaxDevices) ptrs[dev].store(p, std::memory_order_release);
  *out = p;
  return hipSuccess;
}

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.n_qtiles * a.batch * a.heads);
  const dim3 block(64 * kPrefillWaves);
  hipLaunchKernelGGL(attn_prefill, grid, block, 0, stream, a);
  return hipGetLastError();
}

// Query-tile mix of the 12-wave decode for n rows per (batch, head), nb (batch, head) entries
// per XCD and cx CUs per XCD.  Candidates: n2 tiles of 256 rows (0..16) and n1 of 128 rows (0..2)
// after as many 384-row tiles as the rest needs, no tile without rows.  Each is priced by a list
// schedule of the XCD's tiles in launch order on cx CUs (a free CU takes the next tile), a tile
// costing the step time of its busiest SIMD: 1, 0.88 and 0.66 for 3, 2 and 1 waves with rows
// (measured on the CFG cached step, 12,400 keys, whose query tiles share each K/V tile in L2),
// plus 0.01 for its prologue and epilogue.  When 256- or 128-row tiles follow, every 384-row tile
// is full and that phase is dealt in whole rounds (the first k3 % cx CUs take one tile more).
// The shortest schedule wins; a tie keeps the earlier candidate (fewer 256-row, then fewer
// 128-row tiles).  The last 8 queries are cached per thread.
void decode_mix(int n, int nb, int cx, int32_t mix[3], double* span_out) {
  struct Entry {
    int n, nb, cx;
    int32_t m[3];
    double span;
  };
  thread_local Entry cache[8];
  thread_local int cached = 0, next = 0;
  for (int i = 0; i < cached; ++i)
    if (cache[i].n == n && cache[i].nb == nb && cache[i].cx == cx) {
      mix[0] = cache[i].m[0], mix[1] = cache[i].m[1], mix[2] = cache[i].m[2];
      *span_out = cache[i].span;
      return;
    }
  const int quarters = (n + 127) / 128;
  auto tile_cost = [&](int row0, int rows) {
    const int live = std::min(rows, n - row0);
    const int waves = (live + 31) / 32;
    const int busiest = (waves + 3) / 4;
    return (busiest >= 3 ? 1.0 : busiest == 2 ? 0.88 : 0.66) + 0.01;
  };
  std::vector<double> loads((size_t)cx);
  double best = 0.0;
  int32_t pick[3] = {(n + 383) / 384, 0, 0};
  bool have = false;
  for (int n2 = 0; n2 <= 16; ++n2)
    for (int n1 = 0; n1 <= 2; ++n1) {
      const int n3 = std::max(0, (quarters - 2 * n2 - n1 + 2) / 3);
      const int covered = 384 * n3 + 256 * n2 + 128 * n1;
      const int last_rows = n1 ? 128 : n2 ? 256 : 384;
      if (n3 + n2 + n1 == 0 || covered < n || covered - last_rows >= n) continue;
      const int counts[3] = {n3, n2, n1}, heights[3] = {384, 256, 128};
      int k0 = 0;
      std::fill(loads.begin(), loads.end(), 0.0);
      if (n2 + n1 > 0) {
        const int64_t k3 = (int64_t)nb * n3;
        const double c3 = tile_cost(0, 384);
        for (int c = 0; c < cx; ++c) loads[(size_t)c] = (double)(k3 / cx + (c < k3 % cx)) * c3;
        k0 = 1;
      }
      std::priority_queue<double, std::vector<double>, std::greater<double>> free_at(
          loads.begin(), loads.end());
      double span = *std::max_element(loads.begin(), loads.end());
      int base = k0 ? 384 * n3 : 0;
      for (int k = k0; k < 3; ++k) {
        for (int e = 0; e < nb; ++e)
          for (int t = 0; t < counts[k]; ++t) {
            const double done = free_at.top() + tile_cost(base + heights[k] * t, heights[k]);
            free_at.pop();
            free_at.push(done);
            span = std::max(span, done);
          }
        base += heights[k] * counts[k];
      }
      if (!have || span < best - 1e-9) {
        best = span;
        pick[0] = n3, pick[1] = n2, pick[2] = n1;
        have = true;
      }
    }
  mix[0] = pick[0], mix[1] = pick[1], mix[2] = pick[2];
  *span_out = best;
  cache[next] = Entry{n, nb, cx, {pick[0], pick[1], pick[2]}, best};
  next = (next + 1) % 8;
  cached = std::min(cached + 1, 8);
}

// Two launches instead of one mixed launch: n3 tiles of 384 rows per (batch, head) in the 12-wave
// kernel, then the remaining rows in 256-row tiles of the 8-wave tail kernel, which start once
// the first launch has ended.  Both phases deal equal tiles, in whole rounds of the XCD's cx CUs:
// ceil(nb n3 / cx) * 1.01 + 0.02 (the launch boundary) + ceil(nb n_tail / cx) * 0.737, a 256-row
// tail tile costing 0.727 of a 384-row 12-wave tile (measured on the CFG cached step) + 0.01.
// Returns the best n3 and its span, or n3 = -1 when no rows are left for a tail.
static void decode_two_launch(int n, int nb, int cx, int* best_n3, double* best_span) {
  *best_n3 = -1;
  *best_span = 0.0;
  auto rounds = [&](int64_t k) { return (double)((k + cx - 1) / cx); };
  for (int n3 = 0; 384 * n3 < n; ++n3) {
    const int n_tail = (n - 384 * n3 + 255) / 256;
    const double span = rounds((int64_t)nb * n3) * 1.01 + (n3 > 0 ? 0.02 : 0.0) +
                        rounds((int64_t)nb * n_tail) * 0.737;
    if (*best_n3 < 0 || span < *best_span - 1e-9) {
      *best_n3 = n3;
      *best_span = span;
    }
  }
}

DecodeLayout decode_layout(int64_t n_q, int64_t groups, int n_split, int cus, int cache_fmt) {
  DecodeLayout l{};
  auto tiles = [&](int waves) {
    const int64_t rows = 32 * kQueryBlocks * waves;
    return (n_q + rows - 1) / rows;
  };
  const int64_t t12 = tiles(kDecodeDirectWaves);
  if (n_split <= 1 && groups % 8 == 0 && cus % 8 == 0) {
    // mixed tile heights: 12-wave workgroups once 384-row tiles would fill one round
    if (t12 * groups >= (int64_t)cus) {
      l.waves = kDecodeDirectWaves;
      double span = 0.0;
      decode_mix((int)n_q, (int)(groups / 8), cus / 8, l.tiles, &span);
      l.mixed = true;
      // a bf16 cache may instead finish with the 8-wave tail launch, taken when the replay
      // predicts it at least 3% shorter and each XCD holds at least 4 (batch, head) entries
      // (measured from 4 to 16; the replay overstates the gain, which is 0-9%)
      if (cache_fmt == kCacheBf16 && groups / 8 >= 4) {
        int n3 = -1;
        double two = 0.0;
        decode_two_launch((int)n_q, (int)(groups / 8), cus / 8, &n3, &two);
        if (n3 >= 0 && two < 0.97 * span) {
          l.tiles[0] = n3;
          l.tiles[1] = l.tiles[2] = 0;
          l.tail = (int32_t)((n_q - 384 * (int64_t)n3 + 255) / 256);
        }
      }
      return l;
    }
    // Under one round of 384-row tiles, over a bf16 cache: every row in 256-row tiles of the
    // 8-wave kernel when those fill more than half of the CUs in one round, one round of 12-wave
    // workgroups when the 256-row tiles would need a second; else the 4-wave launch below (it
    // measured ahead once half the CUs or fewer would be busy).
    if (cache_fmt == kCacheBf16) {
      const int64_t n_tail = (n_q + 255) / 256;
      if (n_tail * groups > (int64_t)cus) {
        l.waves = kDecodeDirectWaves;
        l.tiles[0] = (int32_t)t12;
        l.mixed = true;
        return l;
      }
      if (2 * n_tail * groups > (int64_t)cus) {
        l.waves = kDecodeDirectWaves;
        l.mixed = true;
        l.tail = (int32_t)n_tail;
        return l;
      }
    }
  } else if (t12 * groups * std::max(n_split, 1) >= 2 * (int64_t)cus) {
    // 384-row tiles only: 12-wave workgroups where they give every CU at least two
    l.waves = kDecodeDirectWaves;
    l.tiles[0] = (int32_t)t12;
    return l;
  }
  l.waves = kDecodeDirectSmallWaves;
  l.tiles[2] = (int32_t)tiles(kDecodeDirectSmallWaves);
  return l;
}

hipError_t launch_decode(const AttnArgs& args, hipStream_t stream) {
  AttnArgs a = args;
  const int n_split = a.n_split > 1 ? a.n_split : 1;
  const int64_t heads = (int64_t)a.batch * a.heads * n_split;
  const DecodeLayout l =
      decode_layout(a.n_q, (int64_t)a.batch * a.heads, n_split, device_cus(), a.cache_fmt);
  a.n_qtiles = l.tiles[0] + l.tiles[1] + l.tiles[2];
  for (int i = 0; i < 3; ++i) a.mix[i] = l.mixed ? l.tiles[i] : 0;
  a.row_base = 0;
  if (l.tail > 0) {
    // 384-row tiles in the 12-wave kernel, then the 8-wave tail kernel from row 384 n3 on
    if (a.n_qtiles > 0)
      hipLaunchKernelGGL((attn_decode_direct<kCacheBf16, kDecodeDirectWaves>),
                         dim3((unsigned)(a.n_qtiles * heads)), dim3(64 * kDecodeDirectWaves), 0,
                         stream, a);
    AttnArgs t = a;
    t.row_base = 384 * l.tiles[0];
    t.n_qtiles = l.tail;
    t.mix[0] = t.mix[1] = t.mix[2] = 0;
    hipLaunchKernelGGL(attn_decode_tail, dim3((unsigned)(t.n_qtiles * heads)),
                       dim3(64 * kDecodeTailWaves), 0, stream, t);
    return hipGetLastError();
  }
  auto launch = [&](auto kernel, int waves) {
    const dim3 grid((unsigned)(a.n_qtiles * heads));
    hipLaunchKernelGGL(kernel, grid, dim3(64 * waves), 0, stream, a);
  };
  auto direct = [&](auto fmt_c) {
    constexpr int kF = decltype(fmt_c)::value;
    if (l.waves == kDecodeDirectWaves)
      launch(attn_decode_direct<kF, kDecodeDirectWaves>, kDecodeDirectWaves);
    else
      launch(attn_decode_direct<kF, kDecodeDirectSmallWaves>, kDecodeDirectSmallWaves);
  };
  switch (a.cache_fmt) {
    case kCacheBf16: direct(std::integral_constant<int, kCacheBf16>{}); break;
    case kCacheFp8V: direct(std::integral_constant<int, kCacheFp8V>{}); break;
    case kCacheFp8KV: direct(std::integral_constant<int, kCacheFp8KV>{}); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_split == 1) return e;
  const int64_t rows = (int64_t)a.batch * a.n_q * a.heads;
  hipLaunchKernelGGL(split_combine, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bca
