// Internal interface between the host side of libbca (planner, validation) and the gfx950
// kernels.  Not installed; the public ABI is include/bca.h.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "bca_plan.h"  // kTileInts: ints per prefill tile descriptor

namespace bca {

// Tile shape.  A wave owns kQueryBlocks blocks of 32 query rows, and a workgroup's query rows
// form one tile.  Per kernel: waves per workgroup, keys per key tile and waves per SIMD.  The
// prefill and the decode (any cache format) are filled by direct loads and run 32-key tiles at 3
// waves per SIMD; their workgroups have 12 waves (one workgroup per CU), so each K/V tile loaded
// into LDS serves 384 query rows.  A decode whose 12-wave grid would not give every CU two
// workgroups runs 4-wave ones instead.
constexpr int kHeadDim = 128;  // the only head width the kernels are built for
constexpr int kQueryBlocks = 1;
constexpr int kPrefillWaves = 12;
constexpr int kDecodeDirectWaves = 12;      // large decode grids
constexpr int kDecodeDirectSmallWaves = 4;  // small decode grids
constexpr int kBlockM = 32 * kQueryBlocks * kPrefillWaves;  // prefill query tile (= plan tile)
// Fewest query rows any decode workgroup takes (bounds the decode's grid).
constexpr int kDecodeMinBlockM = 32 * kQueryBlocks * 4;
constexpr int kPrefillBlockN = 32;
constexpr int kPrefillWavesPerSimd = 3;
constexpr int kDecodeDirectBlockN = 32;
constexpr int kDecodeDirectWavesPerSimd = 3;
constexpr int kDecodeTailWaves = 8;    // decode tail launch: 256-row tiles
constexpr int kDecodeTailBlockN = 64;  // ... filled 64 keys at a time
// A split decode's key ranges are whole multiples of kSplitUnit keys, whatever the kernel's tile
// width (which divides it), so the workspace a plan needs does not depend on the cache format.
constexpr int kSplitUnit = 64;
static_assert(kSplitUnit % kDecodeDirectBlockN == 0, "split units hold whole key tiles");

// Prefix-cache storage formats (values of bca_cache_format).
constexpr int kCacheBf16 = 0;   // K and V bf16
constexpr int kCacheFp8V = 1;   // V as E4M3 codes + fp32 scale per (token, head)
constexpr int kCacheFp8KV = 2;  // K and V as E4M3 codes + scales

// One attention launch.  Prefill and decode share the kernel: keys j < split come from (k, v),
// keys j >= split from (k2, v2) at index j - split.  Prefill sets split = kv_len.  k and v are
// bf16, except in a decode over a quantised cache, where the quantised one holds uint8 codes
// (strides in bytes) and kcs / vcs hold its scales.
struct AttnArgs {
  const uint16_t* q;
  int64_t q_sb, q_ss, q_sh;
  const void* k;
  int64_t k_sb, k_ss, k_sh;
  const void* v;
  int64_t v_sb, v_ss, v_sh;
  const uint16_t* k2;
  int64_t k2_sb, k2_ss, k2_sh;
  const uint16_t* v2;
  int64_t v2_sb, v2_ss, v2_sh;
  float* o;
  int64_t o_sb, o_ss, o_sh;
  // Prefill only: bf16 prefix-cache tensors receiving each sequence's K/V rows [0, P) at cache
  // rows [cache_row, cache_row + P) (both from the tile descriptors), or NULL (no cache, or a
  // quantised tensor, which launch_quantize writes).  The workgroup of a query tile writes the
  // tile's own rows of them.
  void* kc;
  int64_t kc_sb, kc_ss, kc_sh;
  void* vc;
  int64_t vc_sb, vc_ss, vc_sh;
  int32_t n_q;       // query rows per (batch, head): S for prefill, N for decode
  int32_t kv_len;    // keys per (batch, head): S for prefill, P + N for decode
  int32_t split;     // first key taken from the second source
  int32_t heads;
  int32_t batch;
  int32_t n_qtiles;  // ceil(n_q / query rows per workgroup); launch_decode sets it itself
  float scale_log2;  // softmax scale * log2(e)
  // Prefill only (NULL for decode): per-row key limit and per-tile ranges / order.
  const int32_t* row_limit;
  const int32_t* kv_full;
  const int32_t* kv_end;
  const int32_t* order;
  // Prefill only: per query tile {sequence's first tensor row, first local row (negative for a
  // partial first tile, whose rows below 0 are padding), sequence length,
  // offset of the sequence's row limits, kv_full, kv_end, prefix length P, first cache row};
  // row_limit and the key bounds are local to the sequence.
  const int32_t* tiles;
  // Decode over a batch of sequences (NULL otherwise): per batch entry b, kSeqInts ints of which
  // [2] = P_b, [3] = N_b, [4] = first cache row, [5] = first target row.  Entry b then takes its
  // n_q = N_b queries at rows [5] + n of q / o, its keys from cache rows [4] + j (j < P_b) and
  // target rows [5] + j - P_b; batch strides are unused and n_q is the largest N_b.
  const int32_t* seqs;
  // Decode only: scales [B, cache_len, H] of the quantised cache tensors (NULL for a bf16 one).
  float* kcs;
  int64_t kcs_sb, kcs_ss, kcs_sh;
  float* vcs;
  int64_t vcs_sb, vcs_ss, vcs_sh;
  int32_t cache_fmt;  // decode only: kCacheBf16 / kCacheFp8V / kCacheFp8KV
  // Decode only: key ranges of split_units x kSplitUnit keys each, n_split of them (1 = no
  // split), whose partial results go to part_o [n_split][B][N][H][D] and part_ml
  // [n_split][B][N][H][2] (m, l) and are merged into o by a second kernel.
  int32_t n_split;
  int32_t split_units;
  float* part_o;
  float* part_ml;
  // Decode, 12-wave kernel: query tiles per (batch, head) of 384, 256 and 128 rows (mix[0..2]),
  // laid out along the rows in that order.  Each XCD takes the tiles of its own (batch, head)
  // entries, all 384-row tiles first, then the 256-row ones, then the 128-row ones.  mix[0] == 0:
  // every tile 384 rows, (batch, head)-major (launch_decode fills it in).
  int32_t mix[3];
  // Decode tail launch (attn_decode_tail): first query row of its tile 0 in every (batch, head).
  int32_t row_base;
};

// Q/K prologue: RMS-normalise each 128-value head row of q and k (weights wq, wk), rotate its
// adjacent pairs by the position's angles (table [S][64][2] of {cos, sin}), store bf16.
struct PrologueArgs {
  const uint16_t* q;
  int64_t q_sb, q_ss, q_sh;
  const uint16_t* k;
  int64_t k_sb, k_ss, k_sh;
  uint16_t* qo;
  int64_t qo_sb, qo_ss, qo_sh;
  uint16_t* ko;
  int64_t ko_sb, ko_ss, ko_sh;
  const float* wq;
  const float* wk;
  const float* table;
  int64_t rows;  // B * S * H head rows
  int32_t seq;   // S
  int32_t heads;
  float eps;
};

// Cache expansion: K and V of a prefix cache (any format) written as bf16 [B, P, H, D].  A
// quantised tensor's values are E4M3(code) * scale in fp32, rounded to bf16 (RNE); a bf16 tensor
// is copied.
struct DequantArgs {
  const void* k;
  int64_t k_sb, k_ss, k_sh;
  const void* v;
  int64_t v_sb, v_ss, v_sh;
  const float* ks;
  int64_t ks_sb, ks_ss, ks_sh;
  const float* vs;
  int64_t vs_sb, vs_ss, vs_sh;
  uint16_t* ko;
  int64_t ko_sb, ko_ss, ko_sh;
  uint16_t* vo;
  int64_t vo_sb, vo_ss, vo_sh;
  int64_t rows;  // B * P * H
  int32_t prefix;
  int32_t heads;
  int32_t fmt;   // kCacheBf16 / kCacheFp8V / kCacheFp8KV
};

// Cache quantisation: prefix rows [0, P) of bf16 K and V [B, S, H, D] written as E4M3 codes
// [B, P, H, D] plus one fp32 scale per (b, p, h) for each tensor with a code pointer (ko, vo;
// NULL: that tensor is not quantised).  The rule is the cache format's (scale = the smallest power
// of two 2^k >= amax / 448 with k >= -126, 1 for an all-zero row; codes = E4M3(x * 2^-k), RNE).
struct QuantArgs {
  const uint16_t* k;
  int64_t k_sb, k_ss, k_sh;
  const uint16_t* v;
  int64_t v_sb, v_ss, v_sh;
  uint8_t* ko;
  int64_t ko_sb, ko_ss, ko_sh;
  float* ks;
  int64_t ks_sb, ks_ss, ks_sh;
  uint8_t* vo;
  int64_t vo_sb, vo_ss, vo_sh;
  float* vs;
  int64_t vs_sb, vs_ss, vs_sh;
  int64_t rows;  // B * P * H
  int32_t prefix;
  int32_t heads;
};

// Device scratch owned by the library for the allocation-free split decode: kScratchBytes per
// GPU.  scratch_memory returns the current device's copy (its address is looked up once per
// device); it allocates nothing.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
hipError_t scratch_memory(void** out);

hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t stream);
hipError_t launch_decode(const AttnArgs& a, hipStream_t stream);

// Launch shape of the decode: n_q query rows per (batch, head), `groups` = B * H, n_split key
// ranges, on a device of `cus` compute units.  tiles: query tiles per (batch, head, key range) of
// 384, 256 and 128 rows, laid along the rows in that order.
//   Unsplit, groups and cus multiples of the 8 XCDs: 12-wave workgroups with the mix decode_mix
//   picks (mixed = true) once 384-row tiles would fill one round of the CUs; under that round,
//   with a bf16 cache, one round of 384-row tiles {ceil(n_q / 384), 0, 0} (mixed = true) when
//   256-row tiles would need a second round, else every row in the tail kernel (tiles all 0,
//   tail = ceil(n_q / 256)) when its tiles fill more than half of the CUs; else 4-wave ones.
//   Otherwise: 12-wave workgroups in 384-row tiles {ceil(n_q / 384), 0, 0} where those give every
//   CU at least two, else 4-wave ones.  4 waves: {0, 0, ceil(n_q / 128)}.
//   With a bf16 cache, an unsplit mixed launch may instead be two launches (tail > 0): tiles[0]
//   384-row tiles in the 12-wave kernel (mixed = true, tiles[1] = tiles[2] = 0), then `tail`
//   256-row tiles of the 8-wave tail kernel from row 384 * tiles[0] on.  tail > 0 only for
//   unsplit launches (launch_decode merges key ranges after the one-kernel launches only).
struct DecodeLayout {
  int waves;
  int32_t tiles[3];
  bool mixed;
  int32_t tail;
};
DecodeLayout decode_layout(int64_t n_q, int64_t groups, int n_split, int cus, int cache_fmt);
// Compute units of the current device (256 where the runtime cannot tell).
int device_cus();

}  // namespace bca
