/*
 * bca.h -- C ABI of the block-causal attention library (libbca.so) for AMD MI355X (gfx950).
 *
 * What it computes.  One layer's attention of a single-stream diffusion transformer whose
 * sequence is [text][reference-image latents]...[target latents].  Position i may attend to key
 * j exactly when i >= j or when i and j lie in the same image block: text is strictly causal,
 * every image block is bidirectional inside, and blocks are causal in sequence order
 * ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo", section "Block-causal
 * attention is the cache-enabling boundary"; the 10100.com Qwen-Image 2.1 article, Block-Causal
 * mask part, which states the same rule as a boolean expression over positions and blocks).
 *
 * Shapes.  Multi-head attention (not GQA) with H heads of width D = 128; Q, K and V are
 * [B, S, H, D] bf16 with D contiguous (same guide, section "One stream for text, reference
 * images, and the target").  Outputs are fp32.
 *
 * Conventions for every call below.
 *  - All functions return a bca_status.  On failure nothing has been enqueued and
 *    bca_last_error() returns a description (thread-local, valid until the next failing call on
 *    the same thread).
 *  - Tensor pointers are DEVICE pointers owned by the caller.  bca_prefill and bca_decode never
 *    allocate and never synchronise; they enqueue on `stream` (a hipStream_t; NULL = the
 *    default stream) and return.
 *  - bca_tensor strides are in elements; the D stride is 1.  data must be 16-byte aligned;
 *    stride_b, stride_s and stride_h must be non-negative multiples of 8 (bf16) or 4 (fp32).
 *    For K, V and the caches, stride_s must be below 2^24 and rows * stride_s below 2^31 (rows
 *    within one (batch, head) slice are addressed with 32-bit offsets); else BCA_ERR_ARG.
 *  - scale is the softmax multiplier of q.k; 0 selects 1/sqrt(D).  Negative or NaN -> ARG.
 *  - Q, K and V must be finite: keys a row cannot see, inside a tile it computes, still enter the
 *    P.V product with weight 0, so an infinite or NaN value there would reach the output.
 */
#ifndef BCA_H
#define BCA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bca_status {
  BCA_OK = 0,
  BCA_ERR_ARG = 1,         /* bad size, pointer, stride, alignment, scale, or host-only plan */
  BCA_ERR_BLOCK_IDS = 2,   /* an id < -1, or an image id that occupies more than one run */
  BCA_ERR_UNSUPPORTED = 3, /* head width other than 128 */
  BCA_ERR_NO_DECODE = 4,   /* decode asked for a layout whose last block is text */
  BCA_ERR_ALLOC = 5,       /* host or device allocation failed (bca_plan only) */
  BCA_ERR_HIP = 6          /* a HIP call or kernel launch failed; text has hipGetErrorString */
} bca_status;

/* Opaque, immutable once built.  Independent of B and H: one plan serves every layer, every
 * denoising step, every stream and thread.  Free it only when no launch using it is in flight. */
typedef struct bca_plan_s* bca_plan_t;

typedef struct bca_tensor {
  void* data;       /* device pointer to element [0, 0, 0, 0] */
  int64_t stride_b; /* elements between consecutive batch entries */
  int64_t stride_s; /* elements between consecutive sequence positions */
  int64_t stride_h; /* elements between consecutive heads */
} bca_tensor;

typedef struct bca_plan_info {
  int64_t seq_len;      /* S */
  int64_t prefix_len;   /* P: start of the last block (text + reference positions before it);
                           a bca_plan_varlen plan: the sum of its sequences' P_b */
  int64_t target_len;   /* N = S - P; a bca_plan_varlen plan: the sum of its sequences' N_b */
  int64_t useful_pairs; /* number of visible (query, key) pairs per (batch, head) = sum of hi(i) */
  int32_t n_segments;   /* maximal runs of equal block id */
  int32_t block_m;      /* query rows per prefill tile */
  int32_t block_n;      /* keys per key tile */
  int32_t n_qtiles;     /* ceil(S / block_m) */
  int32_t decode_ok;    /* 1 when the last block (of every sequence) is an image block */
  int32_t host_only;    /* 1 when built with BCA_PLAN_HOST_ONLY (no device arrays) */
  int32_t n_sequences;  /* 1, or the batch of a bca_plan_varlen plan */
  int32_t reserved;     /* 0 */
  int64_t rows;         /* tensor rows the plan spans: S, or max(row_start + length) */
} bca_plan_info;

enum { BCA_PLAN_HOST_ONLY = 1u };

/*
 * bca_plan -- turn a per-position block-id vector into the launch plan.
 *
 * block_ids: HOST array [seq_len]; -1 marks text, k >= 0 marks image block k (same guide,
 * section "Block-causal attention is the cache-enabling boundary": -1 for text, a unique
 * non-negative id per reference image and another for the target; adjacent images keep distinct
 * ids).  Ids need not be increasing; an id >= 0 must form exactly one contiguous run (reuse is
 * rejected: BCA_ERR_BLOCK_IDS).  seq_len >= 1 and < 2^31.
 *
 * The plan holds, for every row i, its key limit hi(i): row i sees exactly the keys [0, hi(i)),
 * with hi(i) = i + 1 for text and the end of its block for image rows.  For text this is the
 * bottom-right aligned causal triangle of a segment whose query count is below its key count
 * (10100.com article, piecewise-attention part: a segment of q queries after k - q earlier keys
 * lets its query r see keys 0 .. k - q + r).
 * The rows are cut into n_qtiles tiles of block_m rows that end at the last row: tile t holds
 * rows [S - (n_qtiles - t) block_m, S - (n_qtiles - 1 - t) block_m) clipped at 0, so only tile 0
 * may be partial.  Per tile it stores kv_full[t] (min hi over its rows: key tiles below it need no
 * mask) and kv_end[t] (max hi: key tiles at or past it are skipped), and a heavy-first order.
 *
 * flags: 0, or BCA_PLAN_HOST_ONLY to skip the device upload (such a plan can be inspected but
 * not launched).  Without it, the plan owns small int32 device arrays on the current device
 * (one hipMalloc and one synchronous hipMemcpy, the only allocations in this library).
 * *out receives the plan; release it with bca_plan_free.
 */
bca_status bca_plan(const int32_t* block_ids, int64_t seq_len, uint32_t flags, bca_plan_t* out);

/*
 * bca_plan_varlen -- a plan for a batch of independent sequences with their own lengths and
 * block-id layouts (the guide's section "Block-causal attention is the cache-enabling boundary":
 * padded keys are ignored; the SenseNova-U1 infrastructure document, section "NEO-Unify 多模态
 * Prefill 的注意力": batches of long, mostly-text prompts).  Each sequence is planned as by
 * bca_plan; its query tiles never cross into another sequence, and all tiles of the batch run in
 * one heavy-first order.
 *
 * block_ids: HOST [sum(lengths)], the sequences' id vectors one after another (ids are local to
 * a sequence).  lengths: HOST int64 [batch], each >= 1.  row_start: HOST int64 [batch], the row of
 * the [rows, H, D] tensors where sequence b starts, or NULL for packed (row_start[b] =
 * sum_{c<b} lengths[c]).  Rows of different sequences must not overlap; gaps (padding) are
 * allowed and never read or written.  Exported arrays are concatenated over the sequences
 * (segments and row_limit local to each sequence).
 *
 * Each sequence b has its own prefix P_b (start of its last block) and target N_b = len_b - P_b,
 * as bca_plan defines them: the guide's section "The prefix cache is a compute-for-memory trade"
 * keeps one prefix cache per CFG branch, and the cond and uncond prompts differ in length.  The
 * batch's prefix caches are packed: sequence b's prefix K/V sit at cache rows [c_b, c_b + P_b)
 * with c_b = sum_{c<b} P_c, and its decode tensors (target Q/K/V and output) at target rows
 * [t_b, t_b + N_b) with t_b = sum_{c<b} N_c (bca_plan_sequences lists them).  Such a plan has
 * n_sequences = batch, prefix_len = sum P_b, target_len = sum N_b and decode_ok = 1 when every
 * sequence ends in an image block; it is launched with bca_prefill_varlen and bca_decode_varlen.
 */
bca_status bca_plan_varlen(const int32_t* block_ids, const int64_t* lengths,
                           const int64_t* row_start, int32_t batch, uint32_t flags,
                           bca_plan_t* out);

/*
 * Per sequence of a plan (one row for a bca_plan plan), six int64 written to out[6 b .. 6 b + 5]:
 * tensor row of its first position, length, prefix length P_b, target length N_b, first cache
 * row c_b, first target row t_b.  out must hold 6 * n_sequences values.
 */
bca_status bca_plan_sequences(bca_plan_t plan, int64_t* out);

/* Releases a plan (host and device arrays).  NULL is accepted and ignored. */
bca_status bca_plan_free(bca_plan_t plan);

/* Fills *out with the plan's scalars. */
bca_status bca_plan_get_info(bca_plan_t plan, bca_plan_info* out);

/*
 * Copies the plan's arrays to HOST buffers (any pointer may be NULL to skip it):
 *   segments [n_segments * 3]  (start, end exclusive, id) per maximal run
 *   row_limit [seq_len]        hi(i)
 *   kv_full, kv_end, order [n_qtiles]
 */
bca_status bca_plan_export(bca_plan_t plan, int32_t* segments, int32_t* row_limit,
                           int32_t* kv_full, int32_t* kv_end, int32_t* order);

/*
 * bca_prefill -- block-causal attention over the whole joint sequence (single-sequence plans;
 * a plan with n_sequences > 1 is BCA_ERR_ARG here) (the first denoising step,
 * "extract" in the guide's section "Timestep-zero conditioning makes the prefix invariant"),
 * optionally storing the per-layer prefix K/V cache.
 *
 *   o[b, i, h, :] = sum_{j < hi(i)} softmax_j(scale * q[b,i,h,:] . k[b,j,h,:]) v[b,j,h,:]
 *
 * q, k, v: bf16 [B, S, H, D] (S = the plan's seq_len).  o: fp32 [B, S, H, D], fully written.
 * k_cache, v_cache: bf16 [B, P, H, D] with P = the plan's prefix_len, or both NULL.  When given,
 * they receive copies of k[:, :P] and v[:, :P] (the guide clones the prefix slices rather than
 * keeping views).  The cache holds K as handed in (post-RoPE when the caller applied RoPE).
 * Output buffers must not overlap the inputs.  D must be 128 (else BCA_ERR_UNSUPPORTED).
 * The call is one attention launch, or two (bca_prefill_layout): the prefix rows, then the
 * target rows by the cached step's kernels over rows [0, P) of k and v as their prefix keys.
 * Every output row is bitwise the same either way.
 */
bca_status bca_prefill(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                       const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                       const bca_tensor* o, const bca_tensor* k_cache, const bca_tensor* v_cache,
                       void* stream);

/*
 * bca_prefill_layout -- HOST.  How bca_prefill and bca_prefill_ex launch a single-sequence plan
 * for B batch items and H heads on a GPU of `cus` compute units (0 = the current device's, 256
 * where the runtime cannot tell).  out[0] = attention launches (1 or 2); out[1] = query tiles per
 * (batch, head) of the prefill launch; out[2] = target rows handed to the second launch (0 with
 * one launch).  Two launches when the plan's last block is an image block after a non-empty
 * prefix, B * H * (the plan's query tiles) < 2 * cus (one launch would fill under two rounds of
 * the CUs), and the target rows alone fill at least one round of 384-row tiles
 * (ceil(N / 384) * B * H >= cus) in the cached step's 12-wave launch (bca_decode_layout
 * out[0] = 12 for n_q = N, batch_heads = B * H, a bf16 cache): the first launch then covers the
 * prefix rows [0, P) in query tiles of their own (out[1] of them, ending at row P) and stores
 * the cache, the second the target rows over all S keys.  Plans with several sequences take one
 * launch.  BCA_ERR_ARG for a NULL plan or out, B or H < 1, or cus < 0.
 */
bca_status bca_prefill_layout(bca_plan_t plan, int32_t B, int32_t H, int32_t cus, int32_t* out);

/*
 * bca_prefill_varlen -- block-causal attention of every sequence of a bca_plan_varlen plan (or of
 * the single sequence of a bca_plan plan): q, k, v bf16 and o fp32 are [rows, H, D] tensors
 * (bca_tensor with stride_b unused), sequence b at rows [row_start[b], row_start[b] + len_b).
 * Output rows of a sequence are fully written; rows outside every sequence are not touched.
 * k_cache, v_cache: bf16 [sum P_b, H, D] (stride_b unused), or both NULL.  When given, cache rows
 * [c_b, c_b + P_b) receive copies of sequence b's k and v rows [0, P_b) (its per-branch prefix
 * cache, packed as bca_plan_varlen describes).  D must be 128.
 */
bca_status bca_prefill_varlen(bca_plan_t plan, int32_t H, int32_t D, float scale,
                              const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                              const bca_tensor* o, const bca_tensor* k_cache,
                              const bca_tensor* v_cache, void* stream);

/*
 * bca_decode -- a cached denoising step: the N target queries attend with no mask to the
 * concatenation [cached prefix K/V ; current target K/V] (10100.com article, prefix-KV-cache
 * part: Query = current target latents, Key/Value = cached prefix K/V + current target K/V, one
 * full attention; guide, section "Two exact attention paths, with different operating
 * requirements").
 *
 *   o[b, n, h, :] = sum_{j < P + N} softmax_j(scale * q_tgt[b,n,h,:] . kk[b,j,h,:]) vv[b,j,h,:]
 *   with kk[j] = k_cache[j] for j < P and k_tgt[j - P] otherwise (same for vv).
 *
 * q_tgt, k_tgt, v_tgt: bf16 [B, N, H, D]; k_cache, v_cache: bf16 [B, P, H, D] (P, N from the
 * plan); o: fp32 [B, N, H, D].  The plan's last block must be an image block
 * (else BCA_ERR_NO_DECODE); a plan of several sequences is BCA_ERR_ARG here (bca_decode_varlen
 * takes it).  D must be 128.
 */
bca_status bca_decode(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                      const bca_tensor* q_tgt, const bca_tensor* k_cache,
                      const bca_tensor* v_cache, const bca_tensor* k_tgt,
                      const bca_tensor* v_tgt, const bca_tensor* o, void* stream);

/*
 * bca_decode_varlen -- the cached step of every sequence of a bca_plan_varlen plan in one launch
 * (the guide's section "The prefix cache is a compute-for-memory trade": the cond and uncond CFG
 * branches each keep their own prefix cache, of their own length).  Sequence b's N_b target
 * queries attend with no mask to [its cache rows ; its target keys]:
 *
 *   o[t_b + n, h, :] = sum_{j < P_b + N_b} softmax_j(scale * q_tgt[t_b + n, h, :] . kk_b[j, h, :])
 *                      vv_b[j, h, :],
 *   kk_b[j] = k_cache[c_b + j] for j < P_b, k_tgt[t_b + j - P_b] otherwise (same for vv_b).
 *
 * q_tgt, k_tgt, v_tgt: bf16 [sum N_b, H, D]; k_cache, v_cache: bf16 [sum P_b, H, D] (as
 * bca_prefill_varlen stores them; may be NULL when every P_b is 0); o: fp32 [sum N_b, H, D],
 * fully written.  stride_b is unused.  Every sequence must end in an image block (else
 * BCA_ERR_NO_DECODE); a bca_plan plan is accepted (one sequence).  D must be 128.
 */
bca_status bca_decode_varlen(bca_plan_t plan, int32_t H, int32_t D, float scale,
                             const bca_tensor* q_tgt, const bca_tensor* k_cache,
                             const bca_tensor* v_cache, const bca_tensor* k_tgt,
                             const bca_tensor* v_tgt, const bca_tensor* o, void* stream);

/*
 * bca_decode_layout -- HOST.  The launch shape the cached step (bca_decode, bca_decode_varlen,
 * bca_decode_ex, bca_decode_split) takes for n_q query rows per (batch, head) (for
 * bca_decode_varlen, the largest N_b), batch_heads = B * H, n_split key ranges (1 = unsplit) and
 * a cache of format cache_fmt, on a GPU of `cus` compute units (0 = the current device's, 256
 * where the runtime cannot tell).  out[0] = waves per workgroup (12 or 4) of the launch over the
 * query tiles out[1..3] per (batch, head, key range) of 384, 256 and 128 rows, laid along the rows
 * in that order (no such launch when all three are 0); out[4] = query tiles of 256 rows that a
 * launch of 8-wave workgroups takes from row 384 * out[1] on, after the first (0 = none).  The
 * tiles cover every row, and every tile holds one.
 *   Unsplit, with batch_heads and cus multiples of 8 (one share per XCD): 12-wave workgroups once
 *   384-row tiles would fill one round of the CUs (ceil(n_q / 384) * batch_heads >= cus).  Each
 *   XCD runs its (batch, head) entries' 384-row tiles, then their 256-row ones, then their 128-row
 *   ones, and the mix is the candidate (0..16 tiles of 256 rows, 0..2 of 128, as many of 384 as
 *   the rest needs) whose replayed list schedule on the XCD's CUs ends first.  The replay prices
 *   a tile at its busiest SIMD's step time, 1, 0.88 and 0.66 for 3, 2 and 1 waves with rows (the
 *   384-, 256- and 128-row tiles' ratios measured on an MI355X), plus 0.01; a tie keeps the
 *   candidate with fewer 256-row, then fewer 128-row tiles.
 *   With a bf16 cache and batch_heads >= 32 (4 entries per XCD) the step may instead take two
 *   launches: n3 tiles of 384 rows in the 12-wave kernel, then the rest in 256-row tiles of
 *   8-wave workgroups (2 waves per SIMD, 64-key fills), priced in whole rounds of the XCD's CUs
 *   at 1.01 and 0.737 per tile plus 0.02 for the second launch; the best n3 is taken when it
 *   replays at least 3% shorter than the mix.
 *   Unsplit and mixable under that round, with a bf16 cache: one round of 12-wave workgroups in
 *   384-row tiles (out[1] = ceil(n_q / 384)) when 256-row tiles would need a second round
 *   (ceil(n_q / 256) * batch_heads > cus); else every row in the 8-wave launch (out[1..3] = 0,
 *   out[4] = ceil(n_q / 256)) when its tiles fill more than half of the CUs
 *   (2 * ceil(n_q / 256) * batch_heads > cus).
 *   Otherwise: 12-wave workgroups in 384-row tiles where those give every CU at least two
 *   (not mixable, ceil(n_q / 384) * batch_heads * n_split >= 2 * cus).
 *   4-wave workgroups in 128-row tiles in the remaining cases.
 * A row's result does not depend on the tile or launch that holds it.  BCA_ERR_ARG for n_q or
 * batch_heads outside [1, 2^31 - 1], n_split < 1, batch_heads * n_split >= 2^31, an unknown
 * cache_fmt, cus < 0 or out NULL.
 */
bca_status bca_decode_layout(int64_t n_q, int64_t batch_heads, int32_t n_split, int32_t cache_fmt,
                             int32_t cus, int32_t* out);

/*
 * FP8 prefix cache (10100.com article, FP8 part: the prefix K/V cache may be stored as FP8 E4M3
 * with one fp32 scale per token and attention head; quantising V alone keeps K exact, which the
 * article finds the safer trade, and still saves about a quarter of the cache).
 *
 * Formats.  BCA_CACHE_BF16: K and V bf16 [B, P, H, D].  BCA_CACHE_FP8_V: K bf16, V quantised.
 * BCA_CACHE_FP8_KV: both quantised.  A quantised tensor is a uint8 code tensor [B, P, H, D]
 * (OCP E4M3FN: bias 7, largest finite 448, subnormals, no infinities, 0x7F/0xFF = NaN) plus an
 * fp32 scale tensor [B, P, H].  For each (b, j, h) row x of D values:
 *     amax  = max_d |x[d]|
 *     scale = 2^k, the smallest power of two with amax <= 448 * 2^k and k >= -126; 1 if amax = 0
 *     code[d] = E4M3(x[d] * 2^-k)  (an exact fp32 product, then the nearest E4M3 value, ties to
 *                                   even; it never exceeds 448)
 * and the value the decode uses is E4M3 value(code[d]) * scale, which bf16 holds exactly (down to
 * bf16's smallest normal number; below it, rounded to nearest even).  The row's largest value
 * lands in E4M3's top binade, so the power-of-two scale costs no relative precision.  Inputs must
 * be finite.
 *
 * Layout rules on top of the general ones: code tensors follow the bf16 rules with 1-byte
 * elements (data 16-byte aligned, strides non-negative multiples of 16); scale tensors are fp32
 * with data 4-byte aligned and non-negative strides (stride_h is the element stride between
 * heads), stride_s below 2^24 and P * stride_s below 2^29 elements.  A scale tensor that its
 * format does not use is ignored (data may be NULL).
 */
typedef enum bca_cache_format {
  BCA_CACHE_BF16 = 0,
  BCA_CACHE_FP8_V = 1,
  BCA_CACHE_FP8_KV = 2
} bca_cache_format;

typedef struct bca_kv_cache {
  int32_t format;      /* a bca_cache_format */
  bca_tensor k;        /* bf16 [B, P, H, D], or uint8 codes [B, P, H, D] for BCA_CACHE_FP8_KV */
  bca_tensor v;        /* bf16 [B, P, H, D], or uint8 codes for BCA_CACHE_FP8_V / _FP8_KV */
  bca_tensor k_scale;  /* fp32 [B, P, H]: used by BCA_CACHE_FP8_KV */
  bca_tensor v_scale;  /* fp32 [B, P, H]: used by BCA_CACHE_FP8_V and BCA_CACHE_FP8_KV */
} bca_kv_cache;

/*
 * bca_prefill_ex -- bca_prefill with the prefix cache given as a descriptor of any format (NULL:
 * no cache).  The attention itself always uses the bf16 k and v; only the stored cache is
 * quantised, by the rule above: the attention kernel stores the cache's bf16 tensors, and a second
 * kernel on the same stream quantises rows [0, P) of k and v into the code and scale tensors.
 * Ownership, errors and the other arguments are those of bca_prefill; an unknown format is
 * BCA_ERR_ARG.
 */
bca_status bca_prefill_ex(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                          const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                          const bca_tensor* o, const bca_kv_cache* cache, void* stream);

/*
 * bca_decode_ex -- bca_decode reading the prefix from a cache of any format.  Quantised rows are
 * brought on chip as codes and scales and dequantised there into the kernel's bf16 tiles
 * (value * scale, rounded to bf16); nothing is written back.  cache may be NULL only when the plan's prefix_len is 0.
 */
bca_status bca_decode_ex(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                         const bca_tensor* q_tgt, const bca_kv_cache* cache,
                         const bca_tensor* k_tgt, const bca_tensor* v_tgt, const bca_tensor* o,
                         void* stream);

/*
 * bca_cache_dequantize -- writes a prefix cache of any format back as bf16: k_out, v_out bf16
 * [B, P, H, D] receive E4M3(code) * scale formed in fp32 and rounded to bf16 (RNE) for a quantised
 * tensor, a copy for a bf16 one.  That is the value bca_decode_ex uses for the same code, so the
 * decode over the expanded cache sees bitwise the K and V of bca_decode_ex over the FP8 one, and
 * the two outputs are bitwise equal (both decodes walk the same bf16 tiles).
 * Meant for expanding one layer's FP8 cache into a transient buffer just before that layer's
 * cached step (the FP8 form keeps the memory of all layers; the bf16 decode is the faster one).
 * The outputs must not overlap the cache.  D must be 128.  Enqueues one kernel on stream.
 */
bca_status bca_cache_dequantize(int32_t B, int64_t P, int32_t H, int32_t D,
                                const bca_kv_cache* cache, const bca_tensor* k_out,
                                const bca_tensor* v_out, void* stream);

/*
 * Q/K prologue ("Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo": section
 * "One stream for text, reference images, and the target" normalises Q and K per head before
 * RoPE; section "Three-axis RoPE preserves image geometry" splits a head's 128 dims (16, 56, 56)
 * over frame, height and width, base 10,000, advances text on all three axes together and gives
 * an image the frame reached by preceding text plus a height/width grid centred on zero).
 * Readings where the pages are silent: a counter c starts at 0; a text token takes (c, c, c) and
 * advances c; an H x W image block (row-major) takes (c, h - H/2, w - W/2) and then advances c by
 * one; rotation pairs are adjacent dims (2i, 2i + 1); pair k of an axis of width d turns by
 * pos * base^(-2k/d); the RMS norm is x / sqrt(mean(x^2) + eps) * w with w[128] shared by heads.
 */

/*
 * bca_rope_positions -- HOST.  pos_out[3 * i + {0, 1, 2}] = (frame, height, width) of position i
 * of the block-id layout (same ids and rules as bca_plan).  image_hw: NULL (every image block is
 * square) or [n_images][2] = (H, W) of each image block in sequence order; H * W must equal the
 * block's length (else BCA_ERR_ARG).  pos_out: HOST int32 [seq_len][3].
 */
bca_status bca_rope_positions(const int32_t* block_ids, int64_t seq_len, const int32_t* image_hw,
                              int32_t n_images, int32_t* pos_out);

/*
 * bca_rope_table -- HOST.  table_out[(i * 64 + p) * 2 + {0, 1}] = {cos, sin} of the angle of
 * rotation pair p at position i (pairs 0..7 frame, 8..35 height, 36..63 width), computed in
 * double and rounded to float.  pos: HOST int32 [n][3]; table_out: HOST float [n][64][2].  Copy
 * it to the device for bca_qk_prologue; one table serves every layer, head and step.
 */
bca_status bca_rope_table(const int32_t* pos, int64_t n, double base, float* table_out);

/*
 * bca_qk_prologue -- q_out = RoPE(RMSNorm(q) * q_weight) and k_out likewise, for S positions:
 * q, k, q_out, k_out bf16 [B, S, H, D] (D = 128; bca_tensor rules); q_weight, k_weight DEVICE
 * fp32 [D]; rope_table DEVICE fp32 [S][64][2] from bca_rope_table for the same S positions (for a
 * cached step, the table rows of the target).  eps >= 0.  fp32 arithmetic, bf16 (RNE) output.
 * q_out may be q itself (in place), and k_out k; other overlaps are not allowed.  The prefill
 * then stores the post-RoPE K it is given in the prefix cache.  Enqueues one kernel on stream.
 */
bca_status bca_qk_prologue(int32_t B, int64_t S, int32_t H, int32_t D, float eps,
                           const bca_tensor* q, const bca_tensor* k, const bca_tensor* q_out,
                           const bca_tensor* k_out, const float* q_weight, const float* k_weight,
                           const float* rope_table, void* stream);

/*
 * Split-KV decode.  The cached step of bca_decode_ex (same arguments and result; the guide's
 * section "Two exact attention paths, with different operating requirements") for targets too
 * small to fill the GPU, e.g. a 512 x 512 target (N = 1,024) under a long prefix: each
 * (batch, head, query tile) is cut into n_split key ranges, each a whole number of 64-key
 * units (the last may be shorter), handled by separate workgroups.  Each range leaves its unnormalised output, running maximum m (base 2, scaled) and
 * row sum l in a caller workspace; a second kernel merges them:
 *     O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,   M = max_c m_c,
 * which is the same softmax up to rounding.
 *
 * bca_decode_split_workspace -- HOST.  *bytes = workspace bytes for (plan, B, H, n_split);
 * n_split = 0 lets the library choose: one range where the unsplit decode already has 768
 * workgroups of 128 query rows per (batch, head) tile (three per CU on 256 CUs), else the count n
 * that best fills whole rounds of 768 workgroups (minimising ceil(768-unit rounds) / n + n / 100),
 * with ranges of at least 8 units of 64 keys; at most one range per unit.  *n_split_used (may be
 * NULL) = the number of ranges it will use (1 = plain decode, bytes = 0).  Neither depends on the cache format.  The plan's last block must be an image block (else BCA_ERR_NO_DECODE).
 *
 * bca_decode_split -- as bca_decode_ex, plus n_split (>= 0) and a DEVICE workspace of at least
 * that many bytes, 16-byte aligned, owned by the caller and not used by anything else while the
 * call runs (it may be NULL when n_split_used is 1).  Enqueues two kernels on stream.
 */
bca_status bca_decode_split_workspace(bca_plan_t plan, int32_t B, int32_t H, int32_t n_split,
                                      int64_t* bytes, int32_t* n_split_used);
bca_status bca_decode_split(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                            const bca_tensor* q_tgt, const bca_kv_cache* cache,
                            const bca_tensor* k_tgt, const bca_tensor* v_tgt, const bca_tensor* o,
                            int32_t n_split, void* workspace, int64_t workspace_bytes,
                            void* stream);

/*
 * bca_decode_split_noalloc -- for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): bca_decode_split with the
 * same arguments and result, minus the workspace.  The key ranges' partial results go to a
 * scratch buffer the library owns: BCA_SCRATCH_BYTES (64 MiB) of device memory per GPU, reserved
 * when the library is loaded on that GPU and held until the process ends.  This call allocates
 * nothing (its first call on a device looks up that device's copy of the buffer once).  A split
 * whose partial results (bca_decode_split_workspace's bytes) exceed BCA_SCRATCH_BYTES is
 * BCA_ERR_ARG and enqueues nothing; one range (n_split_used = 1) uses no scratch.  Every call on
 * one GPU shares its scratch, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that may overlap on one GPU (different streams, or threads racing on one)
 * race on it and must be ordered by the caller.  Enqueues two kernels on stream (one when
 * unsplit).
 */
#define BCA_SCRATCH_BYTES (64ll << 20)
bca_status bca_decode_split_noalloc(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                                    const bca_tensor* q_tgt, const bca_kv_cache* cache,
                                    const bca_tensor* k_tgt, const bca_tensor* v_tgt,
                                    const bca_tensor* o, int32_t n_split, void* stream);

/* Static name of a status code ("BCA_OK", ...); "unknown status" for other values. */
const char* bca_status_str(bca_status status);

/* Thread-local text of the last failure on this thread ("" if none). */
const char* bca_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BCA_H */
