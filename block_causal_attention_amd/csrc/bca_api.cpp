// C ABI of libbca (include/bca.h): argument validation, plan ownership, launches.
// Every check runs on the host before anything is enqueued.
#include "bca.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "bca_internal.h"
#include "bca_plan.h"

struct bca_plan_s {
  bca::HostPlan host;
  int32_t host_only = 1;
  int device = -1;
  // One device allocation holds every plan array (uploaded with one copy); the pointers below
  // point into it.
  void* d_arena = nullptr;
  int32_t* d_row_limit = nullptr;
  int32_t* d_kv_full = nullptr;
  int32_t* d_kv_end = nullptr;
  int32_t* d_order = nullptr;
  int32_t* d_tiles = nullptr;
  int32_t* d_seqs = nullptr;
  int32_t* d_prefix_tiles = nullptr;
  int32_t* d_prefix_order = nullptr;
};

namespace {

constexpr int64_t kHeadDimElems = bca::kHeadDim;
static_assert(BCA_SCRATCH_BYTES == bca::kScratchBytes, "bca.h states the scratch size");
thread_local std::string g_last_error;

bca_status fail(bca_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bca_status hip_fail(hipError_t e, const char* what) {
  return fail(BCA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

void free_device(bca_plan_s* p) {
  if (p->d_arena) (void)hipFree(p->d_arena);
  p->d_arena = nullptr;
  p->d_row_limit = p->d_kv_full = p->d_kv_end = p->d_order = p->d_tiles = p->d_seqs = nullptr;
  p->d_prefix_tiles = p->d_prefix_order = nullptr;
}

// The plan's device arrays: packed into one host staging buffer (each array starting on a
// 256-byte boundary), then one hipMalloc and one synchronous hipMemcpy.
bca_status upload(bca_plan_s* p) {
  const bca::HostPlan& h = p->host;
  constexpr int kArrays = 8;
  const std::vector<int32_t>* src[kArrays] = {&h.row_limit, &h.kv_full, &h.kv_end,
                                              &h.order,     &h.tiles,   &h.seqs,
                                              &h.prefix_tiles, &h.prefix_order};
  int32_t** dst[kArrays] = {&p->d_row_limit, &p->d_kv_full, &p->d_kv_end,
                            &p->d_order,     &p->d_tiles,   &p->d_seqs,
                            &p->d_prefix_tiles, &p->d_prefix_order};
  constexpr size_t kAlignInts = 64;
  size_t off[kArrays], total = 0;
  for (int i = 0; i < kArrays; ++i) {
    off[i] = total;
    total += (src[i]->size() + kAlignInts - 1) / kAlignInts * kAlignInts;
  }
  std::vector<int32_t> staging(total, 0);
  for (int i = 0; i < kArrays; ++i)
    std::copy(src[i]->begin(), src[i]->end(), staging.begin() + (ptrdiff_t)off[i]);
  hipError_t e = hipMalloc(&p->d_arena, total * sizeof(int32_t));
  if (e != hipSuccess) {
    p->d_arena = nullptr;
    return fail(BCA_ERR_ALLOC, std::string("hipMalloc of the plan arrays: ") +
                                   hipGetErrorString(e));
  }
  e = hipMemcpy(p->d_arena, staging.data(), total * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy of the plan arrays");
  for (int i = 0; i < kArrays; ++i) *dst[i] = static_cast<int32_t*>(p->d_arena) + off[i];
  return BCA_OK;
}

// A tensor descriptor must point at 16-byte aligned memory with strides that keep every row
// 16-byte aligned (8 bf16 or 4 fp32 elements).
bca_status check_tensor(const bca_tensor* t, const char* name, int elem_bytes) {
  if (t == nullptr) return fail(BCA_ERR_ARG, std::string(name) + ": descriptor is NULL");
  if (t->data == nullptr) return fail(BCA_ERR_ARG, std::string(name) + ": data is NULL");
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(BCA_ERR_ARG, std::string(name) + ": data is not 16-byte aligned");
  const int64_t q = 16 / elem_bytes;
  const int64_t st[3] = {t->stride_b, t->stride_s, t->stride_h};
  for (int64_t s : st)
    if (s < 0 || s % q != 0)
      return fail(BCA_ERR_ARG, std::string(name) + ": strides must be non-negative multiples of " +
                                   std::to_string(q) + " elements");
  return BCA_OK;
}

// Size, head width and scale checks; they need no device, so they run first.
bca_status check_common(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                        float* scale_log2) {
  if (plan == nullptr) return fail(BCA_ERR_ARG, "plan is NULL");
  if (B < 1 || H < 1) return fail(BCA_ERR_ARG, "B and H must be >= 1");
  if (D != bca::kHeadDim)
    return fail(BCA_ERR_UNSUPPORTED, "head width " + std::to_string(D) + " (only 128 is built)");
  if (std::isnan(scale) || scale < 0.0f || std::isinf(scale))
    return fail(BCA_ERR_ARG, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  const double sc = scale == 0.0f ? 1.0 / std::sqrt((double)D) : (double)scale;
  *scale_log2 = (float)(sc * 1.4426950408889634);  // log2(e)
  return BCA_OK;
}

// The plan must own device arrays on the current device.
bca_status check_launchable(bca_plan_t plan) {
  if (plan->host_only) return fail(BCA_ERR_ARG, "plan was built with BCA_PLAN_HOST_ONLY");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(BCA_ERR_ARG, "plan lives on device " + std::to_string(plan->device) +
                                 " but device " + std::to_string(dev) + " is current");
  return BCA_OK;
}

// K and V rows are addressed with 32-bit element offsets inside one (batch, head) slice: the row
// stride must stay below 2^24 elements and rows * stride below 2^31.
bca_status check_extent(const bca_tensor* t, const char* name, int64_t rows) {
  if (t->stride_s >= (int64_t(1) << 24))
    return fail(BCA_ERR_ARG, std::string(name) + ": stride_s must be below 2^24 elements");
  if (rows * t->stride_s + kHeadDimElems >= (int64_t(1) << 31))
    return fail(BCA_ERR_ARG, std::string(name) + ": rows * stride_s must be below 2^31 elements");
  return BCA_OK;
}

// A scale tensor: fp32, 4-byte aligned, non-negative strides; like K and V, rows of one (batch,
// head) slice are addressed with 32-bit offsets.
bca_status check_scale_tensor(const bca_tensor* t, const char* name, int64_t rows) {
  if (t->data == nullptr) return fail(BCA_ERR_ARG, std::string(name) + ": data is NULL");
  if (reinterpret_cast<uintptr_t>(t->data) % 4 != 0)
    return fail(BCA_ERR_ARG, std::string(name) + ": data is not 4-byte aligned");
  if (t->stride_b < 0 || t->stride_s < 0 || t->stride_h < 0)
    return fail(BCA_ERR_ARG, std::string(name) + ": strides must be non-negative");
  if (t->stride_s >= (int64_t(1) << 24))
    return fail(BCA_ERR_ARG, std::string(name) + ": stride_s must be below 2^24 elements");
  if (rows * t->stride_s + 1 >= (int64_t(1) << 29))
    return fail(BCA_ERR_ARG, std::string(name) + ": rows * stride_s must be below 2^29 elements");
  return BCA_OK;
}

// A prefix cache of `rows` positions: format, then each tensor by its storage type.
bca_status check_format(const bca_kv_cache* c) {
  if (c->format != BCA_CACHE_BF16 && c->format != BCA_CACHE_FP8_V &&
      c->format != BCA_CACHE_FP8_KV)
    return fail(BCA_ERR_ARG, "cache: unknown format " + std::to_string(c->format));
  return BCA_OK;
}

bca_status check_cache(const bca_kv_cache* c, int64_t rows) {
  bca_status s = check_format(c);
  if (s != BCA_OK) return s;
  const bool kq = c->format == BCA_CACHE_FP8_KV;
  const bool vq = c->format != BCA_CACHE_BF16;
  if ((s = check_tensor(&c->k, kq ? "cache.k (codes)" : "cache.k", kq ? 1 : 2)) != BCA_OK) return s;
  if ((s = check_tensor(&c->v, vq ? "cache.v (codes)" : "cache.v", vq ? 1 : 2)) != BCA_OK) return s;
  if ((s = check_extent(&c->k, "cache.k", rows)) != BCA_OK) return s;
  if ((s = check_extent(&c->v, "cache.v", rows)) != BCA_OK) return s;
  if (kq && (s = check_scale_tensor(&c->k_scale, "cache.k_scale", rows)) != BCA_OK) return s;
  if (vq && (s = check_scale_tensor(&c->v_scale, "cache.v_scale", rows)) != BCA_OK) return s;
  return BCA_OK;
}

void set_cache_args(const bca_kv_cache* c, bca::AttnArgs* a) {
  a->cache_fmt = c->format;
  if (c->format == BCA_CACHE_FP8_KV) {
    a->kcs = static_cast<float*>(c->k_scale.data);
    a->kcs_sb = c->k_scale.stride_b; a->kcs_ss = c->k_scale.stride_s; a->kcs_sh = c->k_scale.stride_h;
  }
  if (c->format != BCA_CACHE_BF16) {
    a->vcs = static_cast<float*>(c->v_scale.data);
    a->vcs_sb = c->v_scale.stride_b; a->vcs_ss = c->v_scale.stride_s; a->vcs_sh = c->v_scale.stride_h;
  }
}

// A bf16 cache descriptor from the plain entry points' pair of tensors.
bca_kv_cache bf16_cache(const bca_tensor* k_cache, const bca_tensor* v_cache) {
  bca_kv_cache c{};
  c.format = BCA_CACHE_BF16;
  c.k = *k_cache;
  c.v = *v_cache;
  return c;
}

// A launch of `groups` workgroups of `threads` work-items: a dispatch counts at most 2^32 - 1
// work-items per grid dimension.
bool grid_fits(int64_t groups, int64_t threads) {
  return groups >= 0 && groups <= (int64_t)UINT32_MAX / threads;
}
// The attention grids: tiles * B * H workgroups of the prefill's size, the largest any
// attention kernel uses.
bool grid_fits(int64_t tiles, int32_t B, int32_t H) {
  return tiles <= (int64_t)INT32_MAX / ((int64_t)B * H) &&
         grid_fits(tiles * B * H, 64 * bca::kPrefillWaves);
}

// Whether a single-sequence prefill hands its target rows (the last block, an image block:
// rows [P, S)) to the decode kernels.  That happens when its own grid of B * H * query tiles
// would fill less than two rounds of the CUs while the target rows alone fill at least one round
// of 384-row tiles and so take the decode's 12-wave launch, whose query tiles of mixed heights
// fill whole rounds; the prefix rows then run first in a prefill launch of their own.  A row's
// arithmetic is the same either way (the same 32-key tiles in the same order).
bool prefill_hands_off(const bca::HostPlan& hp, int32_t B, int32_t H, int cus) {
  if (hp.n_sequences != 1 || hp.prefix_tiles.empty()) return false;
  const int64_t groups = (int64_t)B * H;
  if ((int64_t)hp.kv_end.size() * groups >= 2 * (int64_t)cus) return false;
  if ((hp.target_len + 383) / 384 * groups < (int64_t)cus) return false;
  return bca::decode_layout(hp.target_len, groups, 1, cus, bca::kCacheBf16).waves ==
         bca::kDecodeDirectWaves;
}

}  // namespace

namespace bca {
// Error reporting for the other host files of the library (same thread-local text).
bca_status set_error(bca_status s, const std::string& msg) { return fail(s, msg); }
}  // namespace bca

extern "C" {

const char* bca_status_str(bca_status s) {
  switch (s) {
    case BCA_OK: return "BCA_OK";
    case BCA_ERR_ARG: return "BCA_ERR_ARG";
    case BCA_ERR_BLOCK_IDS: return "BCA_ERR_BLOCK_IDS";
    case BCA_ERR_UNSUPPORTED: return "BCA_ERR_UNSUPPORTED";
    case BCA_ERR_NO_DECODE: return "BCA_ERR_NO_DECODE";
    case BCA_ERR_ALLOC: return "BCA_ERR_ALLOC";
    case BCA_ERR_HIP: return "BCA_ERR_HIP";
  }
  return "unknown status";
}

const char* bca_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Builds the host plan with `build`, then (unless host-only) uploads its arrays.
template <typename Build>
bca_status make_plan(uint32_t flags, bca_plan_t* out, Build build) {
  if (out == nullptr) return fail(BCA_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (flags & ~(uint32_t)BCA_PLAN_HOST_ONLY) return fail(BCA_ERR_ARG, "unknown plan flags");
  bca_plan_s* p = new (std::nothrow) bca_plan_s();
  if (p == nullptr) return fail(BCA_ERR_ALLOC, "host allocation of the plan failed");
  std::string err;
  int rc;
  try {
    rc = build(&p->host, &err);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(BCA_ERR_ALLOC, "host allocation of the plan failed");
  }
  if (rc != bca::kPlanOk) {
    delete p;
    return fail(rc == bca::kPlanErrBlockIds ? BCA_ERR_BLOCK_IDS : BCA_ERR_ARG, err);
  }
  p->host_only = (flags & BCA_PLAN_HOST_ONLY) ? 1 : 0;
  if (!p->host_only) {
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "hipGetDevice");
    }
    bca_status s;
    try {
      s = upload(p);
    } catch (const std::bad_alloc&) {
      s = fail(BCA_ERR_ALLOC, "host allocation of the plan's staging buffer failed");
    }
    if (s != BCA_OK) {
      free_device(p);
      delete p;
      return s;
    }
  }
  *out = p;
  return BCA_OK;
}

}  // namespace

extern "C" {

bca_status bca_plan(const int32_t* block_ids, int64_t seq_len, uint32_t flags, bca_plan_t* out) {
  return make_plan(flags, out, [&](bca::HostPlan* h, std::string* err) {
    return bca::build_host_plan(block_ids, seq_len, bca::kBlockM, h, err);
  });
}

bca_status bca_plan_varlen(const int32_t* block_ids, const int64_t* lengths,
                           const int64_t* row_start, int32_t batch, uint32_t flags,
                           bca_plan_t* out) {
  return make_plan(flags, out, [&](bca::HostPlan* h, std::string* err) {
    return bca::build_varlen_plan(block_ids, lengths, row_start, batch, bca::kBlockM, h, err);
  });
}

bca_status bca_plan_free(bca_plan_t plan) {
  if (plan == nullptr) return BCA_OK;
  free_device(plan);
  delete plan;
  return BCA_OK;
}

bca_status bca_plan_get_info(bca_plan_t plan, bca_plan_info* out) {
  if (plan == nullptr || out == nullptr) return fail(BCA_ERR_ARG, "plan or out is NULL");
  const bca::HostPlan& h = plan->host;
  out->seq_len = h.seq_len;
  out->prefix_len = h.prefix_len;
  out->target_len = h.target_len;
  out->useful_pairs = h.useful_pairs;
  out->n_segments = (int32_t)(h.segments.size() / 3);
  out->block_m = bca::kBlockM;
  out->block_n = bca::kPrefillBlockN;
  out->n_qtiles = (int32_t)h.kv_end.size();
  out->decode_ok = h.decode_ok;
  out->host_only = plan->host_only;
  out->n_sequences = h.n_sequences;
  out->reserved = 0;
  out->rows = h.rows;
  return BCA_OK;
}

bca_status bca_plan_export(bca_plan_t plan, int32_t* segments, int32_t* row_limit,
                           int32_t* kv_full, int32_t* kv_end, int32_t* order) {
  if (plan == nullptr) return fail(BCA_ERR_ARG, "plan is NULL");
  const bca::HostPlan& h = plan->host;
  auto put = [](int32_t* dst, const std::vector<int32_t>& v) {
    if (dst) std::memcpy(dst, v.data(), v.size() * sizeof(int32_t));
  };
  put(segments, h.segments);
  put(row_limit, h.row_limit);
  put(kv_full, h.kv_full);
  put(kv_end, h.kv_end);
  put(order, h.order);
  return BCA_OK;
}

bca_status bca_prefill_ex(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                          const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                          const bca_tensor* o, const bca_kv_cache* cache, void* stream) {
  float scale_log2 = 0.0f;
  bca_status s = check_common(plan, B, H, D, scale, &scale_log2);
  if (s != BCA_OK) return s;
  if ((s = check_tensor(q, "q", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k, "k", 2)) != BCA_OK) return s;
  if ((s = check_tensor(v, "v", 2)) != BCA_OK) return s;
  if ((s = check_tensor(o, "o", 4)) != BCA_OK) return s;
  const bca::HostPlan& hp = plan->host;
  if (hp.n_sequences != 1)
    return fail(BCA_ERR_ARG, "plan holds several sequences: launch it with bca_prefill_varlen");
  const bool store = cache != nullptr && hp.prefix_len > 0;  // P = 0: nothing to store
  if (cache != nullptr && (s = check_format(cache)) != BCA_OK) return s;
  if (store && (s = check_cache(cache, hp.prefix_len)) != BCA_OK) return s;
  if ((s = check_extent(k, "k", hp.seq_len)) != BCA_OK) return s;
  if ((s = check_extent(v, "v", hp.seq_len)) != BCA_OK) return s;
  const int64_t nt = (int64_t)hp.kv_end.size();
  if (!grid_fits(nt, B, H)) return fail(BCA_ERR_ARG, "B * H * query tiles is too large a grid");
  if (store && cache->format != BCA_CACHE_BF16 &&
      !grid_fits(((int64_t)B * hp.prefix_len * H + 15) / 16, 256))
    return fail(BCA_ERR_ARG, "B * P * H is too large for the cache quantisation grid");
  if ((s = check_launchable(plan)) != BCA_OK) return s;

  bca::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_sb = q->stride_b; a.q_ss = q->stride_s; a.q_sh = q->stride_h;
  a.k = k->data;
  a.k_sb = k->stride_b; a.k_ss = k->stride_s; a.k_sh = k->stride_h;
  a.v = v->data;
  a.v_sb = v->stride_b; a.v_ss = v->stride_s; a.v_sh = v->stride_h;
  a.k2 = static_cast<const uint16_t*>(k->data);
  a.k2_sb = a.k_sb; a.k2_ss = a.k_ss; a.k2_sh = a.k_sh;
  a.v2 = static_cast<const uint16_t*>(v->data);
  a.v2_sb = a.v_sb; a.v2_ss = a.v_ss; a.v2_sh = a.v_sh;
  a.o = static_cast<float*>(o->data);
  a.o_sb = o->stride_b; a.o_ss = o->stride_s; a.o_sh = o->stride_h;
  a.n_q = (int32_t)hp.seq_len;
  a.kv_len = (int32_t)hp.seq_len;
  a.split = (int32_t)hp.seq_len;
  a.heads = H;
  a.batch = B;
  a.n_qtiles = (int32_t)nt;
  a.scale_log2 = scale_log2;
  a.row_limit = plan->d_row_limit;
  a.kv_full = plan->d_kv_full;
  a.kv_end = plan->d_kv_end;
  a.order = plan->d_order;
  a.tiles = plan->d_tiles;
  a.cache_fmt = BCA_CACHE_BF16;
  // The attention kernel stores the cache's bf16 tensors from its on-chip tiles; a quantised
  // tensor is written afterwards, on the same stream, from the same k / v rows.
  const bool kq = store && cache->format == BCA_CACHE_FP8_KV;
  const bool vq = store && cache->format != BCA_CACHE_BF16;
  if (store) {
    if (!kq) {
      a.kc = cache->k.data;
      a.kc_sb = cache->k.stride_b; a.kc_ss = cache->k.stride_s; a.kc_sh = cache->k.stride_h;
    }
    if (!vq) {
      a.vc = cache->v.data;
      a.vc_sb = cache->v.stride_b; a.vc_ss = cache->v.stride_s; a.vc_sh = cache->v.stride_h;
    }
  }
  const bool hand_off = prefill_hands_off(hp, B, H, bca::device_cus());
  if (hand_off) {  // the prefix rows in tiles of their own (they store the cache)
    a.n_q = a.kv_len = a.split = (int32_t)hp.prefix_len;
    a.n_qtiles = (int32_t)hp.prefix_order.size();
    a.order = plan->d_prefix_order;
    a.tiles = plan->d_prefix_tiles;
  }
  hipError_t e = bca::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  if (hand_off) {
    // then the target rows as a cached step whose prefix keys are rows [0, P) of k and v
    const int64_t P = hp.prefix_len;
    bca::AttnArgs d{};
    d.q = static_cast<const uint16_t*>(q->data) + P * q->stride_s;
    d.q_sb = q->stride_b; d.q_ss = q->stride_s; d.q_sh = q->stride_h;
    d.k = k->data;
    d.k_sb = k->stride_b; d.k_ss = k->stride_s; d.k_sh = k->stride_h;
    d.v = v->data;
    d.v_sb = v->stride_b; d.v_ss = v->stride_s; d.v_sh = v->stride_h;
    d.k2 = static_cast<const uint16_t*>(k->data) + P * k->stride_s;
    d.k2_sb = k->stride_b; d.k2_ss = k->stride_s; d.k2_sh = k->stride_h;
    d.v2 = static_cast<const uint16_t*>(v->data) + P * v->stride_s;
    d.v2_sb = v->stride_b; d.v2_ss = v->stride_s; d.v2_sh = v->stride_h;
    d.o = static_cast<float*>(o->data) + P * o->stride_s;
    d.o_sb = o->stride_b; d.o_ss = o->stride_s; d.o_sh = o->stride_h;
    d.n_q = (int32_t)hp.target_len;
    d.kv_len = (int32_t)hp.seq_len;
    d.split = (int32_t)P;
    d.heads = H;
    d.batch = B;
    d.scale_log2 = scale_log2;
    d.cache_fmt = BCA_CACHE_BF16;
    d.n_split = 1;
    e = bca::launch_decode(d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "prefill launch (target rows)");
  }
  if (kq || vq) {
    bca::QuantArgs qa{};
    qa.k = static_cast<const uint16_t*>(k->data);
    qa.k_sb = k->stride_b; qa.k_ss = k->stride_s; qa.k_sh = k->stride_h;
    qa.v = static_cast<const uint16_t*>(v->data);
    qa.v_sb = v->stride_b; qa.v_ss = v->stride_s; qa.v_sh = v->stride_h;
    if (kq) {
      qa.ko = static_cast<uint8_t*>(cache->k.data);
      qa.ko_sb = cache->k.stride_b; qa.ko_ss = cache->k.stride_s; qa.ko_sh = cache->k.stride_h;
      qa.ks = static_cast<float*>(cache->k_scale.data);
      qa.ks_sb = cache->k_scale.stride_b; qa.ks_ss = cache->k_scale.stride_s;
      qa.ks_sh = cache->k_scale.stride_h;
    }
    qa.vo = static_cast<uint8_t*>(cache->v.data);
    qa.vo_sb = cache->v.stride_b; qa.vo_ss = cache->v.stride_s; qa.vo_sh = cache->v.stride_h;
    qa.vs = static_cast<float*>(cache->v_scale.data);
    qa.vs_sb = cache->v_scale.stride_b; qa.vs_ss = cache->v_scale.stride_s;
    qa.vs_sh = cache->v_scale.stride_h;
    qa.rows = (int64_t)B * hp.prefix_len * H;
    qa.prefix = (int32_t)hp.prefix_len;
    qa.heads = H;
    e = bca::launch_quantize(qa, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cache quantisation launch");
  }
  return BCA_OK;
}

bca_status bca_prefill(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                       const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                       const bca_tensor* o, const bca_tensor* k_cache, const bca_tensor* v_cache,
                       void* stream) {
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(BCA_ERR_ARG, "k_cache and v_cache must both be given or both be NULL");
  if (k_cache == nullptr) return bca_prefill_ex(plan, B, H, D, scale, q, k, v, o, nullptr, stream);
  const bca_kv_cache c = bf16_cache(k_cache, v_cache);
  return bca_prefill_ex(plan, B, H, D, scale, q, k, v, o, &c, stream);
}

bca_status bca_prefill_layout(bca_plan_t plan, int32_t B, int32_t H, int32_t cus, int32_t* out) {
  if (plan == nullptr || out == nullptr) return fail(BCA_ERR_ARG, "plan or out is NULL");
  if (B < 1 || H < 1) return fail(BCA_ERR_ARG, "B and H must be >= 1");
  if (cus < 0) return fail(BCA_ERR_ARG, "cus must be >= 0 (0 = the current device's)");
  const bca::HostPlan& hp = plan->host;
  const bool hand_off = prefill_hands_off(hp, B, H, cus > 0 ? cus : bca::device_cus());
  out[0] = hand_off ? 2 : 1;
  out[1] = (int32_t)(hand_off ? hp.prefix_order.size() : hp.kv_end.size());
  out[2] = hand_off ? (int32_t)hp.target_len : 0;
  return BCA_OK;
}

bca_status bca_prefill_varlen(bca_plan_t plan, int32_t H, int32_t D, float scale,
                              const bca_tensor* q, const bca_tensor* k, const bca_tensor* v,
                              const bca_tensor* o, const bca_tensor* k_cache,
                              const bca_tensor* v_cache, void* stream) {
  float scale_log2 = 0.0f;
  bca_status s = check_common(plan, 1, H, D, scale, &scale_log2);
  if (s != BCA_OK) return s;
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(BCA_ERR_ARG, "k_cache and v_cache must both be given or both be NULL");
  if ((s = check_tensor(q, "q", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k, "k", 2)) != BCA_OK) return s;
  if ((s = check_tensor(v, "v", 2)) != BCA_OK) return s;
  if ((s = check_tensor(o, "o", 4)) != BCA_OK) return s;
  const bca::HostPlan& hp = plan->host;
  if ((s = check_extent(k, "k", hp.rows)) != BCA_OK) return s;
  if ((s = check_extent(v, "v", hp.rows)) != BCA_OK) return s;
  const bool store = k_cache != nullptr && hp.prefix_len > 0;  // no prefix rows: nothing to store
  if (store) {
    if ((s = check_tensor(k_cache, "k_cache", 2)) != BCA_OK) return s;
    if ((s = check_tensor(v_cache, "v_cache", 2)) != BCA_OK) return s;
    if ((s = check_extent(k_cache, "k_cache", hp.prefix_len)) != BCA_OK) return s;
    if ((s = check_extent(v_cache, "v_cache", hp.prefix_len)) != BCA_OK) return s;
  }
  const int64_t nt = (int64_t)hp.kv_end.size();
  if (!grid_fits(nt, 1, H)) return fail(BCA_ERR_ARG, "H * query tiles is too large a grid");
  if ((s = check_launchable(plan)) != BCA_OK) return s;

  bca::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_ss = q->stride_s; a.q_sh = q->stride_h;
  a.k = k->data;
  a.k_ss = k->stride_s; a.k_sh = k->stride_h;
  a.v = v->data;
  a.v_ss = v->stride_s; a.v_sh = v->stride_h;
  a.k2 = static_cast<const uint16_t*>(k->data);
  a.k2_ss = a.k_ss; a.k2_sh = a.k_sh;
  a.v2 = static_cast<const uint16_t*>(v->data);
  a.v2_ss = a.v_ss; a.v2_sh = a.v_sh;
  a.o = static_cast<float*>(o->data);
  a.o_ss = o->stride_s; a.o_sh = o->stride_h;
  a.n_q = (int32_t)hp.rows;
  a.kv_len = (int32_t)hp.rows;
  a.split = (int32_t)hp.rows;
  a.heads = H;
  a.batch = 1;
  a.n_qtiles = (int32_t)nt;
  a.scale_log2 = scale_log2;
  a.row_limit = plan->d_row_limit;
  a.kv_full = plan->d_kv_full;
  a.kv_end = plan->d_kv_end;
  a.order = plan->d_order;
  a.tiles = plan->d_tiles;
  a.cache_fmt = BCA_CACHE_BF16;
  if (store) {
    a.kc = k_cache->data;
    a.kc_ss = k_cache->stride_s; a.kc_sh = k_cache->stride_h;
    a.vc = v_cache->data;
    a.vc_ss = v_cache->stride_s; a.vc_sh = v_cache->stride_h;
  }
  hipError_t e = bca::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return BCA_OK;
}

bca_status bca_plan_sequences(bca_plan_t plan, int64_t* out) {
  if (plan == nullptr || out == nullptr) return fail(BCA_ERR_ARG, "plan or out is NULL");
  const std::vector<int32_t>& sq = plan->host.seqs;
  const size_t n = sq.size() / bca::kSeqInts;
  for (size_t b = 0; b < n; ++b)
    for (int c = 0; c < 6; ++c) out[6 * b + c] = sq[b * bca::kSeqInts + c];
  return BCA_OK;
}

}  // extern "C"

namespace {

// Key ranges of a split decode: the requested count, or (0) the library's choice; at most one
// range per unit, and no empty range.  The choice leaves a grid of at least 768 four-wave
// workgroups (three per CU on 256 CUs) as it is.  A smaller grid is split into n ranges of at
// least 8 units, n minimising ceil(base n / 768) / n + n / 100: whole rounds of 768 workgroups,
// each range a 1/n of the keys, plus a small charge per range for the partial results and the
// merge.  (The 512^2-target step, 256 workgroups unsplit, gets 3 ranges: one round.)
void split_shape(const bca::HostPlan& hp, int32_t B, int32_t H, int32_t n_split,
                 int32_t* n_used, int32_t* tiles_per) {
  // in units of kSplitUnit keys, the same for every cache format
  const int64_t ktiles = (hp.prefix_len + hp.target_len + bca::kSplitUnit - 1) / bca::kSplitUnit;
  // query tiles counted in 128-row units, also independent of the format
  const int64_t nt = (hp.target_len + 127) / 128;
  int64_t want = n_split;
  if (want == 0) {
    constexpr int64_t kSlots = 768;
    const int64_t base = nt * B * H;
    const int64_t most = std::max<int64_t>(1, ktiles / 8);
    want = 1;
    if (base < kSlots) {
      double best = 2.0;  // above any split's cost
      for (int64_t n = 1; n <= most && n <= 4 * kSlots; ++n) {
        const double cost = (double)((base * n + kSlots - 1) / kSlots) / (double)n + n / 100.0;
        if (cost < best) best = cost, want = n;
      }
    }
  }
  want = std::max<int64_t>(1, std::min<int64_t>(want, ktiles));
  const int64_t per = (ktiles + want - 1) / want;
  *tiles_per = (int32_t)per;
  *n_used = (int32_t)((ktiles + per - 1) / per);
}

int64_t split_bytes(const bca::HostPlan& hp, int32_t B, int32_t H, int32_t n_used) {
  return n_used <= 1 ? 0 : (int64_t)n_used * B * hp.target_len * H * (bca::kHeadDim + 2) * 4;
}

bca_status decode_impl(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                       const bca_tensor* q_tgt, const bca_kv_cache* cache,
                       const bca_tensor* k_tgt, const bca_tensor* v_tgt, const bca_tensor* o,
                       bool split_call, int32_t n_split, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  float scale_log2 = 0.0f;
  bca_status s = check_common(plan, B, H, D, scale, &scale_log2);
  if (s != BCA_OK) return s;
  const bca::HostPlan& hp = plan->host;
  if (hp.n_sequences != 1)
    return fail(BCA_ERR_ARG, "plan holds several sequences: launch it with bca_decode_varlen");
  if (!hp.decode_ok)
    return fail(BCA_ERR_NO_DECODE, "the layout's last block is text; cached decode needs the "
                                   "target image block last");
  if ((s = check_tensor(q_tgt, "q_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k_tgt, "k_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(v_tgt, "v_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(o, "o", 4)) != BCA_OK) return s;
  const bool use_cache = hp.prefix_len > 0;
  if (use_cache) {
    if (cache == nullptr)
      return fail(BCA_ERR_ARG, "the prefix is not empty: the cache (K and V) is required");
    if ((s = check_cache(cache, hp.prefix_len)) != BCA_OK) return s;
  }
  const int64_t N = hp.target_len;
  if ((s = check_extent(k_tgt, "k_tgt", N)) != BCA_OK) return s;
  if ((s = check_extent(v_tgt, "v_tgt", N)) != BCA_OK) return s;
  // the largest grid any decode kernel takes (launch_decode picks the kernel and its tiles)
  const int64_t nt = (N + bca::kDecodeMinBlockM - 1) / bca::kDecodeMinBlockM;
  int32_t n_used = 1, per = 0;
  if (split_call) {
    if (n_split < 0) return fail(BCA_ERR_ARG, "n_split must be >= 0 (0 = chosen by the library)");
    split_shape(hp, B, H, n_split, &n_used, &per);
    const int64_t need = split_bytes(hp, B, H, n_used);
    if (n_used > 1) {
      if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return fail(BCA_ERR_ARG, "workspace must be a 16-byte aligned device pointer");
      if (workspace_bytes < need)
        return fail(BCA_ERR_ARG, "workspace holds " + std::to_string(workspace_bytes) +
                                     " bytes, " + std::to_string(need) + " needed");
    }
  }
  if (!grid_fits(nt * n_used, B, H)) return fail(BCA_ERR_ARG, "the decode grid is too large");
  if ((s = check_launchable(plan)) != BCA_OK) return s;

  bca::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q_tgt->data);
  a.q_sb = q_tgt->stride_b; a.q_ss = q_tgt->stride_s; a.q_sh = q_tgt->stride_h;
  a.k2 = static_cast<const uint16_t*>(k_tgt->data);
  a.k2_sb = k_tgt->stride_b; a.k2_ss = k_tgt->stride_s; a.k2_sh = k_tgt->stride_h;
  a.v2 = static_cast<const uint16_t*>(v_tgt->data);
  a.v2_sb = v_tgt->stride_b; a.v2_ss = v_tgt->stride_s; a.v2_sh = v_tgt->stride_h;
  a.cache_fmt = BCA_CACHE_BF16;
  if (use_cache) {
    a.k = cache->k.data;
    a.k_sb = cache->k.stride_b; a.k_ss = cache->k.stride_s; a.k_sh = cache->k.stride_h;
    a.v = cache->v.data;
    a.v_sb = cache->v.stride_b; a.v_ss = cache->v.stride_s; a.v_sh = cache->v.stride_h;
    set_cache_args(cache, &a);
  } else {  // no prefix: every key comes from the target
    a.k = a.k2; a.k_sb = a.k2_sb; a.k_ss = a.k2_ss; a.k_sh = a.k2_sh;
    a.v = a.v2; a.v_sb = a.v2_sb; a.v_ss = a.v2_ss; a.v_sh = a.v2_sh;
  }
  a.o = static_cast<float*>(o->data);
  a.o_sb = o->stride_b; a.o_ss = o->stride_s; a.o_sh = o->stride_h;
  a.n_q = (int32_t)N;
  a.kv_len = (int32_t)(hp.prefix_len + N);
  a.split = (int32_t)hp.prefix_len;
  a.heads = H;
  a.batch = B;
  a.scale_log2 = scale_log2;
  a.n_split = n_used;
  if (n_used > 1) {
    a.split_units = per;
    a.part_o = static_cast<float*>(workspace);
    a.part_ml = a.part_o + (int64_t)n_used * B * N * H * bca::kHeadDim;
  }
  hipError_t e = bca::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return BCA_OK;
}

}  // namespace

extern "C" {

bca_status bca_decode_ex(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                         const bca_tensor* q_tgt, const bca_kv_cache* cache,
                         const bca_tensor* k_tgt, const bca_tensor* v_tgt, const bca_tensor* o,
                         void* stream) {
  return decode_impl(plan, B, H, D, scale, q_tgt, cache, k_tgt, v_tgt, o, false, 1, nullptr, 0,
                     stream);
}

bca_status bca_decode_layout(int64_t n_q, int64_t batch_heads, int32_t n_split, int32_t cache_fmt,
                             int32_t cus, int32_t* out) {
  if (out == nullptr) return fail(BCA_ERR_ARG, "out is NULL");
  if (n_q < 1 || n_q > INT32_MAX) return fail(BCA_ERR_ARG, "n_q must be in [1, 2^31 - 1]");
  if (batch_heads < 1 || batch_heads > INT32_MAX)
    return fail(BCA_ERR_ARG, "batch_heads must be in [1, 2^31 - 1]");
  if (n_split < 1 || batch_heads * n_split > INT32_MAX)
    return fail(BCA_ERR_ARG, "n_split must be >= 1, with batch_heads * n_split below 2^31");
  if (cus < 0) return fail(BCA_ERR_ARG, "cus must be >= 0 (0 = the current device's)");
  if (cache_fmt != BCA_CACHE_BF16 && cache_fmt != BCA_CACHE_FP8_V && cache_fmt != BCA_CACHE_FP8_KV)
    return fail(BCA_ERR_ARG, "cache_fmt must be BCA_CACHE_BF16, BCA_CACHE_FP8_V or BCA_CACHE_FP8_KV");
  const bca::DecodeLayout l = bca::decode_layout(n_q, batch_heads, n_split,
                                                 cus > 0 ? cus : bca::device_cus(), cache_fmt);
  out[0] = l.waves;
  out[1] = l.tiles[0];
  out[2] = l.tiles[1];
  out[3] = l.tiles[2];
  out[4] = l.tail;
  return BCA_OK;
}

bca_status bca_decode_split_workspace(bca_plan_t plan, int32_t B, int32_t H, int32_t n_split,
                                      int64_t* bytes, int32_t* n_split_used) {
  if (plan == nullptr || bytes == nullptr) return fail(BCA_ERR_ARG, "plan or bytes is NULL");
  if (B < 1 || H < 1) return fail(BCA_ERR_ARG, "B and H must be >= 1");
  if (n_split < 0) return fail(BCA_ERR_ARG, "n_split must be >= 0 (0 = chosen by the library)");
  if (!plan->host.decode_ok)
    return fail(BCA_ERR_NO_DECODE, "the layout's last block is text");
  int32_t n_used = 1, per = 0;
  split_shape(plan->host, B, H, n_split, &n_used, &per);
  *bytes = split_bytes(plan->host, B, H, n_used);
  if (n_split_used) *n_split_used = n_used;
  return BCA_OK;
}

bca_status bca_decode_split(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                            const bca_tensor* q_tgt, const bca_kv_cache* cache,
                            const bca_tensor* k_tgt, const bca_tensor* v_tgt, const bca_tensor* o,
                            int32_t n_split, void* workspace, int64_t workspace_bytes,
                            void* stream) {
  return decode_impl(plan, B, H, D, scale, q_tgt, cache, k_tgt, v_tgt, o, true, n_split,
                     workspace, workspace_bytes, stream);
}

bca_status bca_decode_split_noalloc(bca_plan_t plan, int32_t B, int32_t H, int32_t D,
                                    float scale, const bca_tensor* q_tgt,
                                    const bca_kv_cache* cache, const bca_tensor* k_tgt,
                                    const bca_tensor* v_tgt, const bca_tensor* o, int32_t n_split,
                                    void* stream) {
  if (plan == nullptr) return fail(BCA_ERR_ARG, "plan is NULL");
  if (B < 1 || H < 1) return fail(BCA_ERR_ARG, "B and H must be >= 1");
  if (n_split < 0) return fail(BCA_ERR_ARG, "n_split must be >= 0 (0 = chosen by the library)");
  if (!plan->host.decode_ok)
    return fail(BCA_ERR_NO_DECODE, "the layout's last block is text; cached decode needs the "
                                   "target image block last");
  int32_t n_used = 1, per = 0;
  split_shape(plan->host, B, H, n_split, &n_used, &per);
  const int64_t need = split_bytes(plan->host, B, H, n_used);
  if (need > bca::kScratchBytes)
    return fail(BCA_ERR_ARG, "the split needs " + std::to_string(need) +
                                 " bytes of partial results; the library's scratch holds " +
                                 std::to_string(bca::kScratchBytes) +
                                 " (use bca_decode_split with a caller workspace)");
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = bca::scratch_memory(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
  }
  return decode_impl(plan, B, H, D, scale, q_tgt, cache, k_tgt, v_tgt, o, true, n_split, ws,
                     need > 0 ? bca::kScratchBytes : 0, stream);
}

bca_status bca_decode(bca_plan_t plan, int32_t B, int32_t H, int32_t D, float scale,
                      const bca_tensor* q_tgt, const bca_tensor* k_cache,
                      const bca_tensor* v_cache, const bca_tensor* k_tgt,
                      const bca_tensor* v_tgt, const bca_tensor* o, void* stream) {
  if (k_cache == nullptr || v_cache == nullptr)
    return bca_decode_ex(plan, B, H, D, scale, q_tgt, nullptr, k_tgt, v_tgt, o, stream);
  const bca_kv_cache c = bf16_cache(k_cache, v_cache);
  return bca_decode_ex(plan, B, H, D, scale, q_tgt, &c, k_tgt, v_tgt, o, stream);
}

bca_status bca_decode_varlen(bca_plan_t plan, int32_t H, int32_t D, float scale,
                             const bca_tensor* q_tgt, const bca_tensor* k_cache,
                             const bca_tensor* v_cache, const bca_tensor* k_tgt,
                             const bca_tensor* v_tgt, const bca_tensor* o, void* stream) {
  float scale_log2 = 0.0f;
  bca_status s = check_common(plan, 1, H, D, scale, &scale_log2);
  if (s != BCA_OK) return s;
  const bca::HostPlan& hp = plan->host;
  if (!hp.decode_ok)
    return fail(BCA_ERR_NO_DECODE, "a sequence's last block is text; cached decode needs every "
                                   "sequence to end in its target image block");
  if ((s = check_tensor(q_tgt, "q_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k_tgt, "k_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(v_tgt, "v_tgt", 2)) != BCA_OK) return s;
  if ((s = check_tensor(o, "o", 4)) != BCA_OK) return s;
  const bool use_cache = hp.prefix_len > 0;
  if (use_cache) {
    if (k_cache == nullptr || v_cache == nullptr)
      return fail(BCA_ERR_ARG, "the prefixes are not empty: k_cache and v_cache are required");
    if ((s = check_tensor(k_cache, "k_cache", 2)) != BCA_OK) return s;
    if ((s = check_tensor(v_cache, "v_cache", 2)) != BCA_OK) return s;
    if ((s = check_extent(k_cache, "k_cache", hp.prefix_len)) != BCA_OK) return s;
    if ((s = check_extent(v_cache, "v_cache", hp.prefix_len)) != BCA_OK) return s;
  }
  if ((s = check_extent(k_tgt, "k_tgt", hp.target_len)) != BCA_OK) return s;
  if ((s = check_extent(v_tgt, "v_tgt", hp.target_len)) != BCA_OK) return s;
  int32_t n_max = 0;
  for (size_t b = 0; b < hp.seqs.size() / bca::kSeqInts; ++b)
    n_max = std::max(n_max, hp.seqs[b * bca::kSeqInts + 3]);
  const int64_t nt = (n_max + bca::kDecodeMinBlockM - 1) / bca::kDecodeMinBlockM;
  if (!grid_fits(nt, hp.n_sequences, H)) return fail(BCA_ERR_ARG, "the decode grid is too large");
  if ((s = check_launchable(plan)) != BCA_OK) return s;

  bca::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q_tgt->data);
  a.q_ss = q_tgt->stride_s; a.q_sh = q_tgt->stride_h;
  a.k2 = static_cast<const uint16_t*>(k_tgt->data);
  a.k2_ss = k_tgt->stride_s; a.k2_sh = k_tgt->stride_h;
  a.v2 = static_cast<const uint16_t*>(v_tgt->data);
  a.v2_ss = v_tgt->stride_s; a.v2_sh = v_tgt->stride_h;
  a.cache_fmt = BCA_CACHE_BF16;
  if (use_cache) {
    a.k = k_cache->data;
    a.k_ss = k_cache->stride_s; a.k_sh = k_cache->stride_h;
    a.v = v_cache->data;
    a.v_ss = v_cache->stride_s; a.v_sh = v_cache->stride_h;
  } else {  // every key comes from the targets
    a.k = a.k2; a.k_ss = a.k2_ss; a.k_sh = a.k2_sh;
    a.v = a.v2; a.v_ss = a.v2_ss; a.v_sh = a.v2_sh;
  }
  a.o = static_cast<float*>(o->data);
  a.o_ss = o->stride_s; a.o_sh = o->stride_h;
  a.n_q = n_max;
  a.heads = H;
  a.batch = hp.n_sequences;
  a.scale_log2 = scale_log2;
  a.n_split = 1;
  a.seqs = plan->d_seqs;
  hipError_t e = bca::launch_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return BCA_OK;
}

bca_status bca_qk_prologue(int32_t B, int64_t S, int32_t H, int32_t D, float eps,
                           const bca_tensor* q, const bca_tensor* k, const bca_tensor* q_out,
                           const bca_tensor* k_out, const float* q_weight, const float* k_weight,
                           const float* rope_table, void* stream) {
  if (B < 1 || H < 1 || S < 1) return fail(BCA_ERR_ARG, "B, S and H must be >= 1");
  if (S > INT32_MAX) return fail(BCA_ERR_ARG, "S must be below 2^31");
  if (D != bca::kHeadDim)
    return fail(BCA_ERR_UNSUPPORTED, "head width " + std::to_string(D) + " (only 128 is built)");
  if (!(eps >= 0.0f) || std::isinf(eps)) return fail(BCA_ERR_ARG, "eps must be finite and >= 0");
  bca_status s;
  if ((s = check_tensor(q, "q", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k, "k", 2)) != BCA_OK) return s;
  if ((s = check_tensor(q_out, "q_out", 2)) != BCA_OK) return s;
  if ((s = check_tensor(k_out, "k_out", 2)) != BCA_OK) return s;
  const void* vecs[3] = {q_weight, k_weight, rope_table};
  const char* names[3] = {"q_weight", "k_weight", "rope_table"};
  for (int i = 0; i < 3; ++i) {
    if (vecs[i] == nullptr) return fail(BCA_ERR_ARG, std::string(names[i]) + " is NULL");
    if (reinterpret_cast<uintptr_t>(vecs[i]) % 16 != 0)
      return fail(BCA_ERR_ARG, std::string(names[i]) + " is not 16-byte aligned");
  }
  const int64_t rows = (int64_t)B * S * H;
  if ((rows + 15) / 16 > (int64_t)UINT32_MAX) return fail(BCA_ERR_ARG, "B * S * H is too large");
  bca::PrologueArgs a{};
  a.q = static_cast<const uint16_t*>(q->data);
  a.q_sb = q->stride_b; a.q_ss = q->stride_s; a.q_sh = q->stride_h;
  a.k = static_cast<const uint16_t*>(k->data);
  a.k_sb = k->stride_b; a.k_ss = k->stride_s; a.k_sh = k->stride_h;
  a.qo = static_cast<uint16_t*>(q_out->data);
  a.qo_sb = q_out->stride_b; a.qo_ss = q_out->stride_s; a.qo_sh = q_out->stride_h;
  a.ko = static_cast<uint16_t*>(k_out->data);
  a.ko_sb = k_out->stride_b; a.ko_ss = k_out->stride_s; a.ko_sh = k_out->stride_h;
  a.wq = q_weight;
  a.wk = k_weight;
  a.table = rope_table;
  a.rows = rows;
  a.seq = (int32_t)S;
  a.heads = H;
  a.eps = eps;
  hipError_t e = bca::launch_prologue(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  return BCA_OK;
}

bca_status bca_cache_dequantize(int32_t B, int64_t P, int32_t H, int32_t D,
                                const bca_kv_cache* cache, const bca_tensor* k_out,
                                const bca_tensor* v_out, void* stream) {
  if (B < 1 || H < 1 || P < 1) return fail(BCA_ERR_ARG, "B, P and H must be >= 1");
  if (P > INT32_MAX) return fail(BCA_ERR_ARG, "P must be below 2^31");
  if (D != bca::kHeadDim)
    return fail(BCA_ERR_UNSUPPORTED, "head width " + std::to_string(D) + " (only 128 is built)");
  if (cache == nullptr) return fail(BCA_ERR_ARG, "cache is NULL");
  bca_status s;
  if ((s = check_cache(cache, P)) != BCA_OK) return s;
  if ((s = check_tensor(k_out, "k_out", 2)) != BCA_OK) return s;
  if ((s = check_tensor(v_out, "v_out", 2)) != BCA_OK) return s;
  const int64_t rows = (int64_t)B * P * H;
  if (!grid_fits((rows + 15) / 16, 256)) return fail(BCA_ERR_ARG, "B * P * H is too large");
  bca::DequantArgs a{};
  a.k = cache->k.data;
  a.k_sb = cache->k.stride_b; a.k_ss = cache->k.stride_s; a.k_sh = cache->k.stride_h;
  a.v = cache->v.data;
  a.v_sb = cache->v.stride_b; a.v_ss = cache->v.stride_s; a.v_sh = cache->v.stride_h;
  if (cache->format == BCA_CACHE_FP8_KV) {
    a.ks = static_cast<const float*>(cache->k_scale.data);
    a.ks_sb = cache->k_scale.stride_b; a.ks_ss = cache->k_scale.stride_s;
    a.ks_sh = cache->k_scale.stride_h;
  }
  if (cache->format != BCA_CACHE_BF16) {
    a.vs = static_cast<const float*>(cache->v_scale.data);
    a.vs_sb = cache->v_scale.stride_b; a.vs_ss = cache->v_scale.stride_s;
    a.vs_sh = cache->v_scale.stride_h;
  }
  a.ko = static_cast<uint16_t*>(k_out->data);
  a.ko_sb = k_out->stride_b; a.ko_ss = k_out->stride_s; a.ko_sh = k_out->stride_h;
  a.vo = static_cast<uint16_t*>(v_out->data);
  a.vo_sb = v_out->stride_b; a.vo_ss = v_out->stride_s; a.vo_sh = v_out->stride_h;
  a.rows = rows;
  a.prefix = (int32_t)P;
  a.heads = H;
  a.fmt = cache->format;
  hipError_t e = bca::launch_dequant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dequantize launch");
  return BCA_OK;
}

}  // extern "C"
