// Host-only parts of the C ABI: error reporting, pool layout and page
// bookkeeping, the Partial dispatch plan and shared argument validation.
#include <algorithm>
#include <cstring>
#include <string>

#include "dsa_internal.h"

namespace {
thread_local std::string g_last_error;
constexpr int32_t kDefaultCUs = 256;  // MI355X compute units
}  // namespace

namespace dsa {

dsa_status fail(dsa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool fill_layout(int32_t kv_dtype, int32_t num_pages, dsa_pool_layout* out) {
  if (kv_dtype != DSA_KV_BF16 && kv_dtype != DSA_KV_FP8_E4M3_S64) return false;
  if (num_pages < 0) return false;
  dsa_pool_layout l{};
  l.page_tokens = DSA_PAGE_TOKENS;
  l.kv_dtype = kv_dtype;
  l.d_latent = DSA_D_LATENT;
  l.d_rope = DSA_D_ROPE;
  l.d_index = DSA_IDX_DIM;
  if (kv_dtype == DSA_KV_FP8_E4M3_S64) {
    l.latent_row_bytes = DSA_D_QK + 4 * (DSA_D_QK / 64);  // 612
    l.latent_row_stride = 640;
    l.scale_offset = DSA_D_QK;
  } else {
    l.latent_row_bytes = 2 * DSA_D_QK;  // 1152
    l.latent_row_stride = 2 * DSA_D_QK;
    l.scale_offset = -1;
  }
  l.index_row_bytes = 2 * DSA_IDX_DIM;
  l.latent_plane_offset = 0;
  l.index_plane_offset = int64_t(num_pages) * DSA_PAGE_TOKENS * l.latent_row_stride;
  l.total_bytes = l.index_plane_offset + int64_t(num_pages) * DSA_PAGE_TOKENS * l.index_row_bytes;
  *out = l;
  return true;
}

int32_t topk_num_segments(int32_t max_ctx) {
  return max_ctx <= kTopkSeg ? 1 : (max_ctx + kTopkSeg - 1) / kTopkSeg;
}

}  // namespace dsa

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_NO_SPACE: return "DSA_ERR_NO_SPACE";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    default: return "DSA_ERR_UNKNOWN";
  }
}

dsa_status dsa_pool_layout_query(int32_t kv_dtype, int32_t num_pages, dsa_pool_layout* out) {
  if (!out) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_layout_query: out is null");
  if (!dsa::fill_layout(kv_dtype, num_pages, out))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_layout_query: bad kv_dtype or num_pages");
  return dsa::ok();
}

dsa_status dsa_pool_create(void* dev_base, int64_t bytes, int32_t num_pages, int32_t kv_dtype,
                           dsa_pool** out) {
  if (!out) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_create: out is null");
  *out = nullptr;
  dsa_pool_layout l;
  if (!dsa::fill_layout(kv_dtype, num_pages, &l) || num_pages < 1)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_create: bad kv_dtype or num_pages");
  if (!dev_base) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_create: dev_base is null");
  if (!dsa::aligned(dev_base, 256))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_create: dev_base must be 256-byte aligned");
  if (bytes < l.total_bytes)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_create: buffer of " + std::to_string(bytes) +
                                              " bytes is smaller than the " +
                                              std::to_string(l.total_bytes) + " the pool needs");
  auto* p = new dsa_pool;
  p->base = static_cast<char*>(dev_base);
  p->bytes = bytes;
  p->num_pages = num_pages;
  p->kv_dtype = kv_dtype;
  p->layout = l;
  p->refcount.assign(num_pages, 0);
  p->free_list.resize(num_pages);
  // lowest ids are handed out first
  for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;
  *out = p;
  return dsa::ok();
}

void dsa_pool_destroy(dsa_pool* pool) { delete pool; }

dsa_status dsa_pool_alloc(dsa_pool* pool, int32_t n, int32_t* ids) {
  if (!pool) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_alloc: pool is null");
  if (n < 0 || (n > 0 && !ids)) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_alloc: bad n/ids");
  if (size_t(n) > pool->free_list.size())
    return dsa::fail(DSA_ERR_NO_SPACE, "dsa_pool_alloc: " + std::to_string(n) + " pages requested, " +
                                           std::to_string(pool->free_list.size()) + " free");
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = pool->free_list.back();
    pool->free_list.pop_back();
    pool->refcount[id] = 1;
    ids[i] = id;
  }
  return dsa::ok();
}

static dsa_status check_live(const dsa_pool* pool, const int32_t* ids, int32_t n, const char* who) {
  if (!pool) return dsa::fail(DSA_ERR_INVALID_ARG, std::string(who) + ": pool is null");
  if (n < 0 || (n > 0 && !ids)) return dsa::fail(DSA_ERR_INVALID_ARG, std::string(who) + ": bad n/ids");
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (id < 0 || id >= pool->num_pages)
      return dsa::fail(DSA_ERR_INVALID_ARG, std::string(who) + ": page id " + std::to_string(id) +
                                                " out of range");
    if (pool->refcount[id] <= 0)
      return dsa::fail(DSA_ERR_INVALID_ARG, std::string(who) + ": page " + std::to_string(id) +
                                                " is not allocated");
  }
  return DSA_OK;
}

dsa_status dsa_pool_share(dsa_pool* pool, const int32_t* ids, int32_t n) {
  dsa_status s = check_live(pool, ids, n, "dsa_pool_share");
  if (s != DSA_OK) return s;
  for (int32_t i = 0; i < n; ++i) pool->refcount[ids[i]]++;
  return dsa::ok();
}

dsa_status dsa_pool_release(dsa_pool* pool, const int32_t* ids, int32_t n) {
  dsa_status s = check_live(pool, ids, n, "dsa_pool_release");
  if (s != DSA_OK) return s;
  // a page listed more times than its refcount would underflow: reject before changing anything
  std::vector<int32_t> ids_sorted(ids, ids + n);
  std::sort(ids_sorted.begin(), ids_sorted.end());
  for (int32_t i = 0; i < n;) {
    int32_t j = i;
    while (j < n && ids_sorted[j] == ids_sorted[i]) ++j;
    if (j - i > pool->refcount[ids_sorted[i]])
      return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_pool_release: page " + std::to_string(ids_sorted[i]) +
                                                " released more times than it is referenced");
    i = j;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = ids[i];
    if (--pool->refcount[id] == 0) pool->free_list.push_back(id);
  }
  return dsa::ok();
}

int32_t dsa_pool_free_pages(const dsa_pool* pool) {
  return pool ? int32_t(pool->free_list.size()) : -1;
}

int32_t dsa_pool_refcount(const dsa_pool* pool, int32_t page_id) {
  if (!pool || page_id < 0 || page_id >= pool->num_pages) return -1;
  return pool->refcount[page_id];
}

int32_t dsa_pool_num_pages(const dsa_pool* pool) { return pool ? pool->num_pages : -1; }
int32_t dsa_pool_kv_dtype(const dsa_pool* pool) { return pool ? pool->kv_dtype : -1; }

dsa_status dsa_plan_partial(int32_t num_tokens, int32_t width, int32_t kv_tile, int32_t num_splits,
                            int32_t cu_count, dsa_partial_plan* out) {
  if (!out) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_plan_partial: out is null");
  if (num_tokens < 0 || width < 1)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_plan_partial: need num_tokens >= 0 and width >= 1");
  if (kv_tile != 0 && kv_tile != 32 && kv_tile != 64 && kv_tile != 128)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_plan_partial: kv_tile must be 0, 32, 64 or 128");
  if (num_splits < 0) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_plan_partial: num_splits < 0");
  if (cu_count < 0) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_plan_partial: cu_count < 0");
  // Query parallelism: one workgroup per (token, split), one resident workgroup
  // per CU.  With at least a CU's worth of tokens a single split keeps every CU
  // busy, and tile 32 runs the warp-specialized kernel (measured faster than
  // tile 64 on the 64K verify batch and the 32K prefill chunk).  With fewer
  // tokens, splits add workgroups up to one per CU, but each split keeps at
  // least two tiles: a split's fixed costs (its query rows, its partial output,
  // Combine's read of it) outweigh the parallelism of a one-tile split, so
  // these batches take tile 64 (half the splits) unless the index row is short
  // (under 1024 columns), where tile 32 still splits.
  const int32_t cus = cu_count > 0 ? cu_count : kDefaultCUs;
  int32_t tile = kv_tile;
  if (tile == 0) tile = (num_tokens >= cus || width < 1024) ? 32 : 64;
  const int32_t iters = (width + tile - 1) / tile;
  int32_t splits = num_splits;
  if (splits == 0) {
    if (num_tokens >= cus || num_tokens == 0) {
      splits = 1;
    } else {
      const int32_t want = (cus + num_tokens - 1) / num_tokens;   // one workgroup per CU
      splits = std::max(1, std::min(want, iters / 2));
    }
  }
  const int32_t ips = (iters + splits - 1) / splits;
  dsa_partial_plan p{};
  p.tile = tile;
  p.splits = splits;
  p.iters_total = iters;
  p.iters_per_split = ips;
  p.cols_per_split = ips * tile;
  p.virtual_cols = iters * tile;
  p.padding_cols = iters * tile - width;
  *out = p;
  return dsa::ok();
}

size_t dsa_topk_workspace_bytes(int32_t num_tokens, int32_t max_ctx, int32_t k) {
  if (num_tokens <= 0 || max_ctx <= dsa::kTopkSeg || k <= 0) return 0;
  const size_t nseg = size_t(dsa::topk_num_segments(max_ctx));
  const size_t kc = (size_t(k) + 3) & ~size_t(3);
  // candidate scores (fp32) and positions (int32) per token, segment and rank
  return size_t(num_tokens) * nseg * kc * 8;
}

}  // extern "C"
