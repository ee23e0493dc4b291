// Argument validation of the compute entry points, run on the host before any
// launch.  Host-only C++ (no HIP dependency): it builds with a plain C++
// compiler, so the checks can run under the address and undefined-behaviour
// sanitizers on a machine without a GPU.
//
// Two levels:
//   * always: pointers, alignment, sizes and limits of each call;
//   * with DSA_VALIDATE=1 in the environment: the batch description in caller
//     memory (q_offsets, tok_pos and every page-table entry a token can reach)
//     is copied to the host and checked, so that a corrupt page id is reported
//     instead of being clamped into the pool by the kernels.  The pool holds a
//     paged latent plane and a separate indexer-key plane addressed by the same
//     page id (SGLang cookbook "GLM-5.3-Flash", section 2 "Size both memory
//     pools"), so one range check covers both.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dsa_internal.h"

namespace dsa {

namespace {

std::string S(const char* who) { return std::string(who); }

}  // namespace

bool validate_requested() {
  const char* v = std::getenv("DSA_VALIDATE");
  return v && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

dsa_status check_batch(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                       const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                       int32_t num_tokens, const char* who) {
  if (!pool) return fail(DSA_ERR_INVALID_ARG, S(who) + ": pool is null");
  if (num_tokens < 0 || num_reqs < 0) return fail(DSA_ERR_INVALID_ARG, S(who) + ": negative size");
  if (num_tokens == 0) return DSA_OK;
  if (num_reqs < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": tokens without requests");
  if (!page_table || !q_offsets || !tok_pos)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": page_table, q_offsets and tok_pos must be non-null");
  if (pt_stride < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": pt_stride must be >= 1");
  if (!aligned(page_table, 4) || !aligned(q_offsets, 4) || !aligned(tok_pos, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": int32 arrays must be 4-byte aligned");
  return DSA_OK;
}

dsa_status deep_check_batch(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                            int32_t num_tokens, const char* who, void* stream) {
  if (num_tokens == 0 || !validate_requested()) return DSA_OK;
  std::vector<int32_t> qo(size_t(num_reqs) + 1);
  std::vector<int32_t> tp(static_cast<size_t>(num_tokens));
  std::vector<int32_t> pt(size_t(num_reqs) * size_t(pt_stride));
  dsa_status s = copy_to_host(qo.data(), q_offsets, qo.size() * 4, stream);
  if (s == DSA_OK) s = copy_to_host(tp.data(), tok_pos, tp.size() * 4, stream);
  if (s == DSA_OK) s = copy_to_host(pt.data(), page_table, pt.size() * 4, stream);
  if (s != DSA_OK) return s;
  const std::string w = S(who) + " (DSA_VALIDATE)";
  if (qo[0] != 0 || qo[size_t(num_reqs)] != num_tokens)
    return fail(DSA_ERR_INVALID_ARG, w + ": q_offsets must start at 0 and end at num_tokens (" +
                                         std::to_string(num_tokens) + "), got " +
                                         std::to_string(qo[0]) + " .. " +
                                         std::to_string(qo[size_t(num_reqs)]));
  for (int32_t b = 0; b < num_reqs; ++b)
    if (qo[size_t(b) + 1] < qo[size_t(b)])
      return fail(DSA_ERR_INVALID_ARG, w + ": q_offsets decreases at request " + std::to_string(b));
  const int64_t reach = int64_t(pt_stride) * DSA_PAGE_TOKENS;
  for (int32_t b = 0; b < num_reqs; ++b) {
    int32_t top = -1;   // highest position a token of request b can see
    for (int32_t t = qo[size_t(b)]; t < qo[size_t(b) + 1]; ++t) {
      const int32_t p = tp[size_t(t)];
      // -1 is a token that sees nothing (a shard holding none of its positions)
      if (p < -1 || int64_t(p) >= reach)
        return fail(DSA_ERR_INVALID_ARG, w + ": tok_pos[" + std::to_string(t) + "] = " +
                                             std::to_string(p) + " is outside [-1, pt_stride*64 = " +
                                             std::to_string(reach) + ")");
      top = p > top ? p : top;
    }
    for (int32_t j = 0; top >= 0 && j <= top / DSA_PAGE_TOKENS; ++j) {
      const int32_t id = pt[size_t(b) * size_t(pt_stride) + size_t(j)];
      if (id < 0 || id >= pool->num_pages)
        return fail(DSA_ERR_INVALID_ARG, w + ": page_table[" + std::to_string(b) + "][" +
                                             std::to_string(j) + "] = " + std::to_string(id) +
                                             " is not a page of the pool (" +
                                             std::to_string(pool->num_pages) + " pages)");
    }
  }
  return DSA_OK;
}

dsa_status check_index_scores(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                              const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                              const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                              const uint16_t* q_idx, const float* w, const float* scores,
                              int64_t ld) {
  const char* who = "dsa_index_scores";
  dsa_status s = check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens, who);
  if (s != DSA_OK) return s;
  if (num_tokens == 0 || max_ctx == 0) return DSA_OK;
  if (max_q < 1 || max_ctx < 0)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need max_q >= 1 and max_ctx >= 0");
  if (!q_idx || !w || !scores)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_idx, w and scores must be non-null");
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(scores, 16))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_idx/scores must be 16-byte aligned");
  if (ld < max_ctx || ld % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need ld >= max_ctx and ld % 4 == 0");
  return DSA_OK;
}

dsa_status check_topk(const char* who, const float* scores, int64_t ld, const int32_t* tok_pos,
                      int32_t num_tokens, int32_t max_ctx, int32_t k, const int32_t* idx) {
  if (num_tokens < 0 || max_ctx < 0) return fail(DSA_ERR_INVALID_ARG, S(who) + ": negative size");
  if (k < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": k must be >= 1");
  if (k > kTopkMaxK) return fail(DSA_ERR_UNSUPPORTED, S(who) + ": k above 16384");
  if (num_tokens == 0) return DSA_OK;
  if (!scores || !tok_pos || !idx)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": scores, tok_pos and idx must be non-null");
  if (!aligned(scores, 16) || !aligned(tok_pos, 4) || !aligned(idx, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": scores must be 16-byte aligned");
  if (ld < max_ctx || ld % 4 != 0)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need ld >= max_ctx and ld % 4 == 0");
  if (max_ctx > kTopkSeg) {
    if (num_tokens > 65535)
      return fail(DSA_ERR_UNSUPPORTED, S(who) + ": too many long rows for one launch");
    const int64_t kc = (int64_t(k) + 3) & ~int64_t(3);
    if (int64_t(topk_num_segments(max_ctx)) * kc > kTopkSeg)
      return fail(DSA_ERR_UNSUPPORTED, S(who) + ": segments x k exceeds one merge workgroup");
  }
  return DSA_OK;
}

dsa_status check_workspace(const char* who, const void* workspace, size_t bytes, size_t need) {
  if (need == 0) return DSA_OK;
  if (!workspace || bytes < need)
    return fail(DSA_ERR_WORKSPACE, S(who) + ": workspace of " + std::to_string(need) +
                                       " bytes required");
  if (!aligned(workspace, 256))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": workspace must be 256-byte aligned");
  return DSA_OK;
}

FusedLayout fused_layout(int64_t num_tokens, int32_t max_ctx, int32_t cap) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  FusedLayout L{};
  const int64_t pages = (int64_t(max_ctx) + DSA_PAGE_TOKENS - 1) / DSA_PAGE_TOKENS;
  const int64_t spages = (pages + kIndexSampleStride - 1) / kIndexSampleStride;
  L.ls = int32_t(spages * DSA_PAGE_TOKENS);
  L.nch = int32_t((int64_t(max_ctx) + kIndexChunk - 1) / kIndexChunk);
  const size_t T = size_t(num_tokens);
  size_t o = 0;
  L.nflag = o; o += up(4);
  L.list = o; o += up(4 * T);
  L.samples = o; o += up(4 * T * size_t(L.ls));
  L.thr = o; o += up(4 * T);
  L.capr = cand_region_pairs(cap);
  L.cand = o; o += up(8 * T * size_t(L.nch) * size_t(L.capr));
  L.total = o;
  return L;
}

dsa_status check_index_topk(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                            const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                            const uint16_t* q_idx, const float* w, int32_t k, int32_t cap,
                            int32_t cand_target, const int32_t* idx, const void* workspace,
                            size_t workspace_bytes) {
  const char* who = "dsa_index_topk";
  dsa_status s = check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens, who);
  if (s != DSA_OK) return s;
  if (k < 1 || k > kTopkMaxK) return fail(DSA_ERR_INVALID_ARG, S(who) + ": need 1 <= k <= 16384");
  if (cap < 1 || cap > kIndexMaxCap || cand_target < 0)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need 1 <= cap <= 128 and cand_target >= 0");
  if (max_q < 1 || max_ctx < 0)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need max_q >= 1 and max_ctx >= 0");
  if (max_ctx > kTopkSeg)
    return fail(DSA_ERR_UNSUPPORTED,
                S(who) + ": rows above 65,536 positions need dsa_index_scores + dsa_topk");
  if (num_tokens == 0) return DSA_OK;
  if (!q_idx || !w || !idx)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_idx, w and idx must be non-null");
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(idx, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_idx must be 16-byte aligned");
  return check_workspace(who, workspace, workspace_bytes,
                         fused_layout(num_tokens, max_ctx, cap).total);
}

dsa_status check_partial(const char* who, const dsa_pool* pool, const int32_t* page_table,
                         int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                         const int32_t* tok_pos, int32_t num_tokens, const uint16_t* q,
                         const int32_t* idx, int32_t width, float sm_scale, int32_t kv_tile,
                         int32_t num_splits, bool final_form, const void* out_a,
                         const void* out_b) {
  dsa_status s = check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens, who);
  if (s != DSA_OK) return s;
  if (width < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": width must be >= 1");
  if (kv_tile != 32 && kv_tile != 64 && kv_tile != 128)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": kv_tile must be 32, 64 or 128");
  if (num_splits < 1 || num_splits > 65535)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": num_splits must be in [1, 65535]");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": sm_scale must be finite and > 0");
  if (num_tokens == 0) return DSA_OK;
  if (!q || !idx || !out_a || !out_b)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q, idx and the outputs must be non-null");
  // final form: out (bf16) and lse 4-byte aligned; split form: o_part 16-byte, lse_part 4-byte
  if (!aligned(q, 16) || !aligned(idx, 4) || !aligned(out_a, final_form ? 4 : 16) ||
      !aligned(out_b, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q must be 16-byte aligned, o_part 16-byte, "
                                              "out/lse 4-byte");
  return DSA_OK;
}

dsa_status check_quantize_q8(const uint16_t* q, int32_t num_tokens, const uint8_t* q_codes,
                             const float* q_scales) {
  const char* who = "dsa_quantize_q8";
  if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, S(who) + ": num_tokens < 0");
  if (num_tokens == 0) return DSA_OK;
  if (!q || !q_codes || !q_scales)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q, q_codes and q_scales must be non-null");
  if (!aligned(q, 2) || !aligned(q_scales, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q must be 2-byte and q_scales 4-byte aligned");
  if ((int64_t(num_tokens) * DSA_HEADS + 3) / 4 > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, S(who) + ": too many tokens for one launch");
  return DSA_OK;
}

dsa_status check_sparse_mla_q8(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                               const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                               int32_t num_tokens, const uint8_t* q_codes, const float* q_scales,
                               const int32_t* idx, int32_t width, float sm_scale,
                               const uint16_t* out, const float* lse) {
  const char* who = "dsa_sparse_mla_q8";
  dsa_status s = check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens, who);
  if (s != DSA_OK) return s;
  if (pool->kv_dtype != DSA_KV_FP8_E4M3_S64)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": the Q8 path reads an FP8 pool");
  if (width < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": width must be >= 1");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": sm_scale must be finite and > 0");
  if (num_tokens == 0) return DSA_OK;
  if (!q_codes || !q_scales || !idx || !out || !lse)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_codes, q_scales, idx, out and lse must be non-null");
  if (!aligned(q_codes, 16) || !aligned(q_scales, 4) || !aligned(idx, 4) || !aligned(out, 4) ||
      !aligned(lse, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": q_codes must be 16-byte aligned; q_scales, idx, "
                                              "out and lse 4-byte");
  return DSA_OK;
}

dsa_status check_combine(const char* who, const float* o_part, const float* lse_part,
                         int32_t num_tokens, int32_t parts, const uint16_t* out, const float* lse) {
  if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARG, S(who) + ": num_tokens < 0");
  if (parts < 1) return fail(DSA_ERR_INVALID_ARG, S(who) + ": the part count must be >= 1");
  if (num_tokens == 0) return DSA_OK;
  if (!o_part || !lse_part || !out || !lse)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": pointers must be non-null");
  if (!aligned(o_part, 16) || !aligned(out, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": o_part and out must be 16-byte aligned");
  const int64_t rows = int64_t(num_tokens) * DSA_HEADS;
  if ((rows + 3) / 4 > 0x7fffffff)
    return fail(DSA_ERR_UNSUPPORTED, S(who) + ": too many tokens for one launch");
  return DSA_OK;
}

dsa_status check_dcp_merge(int32_t num_shards, int32_t num_tokens, int32_t k,
                           const int32_t* local_idx, const float* local_scores, int64_t ld,
                           const int32_t* idx, const int32_t* shard_idx) {
  const char* who = "dsa_dcp_merge";
  if (num_shards < 1 || num_shards > kDcpMaxShards)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need 1 <= num_shards <= 16");
  if (num_tokens < 0 || k < 1)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need num_tokens >= 0 and k >= 1");
  if (int64_t(num_shards) * k > kDcpMergeMax)
    return fail(DSA_ERR_UNSUPPORTED, S(who) + ": num_shards * k above 16384");
  if (num_tokens == 0) return DSA_OK;
  if (!local_idx || !local_scores || !idx)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": local_idx, local_scores and idx must be non-null");
  if (ld < 1 || !aligned(local_idx, 4) || !aligned(local_scores, 4) || !aligned(idx, 4) ||
      (shard_idx && !aligned(shard_idx, 4)))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need ld >= 1 and 4-byte aligned arrays");
  return DSA_OK;
}

dsa_status check_kv_append(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                           int32_t num_reqs, const int32_t* req, const int32_t* pos, int32_t n,
                           const uint16_t* latent, const uint16_t* keys) {
  const char* who = "dsa_kv_append";
  if (!pool) return fail(DSA_ERR_INVALID_ARG, S(who) + ": pool is null");
  if (n < 0 || num_reqs < 0 || pt_stride < 1)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": need n >= 0, num_reqs >= 0, pt_stride >= 1");
  if (n == 0) return DSA_OK;
  if (!page_table || !req || !pos || !latent)
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": page_table, req, pos and latent must be non-null");
  if (!aligned(latent, 16) || (keys && !aligned(keys, 16)) || !aligned(req, 4) ||
      !aligned(pos, 4) || !aligned(page_table, 4))
    return fail(DSA_ERR_INVALID_ARG, S(who) + ": latent and keys must be 16-byte aligned");
  return DSA_OK;
}

}  // namespace dsa
