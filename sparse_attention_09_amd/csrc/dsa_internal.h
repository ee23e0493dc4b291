// Host-side internals shared by the C-ABI entry points (no HIP dependency, so
// the pool, plan and validation logic also builds with a plain C++ compiler).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "dsa.h"

struct dsa_pool {
  char* base = nullptr;         // caller-owned device buffer
  int64_t bytes = 0;
  int32_t num_pages = 0;
  int32_t kv_dtype = 0;
  dsa_pool_layout layout{};
  std::vector<int32_t> refcount;   // per page; 0 = free
  std::vector<int32_t> free_list;  // stack of free page ids
};

namespace dsa {

// Records `msg` as this thread's last error and returns `s`.
dsa_status fail(dsa_status s, const std::string& msg);
// Clears the thread's last error and returns DSA_OK.
dsa_status ok();

bool fill_layout(int32_t kv_dtype, int32_t num_pages, dsa_pool_layout* out);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }


// Indexer geometry shared by the indexer and the fused top-k host code.
constexpr int32_t kIndexChunkPages = 8;     // pages per indexer workgroup (512 positions)
constexpr int32_t kIndexChunk = kIndexChunkPages * 64;
constexpr int32_t kIndexSampleStride = 32;  // sample pass: logical pages 0, 32, 64, ...
constexpr int32_t kIndexMaxCap = 128;       // emit pass: most candidate slots per token and chunk

// Emit-pass output of the indexer (scores >= thr[t] of token t and chunk j of
// 512 positions).  Each (token, chunk) has a region of capr pairs (cap + 1
// rounded up to whole 16-pair, 128-byte lines): pair 0 holds the chunk's
// candidate count, then its candidates as (score bits, position) pairs in
// position order, padded to whole lines so that no line is written in part.
struct IndexEmit {
  const float* thr;
  int32_t* cand;      // pairs: [token][nch][capr][2]
  int32_t nch, cap, capr;
};
constexpr int32_t kCandAlign = 16;   // pairs per 128-byte line
constexpr int32_t cand_region_pairs(int32_t cap) { return (cap + kCandAlign) / kCandAlign * kCandAlign; }

// Launches the indexer: mode 0 writes scores[t*ld + p]; mode 1 (sample pass)
// writes scores[t*ld + 64*s + x] for position 64*32*s + x; mode 2 emits
// candidates into *em (scores unused).  Arguments are those of
// dsa_index_scores, already validated.
dsa_status launch_index(int mode, const dsa_pool* pool, const int32_t* page_table,
                        int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                        int32_t max_q, const int32_t* tok_pos, int32_t num_tokens,
                        int32_t max_ctx, const uint16_t* q_idx, const float* w, float* scores,
                        int64_t ld, const IndexEmit* em, void* stream);

// Top-k staging geometry (host copy of what the kernels assume).
constexpr int32_t kTopkSeg = 65536;      // positions one workgroup selects from
constexpr int32_t kTopkMaxK = 16384;
int32_t topk_num_segments(int32_t max_ctx);

// DCP merge limits: shards, and shards x k candidates one workgroup holds.
constexpr int32_t kDcpMaxShards = 16;
constexpr int32_t kDcpMergeMax = 16384;

// Workspace of the fused indexer + top-k (byte offsets, each 256-aligned; the
// fallback counter sits at offset 0), and the sample / chunk geometry.
struct FusedLayout {
  size_t nflag, list, samples, thr, cand, total;
  int32_t ls, nch, capr;
};
FusedLayout fused_layout(int64_t num_tokens, int32_t max_ctx, int32_t cap);

// ---------------------------------------------------------------------------
// Argument checks of the compute entry points (dsa_validate.cpp, host-only).
// Each returns DSA_OK, or records a message (fail) and returns the status.
dsa_status check_batch(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                       const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                       int32_t num_tokens, const char* who);
dsa_status check_index_scores(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                              const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                              const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                              const uint16_t* q_idx, const float* w, const float* scores,
                              int64_t ld);
dsa_status check_topk(const char* who, const float* scores, int64_t ld, const int32_t* tok_pos,
                      int32_t num_tokens, int32_t max_ctx, int32_t k, const int32_t* idx);
// need == 0: no workspace required
dsa_status check_workspace(const char* who, const void* workspace, size_t bytes, size_t need);
dsa_status check_index_topk(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* q_offsets, int32_t num_reqs, int32_t max_q,
                            const int32_t* tok_pos, int32_t num_tokens, int32_t max_ctx,
                            const uint16_t* q_idx, const float* w, int32_t k, int32_t cap,
                            int32_t cand_target, const int32_t* idx, const void* workspace,
                            size_t workspace_bytes);
// final_form: out_a = bf16 out, out_b = lse; else out_a = o_part, out_b = lse_part
dsa_status check_partial(const char* who, const dsa_pool* pool, const int32_t* page_table,
                         int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                         const int32_t* tok_pos, int32_t num_tokens, const uint16_t* q,
                         const int32_t* idx, int32_t width, float sm_scale, int32_t kv_tile,
                         int32_t num_splits, bool final_form, const void* out_a,
                         const void* out_b);
dsa_status check_quantize_q8(const uint16_t* q, int32_t num_tokens, const uint8_t* q_codes,
                             const float* q_scales);
dsa_status check_sparse_mla_q8(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                               const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                               int32_t num_tokens, const uint8_t* q_codes, const float* q_scales,
                               const int32_t* idx, int32_t width, float sm_scale,
                               const uint16_t* out, const float* lse);
dsa_status check_combine(const char* who, const float* o_part, const float* lse_part,
                         int32_t num_tokens, int32_t parts, const uint16_t* out, const float* lse);
dsa_status check_dcp_merge(int32_t num_shards, int32_t num_tokens, int32_t k,
                           const int32_t* local_idx, const float* local_scores, int64_t ld,
                           const int32_t* idx, const int32_t* shard_idx);
dsa_status check_kv_append(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                           int32_t num_reqs, const int32_t* req, const int32_t* pos, int32_t n,
                           const uint16_t* latent, const uint16_t* keys);

// DSA_VALIDATE=1 (any value but empty or "0"): the calls that read the page
// table first copy the batch description to the host, after the work already
// queued on `stream`, and check q_offsets (0 .. num_tokens, nondecreasing),
// tok_pos (in [-1, pt_stride*64)) and every page id a token can reach (in
// [0, num_pages)).  A debugging aid: it synchronizes the stream.
bool validate_requested();
dsa_status deep_check_batch(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                            int32_t num_tokens, const char* who, void* stream);
// Copies `bytes` of caller memory (device or host) to host `dst` once the work
// queued on `stream` has completed.  Defined with the HIP runtime in the
// library; a host-only build supplies its own.
dsa_status copy_to_host(void* dst, const void* src, size_t bytes, void* stream);

}  // namespace dsa
