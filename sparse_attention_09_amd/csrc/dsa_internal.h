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

// Validation of the batch description common to the indexer and Partial.
dsa_status check_batch(const dsa_pool* pool, const int32_t* page_table, int32_t pt_stride,
                       const int32_t* q_offsets, int32_t num_reqs, const int32_t* tok_pos,
                       int32_t num_tokens, const char* who);

// Indexer geometry shared by the indexer and the fused top-k host code.
constexpr int32_t kIndexChunkPages = 8;     // pages per indexer workgroup (512 positions)
constexpr int32_t kIndexChunk = kIndexChunkPages * 64;
constexpr int32_t kIndexSampleStride = 32;  // sample pass: logical pages 0, 32, 64, ...
constexpr int32_t kIndexMaxCap = 128;       // emit pass: most candidate slots per token and chunk

// Candidate output of the indexer's emit pass: for token t and chunk j (512
// positions), the scores >= thr[t], in position order, at slots
// [(t*nch + j)*cap, +cap), and their number (possibly > cap) in
// count[t*nch + j].
// Emit-pass output.  Each (token, chunk) has a region of capr pairs (cap + 1
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

}  // namespace dsa
