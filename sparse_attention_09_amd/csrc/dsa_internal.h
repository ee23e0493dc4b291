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

// Top-k staging geometry (host copy of what the kernels assume).
constexpr int32_t kTopkSeg = 65536;      // positions one workgroup selects from
constexpr int32_t kTopkMaxK = 16384;
int32_t topk_num_segments(int32_t max_ctx);

}  // namespace dsa
