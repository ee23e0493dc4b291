// Host-only checks of the library's host logic: pool bookkeeping, the Partial
// dispatch plan, workspace sizes and every argument check, including the
// DSA_VALIDATE checks of the batch description.  Built with a plain C++
// compiler together with dsa_host.cpp and dsa_validate.cpp (no HIP), under
// the address and undefined-behaviour sanitizers, and run on the CPU.
//
//   host_logic_test list          names of the cases
//   host_logic_test CASE [ARGS]   runs one case; exit status 0 = pass
//
// "Device" arrays here are host arrays: this build's copy_to_host is memcpy.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {
dsa_status copy_to_host(void* dst, const void* src, size_t bytes, void*) {
  if (bytes) std::memcpy(dst, src, bytes);
  return DSA_OK;
}
}  // namespace dsa

namespace {

int g_failures = 0;

#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "%s:%d: CHECK failed: %s (last error: %s)\n", __FILE__, \
                   __LINE__, #cond, dsa_last_error());                          \
      ++g_failures;                                                             \
    }                                                                           \
  } while (0)

// A batch of 3 requests on a pool of 40 pages: request b has 3 - b query
// tokens at its last positions; every page id it can reach is valid.
struct Batch {
  std::vector<char> mem;       // stands in for the caller's pool buffer
  dsa_pool* pool = nullptr;
  int32_t pt_stride = 8;
  std::vector<int32_t> page_table, q_offsets, tok_pos;
  Batch() {
    dsa_pool_layout l;
    dsa_pool_layout_query(DSA_KV_FP8_E4M3_S64, 40, &l);
    mem.resize(size_t(l.total_bytes) + 256);
    void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(mem.data()) + 255) & ~uintptr_t(255));
    dsa_pool_create(base, l.total_bytes, 40, DSA_KV_FP8_E4M3_S64, &pool);
    const int32_t ctx[3] = {500, 130, 64};
    q_offsets.push_back(0);
    for (int b = 0; b < 3; ++b) {
      for (int i = 0; i < 3 - b; ++i) tok_pos.push_back(ctx[b] - (3 - b) + i);
      q_offsets.push_back(int32_t(tok_pos.size()));
    }
    page_table.assign(3 * pt_stride, -7);   // unreachable entries hold garbage
    for (int b = 0; b < 3; ++b)
      for (int j = 0; j * 64 < ctx[b]; ++j) page_table[b * pt_stride + j] = (b * 11 + j * 3) % 40;
  }
  ~Batch() { dsa_pool_destroy(pool); }
  dsa_status deep(const char* who = "test") {
    return dsa::deep_check_batch(pool, page_table.data(), pt_stride, q_offsets.data(), 3,
                                 tok_pos.data(), int32_t(tok_pos.size()), who, nullptr);
  }
};

struct Validate {   // DSA_VALIDATE=1 for the scope
  Validate() { setenv("DSA_VALIDATE", "1", 1); }
  ~Validate() { unsetenv("DSA_VALIDATE"); }
};

std::map<std::string, std::function<void(int, char**)>>& cases() {
  static std::map<std::string, std::function<void(int, char**)>> m;
  return m;
}
struct Reg {
  Reg(const char* n, std::function<void(int, char**)> f) { cases()[n] = std::move(f); }
};
#define CASE(name) \
  void case_##name(int, char**); \
  Reg reg_##name(#name, case_##name); \
  void case_##name(int argc, char** argv)

// ---------------------------------------------------------------------------
CASE(pool_bookkeeping) {
  (void)argc; (void)argv;
  std::vector<char> mem(1 << 20);
  void* base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(mem.data()) + 255) & ~uintptr_t(255));
  dsa_pool_layout l;
  CHECK(dsa_pool_layout_query(DSA_KV_FP8_E4M3_S64, 8, &l) == DSA_OK);
  CHECK(l.latent_row_stride == 640 && l.latent_row_bytes == 612 && l.index_row_bytes == 256);
  CHECK(l.total_bytes == 8 * 64 * (640 + 256));
  dsa_pool* p = nullptr;
  CHECK(dsa_pool_create(base, l.total_bytes - 1, 8, DSA_KV_FP8_E4M3_S64, &p) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_pool_create(static_cast<char*>(base) + 16, l.total_bytes, 8, 1, &p) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_pool_create(base, l.total_bytes, 8, 1, &p) == DSA_OK);
  int32_t ids[8];
  CHECK(dsa_pool_alloc(p, 5, ids) == DSA_OK && dsa_pool_free_pages(p) == 3);
  CHECK(dsa_pool_alloc(p, 4, ids + 5) == DSA_ERR_NO_SPACE && dsa_pool_free_pages(p) == 3);
  CHECK(dsa_pool_share(p, ids, 2) == DSA_OK && dsa_pool_refcount(p, ids[0]) == 2);
  CHECK(dsa_pool_release(p, ids, 5) == DSA_OK && dsa_pool_free_pages(p) == 6);
  const int32_t twice[2] = {ids[0], ids[0]};
  CHECK(dsa_pool_release(p, twice, 2) == DSA_ERR_INVALID_ARG && dsa_pool_refcount(p, ids[0]) == 1);
  CHECK(dsa_pool_release(p, ids + 4, 1) == DSA_ERR_INVALID_ARG);   // already free
  const int32_t bad = 99;
  CHECK(dsa_pool_share(p, &bad, 1) == DSA_ERR_INVALID_ARG && dsa_pool_refcount(p, 99) == -1);
  dsa_pool_destroy(p);
}

// argv: width, then (tile, iterations) pairs, then virtual and padding columns at the last tile
CASE(plan_worked_example) {
  CHECK(argc >= 7);
  if (argc < 7) return;
  const int width = std::atoi(argv[2]);
  for (int i = 3; i + 1 < argc - 2; i += 2) {
    dsa_partial_plan pl;
    CHECK(dsa_plan_partial(1024, width, std::atoi(argv[i]), 1, 0, &pl) == DSA_OK);
    CHECK(pl.iters_total == std::atoi(argv[i + 1]) && pl.splits == 1);
  }
  dsa_partial_plan pl;
  CHECK(dsa_plan_partial(1024, width, 128, 1, 0, &pl) == DSA_OK);
  CHECK(pl.virtual_cols == std::atoi(argv[argc - 2]) && pl.padding_cols == std::atoi(argv[argc - 1]));
  CHECK(dsa_plan_partial(4, 100, 48, 0, 0, &pl) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_plan_partial(4, 0, 0, 0, 0, &pl) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_plan_partial(8, 2048, 0, 0, 256, &pl) == DSA_OK && pl.tile == 64 && pl.splits == 16);
}

CASE(workspace_sizes) {
  (void)argc; (void)argv;
  CHECK(dsa_topk_workspace_bytes(1024, 65536, 2048) == 0);
  CHECK(dsa_topk_workspace_bytes(8, 1 << 20, 2048) == size_t(8) * 16 * 2048 * 8);
  const dsa::FusedLayout L = dsa::fused_layout(1024, 65536, 128);
  CHECK(L.nch == 128 && L.ls == 2048 && L.capr == 144);
  CHECK(L.total == 256 + 4096 + size_t(4) * 1024 * 2048 + 4096 + size_t(8) * 1024 * 128 * 144);
}

// ---------------------------------------------------------------------------
// argument checks that run on every call
CASE(check_partial_args) {
  (void)argc; (void)argv;
  Batch B;
  const int32_t* pt = B.page_table.data();
  const int32_t* qo = B.q_offsets.data();
  const int32_t* tp = B.tok_pos.data();
  alignas(16) static uint16_t q[64];
  alignas(16) static float o[64];
  static int32_t idx[8];
  auto call = [&](int width, float scale, int tile, int splits, const void* a, const void* b) {
    return dsa::check_partial("p", B.pool, pt, B.pt_stride, qo, 3, tp, 6, q, idx, width, scale, tile,
                              splits, false, a, b);
  };
  CHECK(call(64, 0.1f, 64, 1, o, o) == DSA_OK);
  CHECK(call(0, 0.1f, 64, 1, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, 0.1f, 48, 1, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, 0.1f, 64, 0, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, -0.1f, 64, 1, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, 1.0f / 0.0f, 64, 1, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, 0.1f, 64, 1, nullptr, o) == DSA_ERR_INVALID_ARG);
  CHECK(call(64, 0.1f, 64, 1, reinterpret_cast<const char*>(o) + 4, o) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_partial("p", nullptr, pt, B.pt_stride, qo, 3, tp, 6, q, idx, 64, 0.1f, 64, 1,
                           false, o, o) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_partial("p", B.pool, pt, 0, qo, 3, tp, 6, q, idx, 64, 0.1f, 64, 1, false, o, o) ==
        DSA_ERR_INVALID_ARG);
}

CASE(check_select_args) {
  (void)argc; (void)argv;
  Batch B;
  alignas(16) static float sc[64];
  alignas(16) static uint16_t qi[64];
  static int32_t idx[8];
  const int32_t* tp = B.tok_pos.data();
  CHECK(dsa::check_topk("t", sc, 64, tp, 6, 64, 8, idx) == DSA_OK);
  CHECK(dsa::check_topk("t", sc, 64, tp, 6, 64, 0, idx) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_topk("t", sc, 64, tp, 6, 64, 20000, idx) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa::check_topk("t", sc, 62, tp, 6, 64, 8, idx) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_topk("t", sc, 1 << 22, tp, 6, 1 << 22, 2048, idx) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa::check_workspace("t", nullptr, 0, 100) == DSA_ERR_WORKSPACE);
  CHECK(dsa::check_workspace("t", sc, 99, 100) == DSA_ERR_WORKSPACE);
  CHECK(dsa::check_workspace("t", nullptr, 0, 0) == DSA_OK);
  CHECK(dsa::check_index_scores(B.pool, B.page_table.data(), B.pt_stride, B.q_offsets.data(), 3, 3,
                                tp, 6, 500, qi, sc, sc, 500) == DSA_OK);
  CHECK(dsa::check_index_scores(B.pool, B.page_table.data(), B.pt_stride, B.q_offsets.data(), 3, 3,
                                tp, 6, 500, qi, sc, sc, 498) == DSA_ERR_INVALID_ARG);
  const size_t need = dsa::fused_layout(6, 500, 128).total;
  std::vector<char> ws(need + 256);
  void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(ws.data()) + 255) & ~uintptr_t(255));
  auto fused = [&](int k, int cap, int max_ctx, size_t bytes) {
    return dsa::check_index_topk(B.pool, B.page_table.data(), B.pt_stride, B.q_offsets.data(), 3, 3,
                                 tp, 6, max_ctx, qi, sc, k, cap, 0, idx, wsa, bytes);
  };
  CHECK(fused(64, 128, 500, need) == DSA_OK);
  CHECK(fused(64, 129, 500, need) == DSA_ERR_INVALID_ARG);
  CHECK(fused(64, 128, 65537, need) == DSA_ERR_UNSUPPORTED);
  CHECK(fused(64, 128, 500, need - 1) == DSA_ERR_WORKSPACE);
  CHECK(dsa::check_dcp_merge(17, 4, 8, idx, sc, 64, idx, nullptr) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_dcp_merge(8, 4, 4096, idx, sc, 64, idx, nullptr) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa::check_dcp_merge(8, 4, 16, idx, sc, 64, idx, nullptr) == DSA_OK);
}

CASE(check_combine_and_append_args) {
  (void)argc; (void)argv;
  Batch B;
  alignas(16) static float o[64];
  alignas(16) static uint16_t lat[64];
  static int32_t r[4];
  CHECK(dsa::check_combine("c", o, o, 1, 2, lat, o) == DSA_OK);
  CHECK(dsa::check_combine("c", o, o, 1, 0, lat, o) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_combine("c", nullptr, o, 1, 2, lat, o) == DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_combine("c", nullptr, nullptr, 0, 2, nullptr, nullptr) == DSA_OK);
  CHECK(dsa::check_kv_append(B.pool, B.page_table.data(), 8, 3, r, r, 1, lat, lat) == DSA_OK);
  CHECK(dsa::check_kv_append(B.pool, B.page_table.data(), 8, 3, r, r, 1, lat + 4, nullptr) ==
        DSA_ERR_INVALID_ARG);
  CHECK(dsa::check_kv_append(nullptr, B.page_table.data(), 8, 3, r, r, 1, lat, lat) ==
        DSA_ERR_INVALID_ARG);
}

// ---------------------------------------------------------------------------
// DSA_VALIDATE: one case per check of the batch description
CASE(validate_accepts_good_batch) {
  (void)argc; (void)argv;
  Batch B;
  {
    Validate v;
    CHECK(B.deep() == DSA_OK);
    B.tok_pos[5] = -1;   // a token that sees nothing
    CHECK(B.deep() == DSA_OK);
  }
  B.page_table[0] = -1;  // without DSA_VALIDATE the batch description is not read
  CHECK(B.deep() == DSA_OK);
}

CASE(validate_page_id_negative) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.page_table[0 * B.pt_stride + 3] = -1;
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
  CHECK(std::strstr(dsa_last_error(), "page_table[0][3] = -1") != nullptr);
}

CASE(validate_page_id_past_pool) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.page_table[1 * B.pt_stride + 2] = 40;          // request 1 reaches position 129: page 2
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
  CHECK(std::strstr(dsa_last_error(), "page_table[1][2] = 40") != nullptr);
}

CASE(validate_unreached_pages_ignored) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.page_table[2 * B.pt_stride + 1] = 12345;       // request 2 sees positions up to 63 only
  CHECK(B.deep() == DSA_OK);
}

CASE(validate_tok_pos_past_page_table) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.tok_pos[4] = B.pt_stride * 64;
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
  CHECK(std::strstr(dsa_last_error(), "tok_pos[4]") != nullptr);
}

CASE(validate_tok_pos_negative) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.tok_pos[0] = -2;
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
}

CASE(validate_q_offsets_start_end) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.q_offsets[3] = 5;                              // 6 tokens
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
  B.q_offsets[3] = 6;
  B.q_offsets[0] = 1;
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
}

CASE(validate_q_offsets_decreasing) {
  (void)argc; (void)argv;
  Batch B;
  Validate v;
  B.q_offsets[2] = 2;                              // 0, 3, 2, 6
  CHECK(B.deep() == DSA_ERR_INVALID_ARG);
  CHECK(std::strstr(dsa_last_error(), "decreases at request 1") != nullptr);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s list | CASE [ARGS]\n", argv[0]);
    return 2;
  }
  if (std::strcmp(argv[1], "list") == 0) {
    for (auto& kv : cases()) std::printf("%s\n", kv.first.c_str());
    return 0;
  }
  auto it = cases().find(argv[1]);
  if (it == cases().end()) {
    std::fprintf(stderr, "no case %s\n", argv[1]);
    return 2;
  }
  it->second(argc, argv);
  if (g_failures) std::fprintf(stderr, "%s: %d check(s) failed\n", argv[1], g_failures);
  return g_failures ? 1 : 0;
}
