// Indexer scores on gfx950.
//
// For every query token t and visible position p of its request:
//   s[t,p] = sum_{h<16} w[t,h] * max(0, q_idx[t,h,:] . key(p))
// (the DSA indexer of "Accelerating GLM-5.3-Flash on H200", section 1; the
// score formula is the reading documented with the oracle).
//
// Decode-shaped batches have a few query tokens per request and a long
// context, so the key stream dominates: each workgroup owns one request, up to
// 8 of its query tokens (8 x 16 heads = 128 MFMA rows) and a chunk of 8 pages
// (512 positions).  Keys are streamed page by page (16 KB) through a
// double-buffered LDS stage with a register prefetch of the next page, and
// every key read from HBM serves all the block's tokens and heads.  Dot
// products run on the bf16 MFMA with fp32 accumulation; relu, the head
// weights and the 16-head sum happen in registers and cross-lane shuffles.
#include <hip/hip_runtime.h>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kQB = 8;             // query tokens per workgroup
#ifndef DSA_INDEX_CHUNK_PAGES
#define DSA_INDEX_CHUNK_PAGES 8
#endif
constexpr int kChunkPages = DSA_INDEX_CHUNK_PAGES;   // pages per workgroup
constexpr int kKeyStride = 136;    // LDS stride of one key row in bf16 (128 + 8 pad)
constexpr int kPageKeysBf16 = DSA_PAGE_TOKENS * DSA_IDX_DIM;

using dsa::bf16x8;
using dsa::f32x4;
using dsa::u32x4;

__global__ __launch_bounds__(kThreads) void index_scores_kernel(
    const uint16_t* __restrict__ keys, int num_pages, const int32_t* __restrict__ page_table,
    int pt_stride, const int32_t* __restrict__ q_offsets, const int32_t* __restrict__ tok_pos,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, float* __restrict__ scores,
    int64_t ld, int max_ctx, int num_tokens) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][DSA_PAGE_TOKENS * kKeyStride];

  const int b = blockIdx.y;
  const int t_begin = q_offsets[b] + blockIdx.z * kQB;
  const int t_end = min(min(q_offsets[b + 1], t_begin + kQB), num_tokens);
  const int nq = t_end - t_begin;
  if (nq <= 0) return;
  int block_max = -1;
  for (int t = t_begin; t < t_end; ++t) block_max = max(block_max, min(tok_pos[t], max_ctx - 1));
  const int p_begin = blockIdx.x * kChunkPages * DSA_PAGE_TOKENS;
  if (p_begin > block_max) return;
  const int page_begin = blockIdx.x * kChunkPages;
  const int page_end = min(min(page_begin + kChunkPages, block_max / DSA_PAGE_TOKENS + 1), pt_stride);
  if (page_end <= page_begin) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;   // lane group: MFMA k-slice / output row group
  const int c = lane & 15;   // MFMA row (A) / column (B, D)

  // Wave -> (token pair, subset of the page's four 16-position blocks).
  const int npair = (nq + 1) >> 1;
  const int pairs_p2 = npair <= 1 ? 1 : (npair <= 2 ? 2 : 4);
  const int nsub = 4 / pairs_p2;
  const int pair = wave % pairs_p2;
  const int sub = wave / pairs_p2;
  const bool wave_active = pair < npair;
  const int tA = t_begin + 2 * pair;
  const int tB = tA + 1;
  const bool hasA = wave_active;
  const bool hasB = wave_active && tB < t_end;

  // Indexer queries of the pair in MFMA A layout (head c, dims 32ks + 8g + i)
  // and the head weights of the heads this lane's outputs hold (4g + j).
  u32x4 qa[4], qb[4];
  float wa[4], wb[4];
  int posA = -1, posB = -1;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qa[ks] = u32x4{0, 0, 0, 0};
    qb[ks] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) wa[j] = wb[j] = 0.f;
  if (hasA) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q_idx + (int64_t(tA) * DSA_IDX_HEADS + c) * DSA_IDX_DIM);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = src[ks * 4 + g];
#pragma unroll
    for (int j = 0; j < 4; ++j) wa[j] = w[int64_t(tA) * DSA_IDX_HEADS + 4 * g + j];
    posA = min(tok_pos[tA], max_ctx - 1);
  }
  if (hasB) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q_idx + (int64_t(tB) * DSA_IDX_HEADS + c) * DSA_IDX_DIM);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = src[ks * 4 + g];
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[j] = w[int64_t(tB) * DSA_IDX_HEADS + 4 * g + j];
    posB = min(tok_pos[tB], max_ctx - 1);
  }

  // Page staging: 1024 16-byte pieces per page, 4 per thread, coalesced.
  auto page_src = [&](int pg) -> const u32x4* {
    int id = page_table[int64_t(b) * pt_stride + pg];
    id = min(max(id, 0), num_pages - 1);
    return reinterpret_cast<const u32x4*>(keys + int64_t(id) * kPageKeysBf16);
  };
  // two register stages: page pg+1 is in flight in one while page pg+2 is
  // requested into the other (the stages alternate, so the loop is unrolled by 2)
  u32x4 pa[4], pb[4];
  auto load_page = [&](u32x4 (&pre)[4], int pg) {
    const u32x4* src = page_src(pg);
#pragma unroll
    for (int i = 0; i < 4; ++i) pre[i] = src[tid + kThreads * i];
  };
  auto store_page = [&](const u32x4 (&pre)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + kThreads * i;
      const int row = piece >> 4, col = (piece & 15) * 8;
      *reinterpret_cast<u32x4*>(&lds[buf][row * kKeyStride + col]) = pre[i];
    }
  };

  load_page(pa, page_begin);
  if (page_begin + 1 < page_end) load_page(pb, page_begin + 1);
  store_page(pa, 0);
  __syncthreads();
  int cur = 0;
  for (int pg = page_begin; pg < page_end; ++pg) {
    // pb holds page pg+1 (if any) when an even step starts, pa when an odd one does
    const bool odd = ((pg - page_begin) & 1) != 0;
    const bool more = pg + 1 < page_end;
    if (pg + 2 < page_end) {
      if (odd) load_page(pb, pg + 2); else load_page(pa, pg + 2);
    }
    if (wave_active) {
      const int pos0 = pg * DSA_PAGE_TOKENS;
      for (int nb = sub; nb < 4; nb += nsub) {
        const uint16_t* krow = &lds[cur][(nb * 16 + c) * kKeyStride + 8 * g];
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = dsa::as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 32 * ks));
          accA = dsa::mfma16x16x32(dsa::as_bf16x8(qa[ks]), kf, accA);
          if (hasB) accB = dsa::mfma16x16x32(dsa::as_bf16x8(qb[ks]), kf, accB);
        }
        float sA = 0.f, sB = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sA = fmaf(wa[j], fmaxf(accA[j], 0.f), sA);
          sB = fmaf(wb[j], fmaxf(accB[j], 0.f), sB);
        }
        sA = dsa::rows4_sum(sA);   // integer-valued: exact in any order
        sB = dsa::rows4_sum(sB);
        const int p = pos0 + nb * 16 + c;
        if (g == 0 && p <= posA) scores[int64_t(tA) * ld + p] = sA;
        if (g == 1 && hasB && p <= posB) scores[int64_t(tB) * ld + p] = sB;
      }
    }
    if (more) {
      if (odd) store_page(pa, cur ^ 1); else store_page(pb, cur ^ 1);
    }
    __syncthreads();
    cur ^= 1;
  }
}

}  // namespace

extern "C" dsa_status dsa_index_scores(const dsa_pool* pool, const int32_t* page_table,
                                       int32_t pt_stride, const int32_t* q_offsets,
                                       int32_t num_reqs, int32_t max_q, const int32_t* tok_pos,
                                       int32_t num_tokens, int32_t max_ctx, const uint16_t* q_idx,
                                       const float* w, float* scores, int64_t ld, void* stream) {
  dsa_status s = dsa::check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos,
                                  num_tokens, "dsa_index_scores");
  if (s != DSA_OK) return s;
  if (num_tokens == 0 || max_ctx == 0) return dsa::ok();
  if (max_q < 1 || max_ctx < 0)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_index_scores: need max_q >= 1 and max_ctx >= 0");
  if (!q_idx || !w || !scores)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_index_scores: q_idx, w and scores must be non-null");
  if (!dsa::aligned(q_idx, 16) || !dsa::aligned(w, 4) || !dsa::aligned(scores, 16))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_index_scores: q_idx/scores must be 16-byte aligned");
  if (ld < max_ctx || ld % 4 != 0)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_index_scores: need ld >= max_ctx and ld % 4 == 0");
  const int64_t chunks = (int64_t(max_ctx) + kChunkPages * DSA_PAGE_TOKENS - 1) /
                         (kChunkPages * DSA_PAGE_TOKENS);
  const int64_t qblocks = (int64_t(max_q) + kQB - 1) / kQB;
  if (chunks > 0x7fffffff || num_reqs > 65535 || qblocks > 65535)
    return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_index_scores: batch exceeds the launch grid limits");
  const uint16_t* keys =
      reinterpret_cast<const uint16_t*>(pool->base + pool->layout.index_plane_offset);
  const dim3 grid{unsigned(chunks), unsigned(num_reqs), unsigned(qblocks)};
  hipLaunchKernelGGL(index_scores_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     keys, pool->num_pages, page_table, pt_stride, q_offsets, tok_pos, q_idx, w,
                     scores, ld, max_ctx, num_tokens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_index_scores: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
