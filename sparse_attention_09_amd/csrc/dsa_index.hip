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
// double-buffered LDS stage with a two-stage register prefetch, and every key
// read from HBM serves all the block's tokens and heads.  Dot products run on
// the bf16 MFMA with fp32 accumulation; relu, the head weights and the 16-head
// sum happen in registers and cross-lane swaps.
//
// Three modes share the kernel: scores (write every visible score), sample
// (score logical pages 0, 32, 64, ... only) and emit (keep, per token and
// chunk, the positions scoring at least a per-token threshold, in position
// order) - the last two feed the fused top-k.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kQB = 8;             // query tokens per workgroup
constexpr int kChunkPages = dsa::kIndexChunkPages;   // pages per workgroup
// LDS page: 64 key rows of 256 bytes, unpadded; 16-byte chunk j of row r sits
// at chunk j ^ (r & 15), so the 16 rows an MFMA operand read touches, and the
// 16 chunks a staging write touches, fall in 16 different bank groups
constexpr int kRowBf16 = DSA_IDX_DIM;
constexpr int kCandLds = dsa::kIndexMaxCap;   // emit pass: candidate slots per token (LDS)
constexpr int kPageKeysBf16 = DSA_PAGE_TOKENS * DSA_IDX_DIM;
constexpr int kSampleStride = dsa::kIndexSampleStride;
constexpr int kSampleChunkPages = 8;   // sample pass: sampled pages per workgroup

enum Mode { kScores = 0, kSample = 1, kEmit = 2 };

using dsa::bf16x8;
using dsa::f32x4;
using dsa::u32x4;

// One work unit: request `req`, query block `qblock` (up to 8 tokens), chunk
// `chunk` of pages.  Contains barriers; every thread of the workgroup runs it
// with the same unit.  lds: two staging buffers of one page; cand_v/cand_p:
// the emit pass's per-token candidate rows.  kStream: the keys are read
// with non-temporal loads, for batches that read each key once (caching
// them only evicts what is reused, such as the emit pass's candidate lists:
// verify batch selection -5%; where keys are read again, by the query blocks
// of a prefill chunk or by requests sharing a prefix, cached loads are
// 19-24% faster).
template <int MODE, bool kStream>
__device__ __forceinline__ void index_unit(
    const uint16_t* __restrict__ keys, int num_pages, const int32_t* __restrict__ page_table,
    int pt_stride, const int32_t* __restrict__ q_offsets, const int32_t* __restrict__ tok_pos,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, float* __restrict__ scores,
    int64_t ld, int max_ctx, int num_tokens, const dsa::IndexEmit& em,
    uint16_t (&lds)[2][DSA_PAGE_TOKENS * kRowBf16], float* cand_v, uint16_t* cand_p, float* sst,
    int chunk, int req, int qblock) {
  // the sample pass visits logical pages 0, 32, 64, ... (its "page" pg is the
  // sample page, logical page 32 pg); the other modes visit every page
  constexpr int kStride = MODE == kSample ? kSampleStride : 1;
  constexpr int kPages = MODE == kSample ? kSampleChunkPages : kChunkPages;

  const int b = req;
  const int t_begin = q_offsets[b] + qblock * kQB;
  const int t_end = min(min(q_offsets[b + 1], t_begin + kQB), num_tokens);
  const int nq = t_end - t_begin;
  if (nq <= 0) return;
  int block_max = -1;
  for (int t = t_begin; t < t_end; ++t) block_max = max(block_max, min(tok_pos[t], max_ctx - 1));
  const int p_begin = chunk * kPages * kStride * DSA_PAGE_TOKENS;
  if (p_begin > block_max) return;
  const int page_begin = chunk * kPages;
  const int last_lp = min(block_max / DSA_PAGE_TOKENS, pt_stride - 1);
  const int page_end = min(page_begin + kPages, last_lp / kStride + 1);
  const int tid = threadIdx.x;
  if (page_end <= page_begin) {
    // only when the page table is shorter than the context: no candidates
    if constexpr (MODE == kEmit)
      for (int i = tid; i < nq; i += kThreads)
        *reinterpret_cast<int2*>(em.cand + 2 * ((int64_t(t_begin + i) * em.nch + chunk) * em.capr)) =
            make_int2(0, 0);
    return;
  }

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;   // lane group: MFMA k-slice / output row group
  const int c = lane & 15;   // MFMA row (A) / column (B, D)

  // Wave -> (token pair, subset of the page's four 16-position blocks).  The
  // emit pass keeps each token's positions in one wave, so its candidates come
  // out in position order.
  const int npair = (nq + 1) >> 1;
  const int pairs_p2 = MODE == kEmit ? 4 : (npair <= 1 ? 1 : (npair <= 2 ? 2 : 4));
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
  float thrA = 0.f, thrB = 0.f;
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
    if constexpr (MODE == kEmit) thrA = em.thr[tA];
  }
  if (hasB) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q_idx + (int64_t(tB) * DSA_IDX_HEADS + c) * DSA_IDX_DIM);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = src[ks * 4 + g];
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[j] = w[int64_t(tB) * DSA_IDX_HEADS + 4 * g + j];
    posB = min(tok_pos[tB], max_ctx - 1);
    if constexpr (MODE == kEmit) thrB = em.thr[tB];
  }
  // Lanes of groups 0 and 2 own the scores of token A and token B (the
  // epilogue leaves A's in lanes 0..31 and B's in 32..63): their position
  // bound, threshold and LDS row (score staging or candidate slots).
  const bool owner = g == 0 || g == 2;
  const bool lane_b = g >= 2;
  const int my_pos = lane_b ? posB : posA;
  const float my_thr = lane_b ? thrB : thrA;
  // emit pass: candidates of this chunk so far (wave-uniform); this lane's
  // token's LDS row (its slot in the block)
  int cntA = 0, cntB = 0;
  const int my_li = 2 * pair + ((lane_b && hasB) ? 1 : 0);

  // Page staging: 1024 16-byte pieces per page, 4 per thread, coalesced.
  auto page_src = [&](int pg) -> const u32x4* {
    int id = page_table[int64_t(b) * pt_stride + pg * kStride];
    id = min(max(id, 0), num_pages - 1);
    return reinterpret_cast<const u32x4*>(keys + int64_t(id) * kPageKeysBf16);
  };
  // two register stages: page pg+1 is in flight in one while page pg+2 is
  // requested into the other
  u32x4 pa[4], pb[4];
  auto load_page = [&](u32x4 (&pre)[4], int pg) {
    const u32x4* src = page_src(pg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kStream) pre[i] = __builtin_nontemporal_load(src + tid + kThreads * i);
      else pre[i] = src[tid + kThreads * i];
    }
  };
  auto store_page = [&](const u32x4 (&pre)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + kThreads * i;
      const int row = piece >> 4, chunk = (piece & 15) ^ (row & 15);
      *reinterpret_cast<u32x4*>(&lds[buf][row * kRowBf16 + chunk * 8]) = pre[i];
    }
  };

  // The memory schedule keeps every step straight-line, so the compiler's
  // wait before staging a page counts exactly the four younger prefetch
  // loads: prefetches are unconditional (past the range they repeat the last
  // page), the idle LDS buffer is always written, and a step's scores are
  // held in LDS and stored at the start of the next step, before its
  // prefetch.
  load_page(pa, page_begin);
  load_page(pb, min(page_begin + 1, page_end - 1));
  store_page(pa, 0);
  __syncthreads();
  int cur = 0;
  // Scores of a computed page (not the emit pass, which writes its candidates
  // to LDS at once) go to the LDS staging sst[parity][token slot][64] and are
  // stored at the start of the next step, after its barrier, by threads
  // 0..127: each takes 4 consecutive positions of one token, so a token's
  // page leaves as whole 16-byte pieces (two full 128-byte lines) instead of
  // 4-byte stores.  held_pos0 / held_col0: the held page's first position and
  // output column (held_pos0 < 0: nothing held); par: the parity computed next.
  int held_pos0 = -1, held_col0 = 0, par = 0;
  const int fslot = tid >> 4, fgrp = tid & 15;   // flush: token slot, 4-position group
  int fpos = -1;
  float* frow = nullptr;
  if constexpr (MODE != kEmit) {
    if (tid < kQB * 16 && fslot < nq) {
      fpos = min(tok_pos[t_begin + fslot], max_ctx - 1);
      frow = scores + int64_t(t_begin + fslot) * ld;
    }
  }
  // scores (or candidates) of page pg, read from LDS buffer `cur`
  auto compute_page = [&](int pg) {
    const int pos0 = pg * kStride * DSA_PAGE_TOKENS;
    // output column of the page's first position: the position itself, or
    // in the sample pass the sample index (64 per sampled page)
    const int col0 = MODE == kSample ? pg * DSA_PAGE_TOKENS : pos0;
    // row nb*16 + c, dims 32ks + 8g.. (chunk 4ks + g, stored at (4ks + g) ^ c)
    const uint16_t* kbase = &lds[cur][c * kRowBf16];
    // one 16-position block: both tokens' dots (token B's are zero when the
    // wave has one token) and the 16-head epilogue
    auto block = [&](int k, int nb) {
      const uint16_t* krow = kbase + nb * 16 * kRowBf16;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = dsa::as_bf16x8(*reinterpret_cast<const u32x4*>(krow + 8 * ((4 * ks + g) ^ c)));
        accA = dsa::mfma16x16x32(dsa::as_bf16x8(qa[ks]), kf, accA);
        accB = dsa::mfma16x16x32(dsa::as_bf16x8(qb[ks]), kf, accB);
      }
      // lanes 0..31: token A's scores, lanes 32..63: token B's; lanes of
      // groups 0 and 2 own position c of the block
      const float sc = dsa::index_score2(accA, wa, accB, wb);
      if constexpr (MODE != kEmit) {
        if (owner && (!lane_b || hasB)) sst[(par * kQB + my_li) * DSA_PAGE_TOKENS + nb * 16 + c] = sc;
      }
      if constexpr (MODE == kEmit) {
        // slots follow the ballot order, i.e. position order
        const int p = pos0 + nb * 16 + c;
        const bool cand = owner && p <= my_pos && sc >= my_thr;
        const uint64_t m = __ballot(cand);
        const uint32_t mA = uint32_t(m) & 0xFFFFu, mB = uint32_t(m >> 32) & 0xFFFFu;
        // candidates below this lane in the ballot, minus token A's for B lanes
        const int below = int(__builtin_amdgcn_mbcnt_hi(mB, __builtin_amdgcn_mbcnt_lo(mA, 0u)));
        const int slot = (lane_b ? cntB - __popc(mA) : cntA) + below;
        // LDS writes need no deferral (they do not count against the loads)
        if (cand && slot < em.cap) {
          cand_v[my_li * kCandLds + slot] = sc;
          cand_p[my_li * kCandLds + slot] = uint16_t(p - p_begin);
        }
        cntA += __popc(mA);
        cntB += __popc(mB);
      }
    };
    if (nsub == 1) {
      block(0, 0);
      block(1, 1);
      block(2, 2);
      block(3, 3);
    } else if (nsub == 2) {
      block(0, sub);
      block(1, sub + 2);
    } else {
      block(0, sub);
    }
    (void)col0;
  };
  // the page a step computes (workgroup-uniform): what the next flush stores
  auto hold = [&](int pg) {
    held_pos0 = pg * kStride * DSA_PAGE_TOKENS;
    held_col0 = MODE == kSample ? pg * DSA_PAGE_TOKENS : held_pos0;
  };
  // stores the held page's visible scores (after the barrier that ends the
  // step which computed them)
  auto flush = [&]() {
    if constexpr (MODE != kEmit) {
      if (held_pos0 >= 0 && frow != nullptr) {
        const int p0 = held_pos0 + 4 * fgrp;
        const float4 v = *reinterpret_cast<const float4*>(
            sst + ((par ^ 1) * kQB + fslot) * DSA_PAGE_TOKENS + 4 * fgrp);
        float* dst = frow + held_col0 + 4 * fgrp;
        if (p0 + 3 <= fpos) {
          *reinterpret_cast<float4*>(dst) = v;
        } else {
          if (p0 <= fpos) dst[0] = v.x;
          if (p0 + 1 <= fpos) dst[1] = v.y;
          if (p0 + 2 <= fpos) dst[2] = v.z;
        }
      }
    }
    held_pos0 = -1;
  };
  // One page step: store the previous page's outputs, request page pg+2 into
  // `fill`, compute page pg, stage page pg+1 (held in `next`) into the other
  // LDS buffer.  Two steps per trip with the register stages swapped, so each
  // stage is a fixed register set (a runtime choice between them makes the
  // compiler wait for the loads right after issuing them).
  auto step = [&](int pg, u32x4 (&next)[4], u32x4 (&fill)[4]) {
    flush();
    load_page(fill, min(pg + 2, page_end - 1));
    if (wave_active) compute_page(pg);
    hold(pg);
    store_page(next, cur ^ 1);
    __syncthreads();
    cur ^= 1;
    par ^= 1;
  };
  if (MODE == kEmit && page_end - page_begin == kPages) {
    // a whole chunk (the common case): the same steps unrolled with the page
    // count known, so the last two steps request no page past the chunk, the
    // last one stages nothing, and the workgroup ends with no load in flight
    // (the modes that hold score stores keep the loop: unrolled, they spill)
    dsa::static_for<kPages>([&](auto S) {
      constexpr int s = decltype(S)::value;
      flush();
      if constexpr (s + 2 < kPages) {
        if constexpr (s % 2 == 0) load_page(pa, page_begin + s + 2);
        else load_page(pb, page_begin + s + 2);
      }
      if (wave_active) compute_page(page_begin + s);
      if constexpr (s + 1 < kPages) {
        if constexpr (s % 2 == 0) store_page(pb, cur ^ 1);
        else store_page(pa, cur ^ 1);
        __syncthreads();
        cur ^= 1;
      }
    });
  } else {
    int pg = page_begin;
    for (; pg + 1 < page_end; pg += 2) {
      step(pg, pb, pa);
      step(pg + 1, pa, pb);
    }
    if (pg < page_end) step(pg, pb, pa);
  }
  flush();
  if constexpr (MODE == kEmit) {
    // each wave writes out its own tokens' LDS slots (the flushes above were
    // its own LDS writes); the count may exceed em.cap: the selection treats
    // that chunk as overflowed
    // after the count, as (score, position) pairs padded to whole 128-byte
    // lines (a line written in part would make the memory side fetch it first)
    if (wave_active) {
      for (int side = 0; side < (hasB ? 2 : 1); ++side) {
        const int li = 2 * pair + side;
        const int tok = side ? tB : tA;
        const int cnt = side ? cntB : cntA;
        const int n = min(cnt, em.cap);
        const int m = (n + dsa::kCandAlign) / dsa::kCandAlign * dsa::kCandAlign;   // n + 1, whole lines
        int32_t* run = em.cand + 2 * ((int64_t(tok) * em.nch + chunk) * em.capr);
        for (int s2 = lane; s2 < m; s2 += 64) {
          const int e = s2 - 1;   // candidate in pair s2
          const bool real = s2 >= 1 && e < n;
          const int32_t v = s2 == 0 ? cnt : real ? __float_as_int(cand_v[li * kCandLds + e]) : 0;
          const int32_t ps = real ? p_begin + int(cand_p[li * kCandLds + e]) : -1;
          if constexpr (kStream) {   // streamed keys: the pairs bypass the cache too (-1.6%)
            typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(i32x2{v, ps}, reinterpret_cast<i32x2*>(run + 2 * s2));
          } else {
            *reinterpret_cast<int2*>(run + 2 * s2) = make_int2(v, ps);
          }
        }
      }
    }
  }
}

// Workgroup = unit (chunk blockIdx.x, request blockIdx.y, query block
// blockIdx.z).  (A persistent grid with static unit assignment measured
// slower: it loses the dispatcher's balancing of uneven units.)
template <int MODE, bool kStream>
__global__ __launch_bounds__(kThreads, 4) void index_kernel(
    const uint16_t* __restrict__ keys, int num_pages, const int32_t* __restrict__ page_table,
    int pt_stride, const int32_t* __restrict__ q_offsets, const int32_t* __restrict__ tok_pos,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, float* __restrict__ scores,
    int64_t ld, int max_ctx, int num_tokens, dsa::IndexEmit em) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][DSA_PAGE_TOKENS * kRowBf16];
  // emit pass: each token's candidates of the chunk (score, position - chunk
  // start), written to memory once at the end
  __shared__ float cand_v[MODE == kEmit ? kQB * kCandLds : 1];
  __shared__ uint16_t cand_p[MODE == kEmit ? kQB * kCandLds : 1];
  // scores and sample passes: the last computed page's scores, per parity
  __shared__ __attribute__((aligned(16))) float sst[MODE != kEmit ? 2 * kQB * DSA_PAGE_TOKENS : 4];
  index_unit<MODE, kStream>(keys, num_pages, page_table, pt_stride, q_offsets, tok_pos, q_idx, w, scores, ld,
                   max_ctx, num_tokens, em, lds, cand_v, cand_p, sst, blockIdx.x, blockIdx.y,
                   blockIdx.z);
}

}  // namespace

namespace dsa {

dsa_status launch_index(int mode, const dsa_pool* pool, const int32_t* page_table,
                        int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                        int32_t max_q, const int32_t* tok_pos, int32_t num_tokens,
                        int32_t max_ctx, const uint16_t* q_idx, const float* w, float* scores,
                        int64_t ld, const IndexEmit* em, void* stream) {
  // the sample pass has one (sample) page per 32 logical pages
  const int64_t pages = (int64_t(max_ctx) + DSA_PAGE_TOKENS - 1) / DSA_PAGE_TOKENS;
  const int64_t units = mode == kSample ? (pages + kSampleStride - 1) / kSampleStride : pages;
  const int64_t per = mode == kSample ? kSampleChunkPages : kChunkPages;
  const int64_t chunks = (units + per - 1) / per;
  const int64_t qblocks = (int64_t(max_q) + kQB - 1) / kQB;
  if (chunks > 0x7fffffff || num_reqs > 65535 || qblocks > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "indexer: batch exceeds the launch grid limits");
  const uint16_t* keys =
      reinterpret_cast<const uint16_t*>(pool->base + pool->layout.index_plane_offset);
  const dim3 grid{unsigned(chunks), unsigned(num_reqs), unsigned(qblocks)};
  const IndexEmit none{nullptr, nullptr, 0, 0, 0};
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto go = [&](auto kernel, const IndexEmit& e) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, st, keys, pool->num_pages, page_table,
                       pt_stride, q_offsets, tok_pos, q_idx, w, scores, ld, max_ctx, num_tokens, e);
  };
  // Keys are streamed (non-temporal loads) when each request has a single
  // query block and the requests' pages could all be distinct (the pool holds
  // at least as many pages as the requests span).  A pool smaller than that
  // means pages shared across requests (a common prefix), whose keys every
  // request reads again: cached loads (shared-prefix batch: streamed 24%
  // slower).  Sharing inside a larger pool is not detected here; it costs
  // time, never correctness.  The scores mode keeps cached loads either
  // way: streamed, it ran 9-10% slower (1M-context decode 397 -> 434 us,
  // verify batch 468 -> 516 us).
  const bool stream_keys =
      mode != kScores && qblocks <= 1 && int64_t(num_reqs) * pages <= pool->num_pages;
  if (stream_keys) {
    if (mode == kScores) go(index_kernel<kScores, true>, none);
    else if (mode == kSample) go(index_kernel<kSample, true>, none);
    else go(index_kernel<kEmit, true>, *em);
  } else {
    if (mode == kScores) go(index_kernel<kScores, false>, none);
    else if (mode == kSample) go(index_kernel<kSample, false>, none);
    else go(index_kernel<kEmit, false>, *em);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, std::string("indexer: launch failed: ") + hipGetErrorString(e));
  return ok();
}

}  // namespace dsa

extern "C" dsa_status dsa_index_scores(const dsa_pool* pool, const int32_t* page_table,
                                       int32_t pt_stride, const int32_t* q_offsets,
                                       int32_t num_reqs, int32_t max_q, const int32_t* tok_pos,
                                       int32_t num_tokens, int32_t max_ctx, const uint16_t* q_idx,
                                       const float* w, float* scores, int64_t ld, void* stream) {
  dsa_status s = dsa::check_index_scores(pool, page_table, pt_stride, q_offsets, num_reqs, max_q,
                                         tok_pos, num_tokens, max_ctx, q_idx, w, scores, ld);
  if (s != DSA_OK || num_tokens == 0 || max_ctx == 0) return s == DSA_OK ? dsa::ok() : s;
  s = dsa::deep_check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens,
                            "dsa_index_scores", stream);
  if (s != DSA_OK) return s;
  return dsa::launch_index(kScores, pool, page_table, pt_stride, q_offsets, num_reqs, max_q, tok_pos,
                           num_tokens, max_ctx, q_idx, w, scores, ld, nullptr, stream);
}
