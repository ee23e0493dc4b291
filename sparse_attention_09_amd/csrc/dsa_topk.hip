// Top-k selection of indexer scores on gfx950.
//
// Keeps the k highest-scoring visible positions of each query token, ties to
// the lower position, and writes them in ascending position order padded with
// -1 (the selection step between the indexer and DSA Partial in "Accelerating
// GLM-5.3-Flash on H200", section 3; tie and order rules are the readings
// documented with the oracle).
//
// One 1024-thread workgroup selects from up to 65,536 elements held in
// registers (64 per thread; element e = 1024*i + tid, loaded with coalesced
// dword loads).  Scores map to order-preserving uint32 keys (invalid -> 0).
//   1. while loading, a 4096-bin LDS histogram of the keys' top 12 bits
//      (sign, exponent, 3 mantissa bits) is built;
//   2. a block suffix scan finds the bin holding the k-th largest key; one
//      pass over the registers marks keys above that bin in an LDS bitmap and
//      appends the bin's keys to an LDS candidate list (rare predicated LDS
//      atomics);
//   3. two 10-bit histogram passes over the candidates only give the exact
//      threshold key and how many keys equal to it are kept (a bin too wide
//      for the list falls back to the same passes over the registers);
//   4. candidates above the threshold and those equal to it go to LDS
//      bitmaps; a block scan over per-thread popcounts keeps the
//      lowest-position equal keys that fit, and a second scan writes the
//      selected positions in ascending order.
// Longer rows are cut into 65,536-position segments whose local top-k
// candidates (kept in ascending position order) are merged by a second pass
// of the same kernel: the global top-k under (score desc, position asc) is
// contained in the union of the segments' top-k.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

using dsa::f32x4;
using dsa::u32x4;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kEPT = 64;                       // elements per thread
constexpr int kSeg = kThreads * kEPT;          // 65536
constexpr int kWords = kSeg / 32;              // bitmap words
constexpr int kCoarseBits = 12;                // top key bits of the first histogram
constexpr int kBins = 1 << kCoarseBits;        // 4096
constexpr int kFineBits = 10;                  // 32 - 12 = 20 remaining bits = 2 x 10
constexpr int kCap = 4096;                     // threshold-bin candidates kept in LDS
// Score bits of an empty slot in a segment's candidate list: a NaN (scores
// never are), whose order key is 0, the key of "no element"; the merge tells
// empty slots by the score alone, without loading their positions.
constexpr uint32_t kEmptyBits = 0xFFFFFFFFu;

static_assert(kSeg == dsa::kTopkSeg, "segment size must match the host side");

enum Mode { kDirect = 0, kSegment = 1, kMerge = 2, kFallback = 3 };

struct Smem {
  uint32_t hist[kBins];
  uint32_t gt_bits[kWords];
  uint32_t eq_bits[kWords];
  uint32_t cand_key[kCap];                     // keys of the threshold bin
  uint32_t cand_idx[kCap];                     // their element indices
  uint32_t wave_tmp[kWaves];
  uint32_t red[4];
  uint32_t sel_digit, sel_above, cand_n;
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive block scan of one value per thread; returns the exclusive prefix,
// and the block total in *total.  Contains barriers.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, Smem& sm, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) sm.wave_tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWaves ? sm.wave_tmp[lane] : 0u;
    uint32_t xi = wave_incl_scan(x, lane);
    if (lane < kWaves) sm.wave_tmp[lane] = xi - x;
    if (lane == kWaves - 1) sm.red[3] = xi;
  }
  __syncthreads();
  uint32_t res = sm.wave_tmp[wave] + inc - v;
  *total = sm.red[3];
  __syncthreads();
  return res;
}

// Finds the bin (of nbins <= kBins, from the top) holding the k_rem-th largest
// key; writes sel_digit and sel_above (count in higher bins).  Thread i looks
// at bins [nbins - (i+1)*per, nbins - i*per).  Contains barriers; the result
// is readable after it returns.
__device__ __forceinline__ void select_bin(Smem& sm, uint32_t k_rem, int nbins, int tid) {
  const int per = nbins / kThreads > 0 ? nbins / kThreads : 1;
  const int top = nbins - per * tid;           // exclusive upper bin of this thread
  uint32_t local = 0;
  if (top > 0)
    for (int b = top - 1; b >= top - per; --b) local += sm.hist[b];
  uint32_t tot;
  const uint32_t above = block_excl_scan(local, sm, &tot);
  if (top > 0 && above < k_rem && k_rem <= above + local) {
    uint32_t acc = above;
    for (int b = top - 1; b >= top - per; --b) {
      const uint32_t h = sm.hist[b];
      if (acc + h >= k_rem) {
        sm.sel_digit = uint32_t(b);
        sm.sel_above = acc;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Indexer inputs of the exact fallback of the fused path (which recomputes a
// token's scores instead of reading them).
struct IndexIn {
  const uint16_t* keys;         // indexer key plane, [page][64][128] bf16
  int num_pages;
  const int32_t* page_table;
  int pt_stride;
  const int32_t* q_offsets;
  int num_reqs;
  const uint16_t* q_idx;        // [T][16][128] bf16
  const float* w;               // [T][16]
};

// The score bits of positions 1024*i + tid (i < kEPT) of token t, computed
// like the indexer kernel: wave v takes the 64 positions (one page) starting
// at 1024*i + 64*v; its four 16-position MFMA blocks use the same operand
// layouts, accumulation order and epilogue as the indexer, so the bits match.
// Positions at or past n are left 0 (masked by the caller).
__device__ __forceinline__ void fallback_scores(uint32_t (&key)[kEPT], const IndexIn& f, int t, int n,
                                                int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  int lo = 0, hi = f.num_reqs;   // request b with q_offsets[b] <= t < q_offsets[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (f.q_offsets[mid] <= t) lo = mid; else hi = mid;
  }
  const int b = lo;
  u32x4 q[4];
  float wv[4];
  const u32x4* qs = reinterpret_cast<const u32x4*>(f.q_idx + (int64_t(t) * DSA_IDX_HEADS + c) * DSA_IDX_DIM);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) q[ks] = qs[ks * 4 + g];
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[j] = f.w[int64_t(t) * DSA_IDX_HEADS + 4 * g + j];
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    const int p0 = kThreads * i + 64 * wave;
    const int lp = p0 / DSA_PAGE_TOKENS;
    float v = 0.f;
    if (p0 < n && lp < f.pt_stride) {   // wave-uniform
      int id = f.page_table[int64_t(b) * f.pt_stride + lp];
      id = min(max(id, 0), f.num_pages - 1);
      const uint16_t* page = f.keys + int64_t(id) * DSA_PAGE_TOKENS * DSA_IDX_DIM;
      for (int b4 = 0; b4 < 4; ++b4) {
        const u32x4* krow = reinterpret_cast<const u32x4*>(page + (16 * b4 + c) * DSA_IDX_DIM) + g;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = dsa::mfma16x16x32(dsa::as_bf16x8(q[ks]), dsa::as_bf16x8(krow[4 * ks]), acc);
        const float sc = dsa::index_score(acc, wv);
        if (g == b4) v = sc;
      }
    }
    key[i] = __float_as_uint(v);
  }
}

struct RowArgs {
  const float* scores;
  int64_t ld;
  const int32_t* tok_pos;
  int max_ctx, k, nseg, kc;
  float* cand_val;
  int32_t* cand_pos;
  int32_t* idx_out;
};

// Selects the top-k of one row: token t's visible scores (kDirect), segment
// seg of them (kSegment), the segments' candidates (kMerge), or the scores
// recomputed from the indexer inputs (kFallback).  Contains barriers; every
// thread of the workgroup calls it with the same row.
template <int MODE>
__device__ __forceinline__ void topk_row(Smem& sm, const RowArgs& a, int t, int seg, const IndexIn& f) {
  const float* __restrict__ scores = a.scores;
  const int64_t ld = a.ld;
  const int max_ctx = a.max_ctx, k = a.k, nseg = a.nseg, kc = a.kc;
  float* __restrict__ cand_val = a.cand_val;
  int32_t* __restrict__ cand_pos = a.cand_pos;
  int32_t* __restrict__ idx_out = a.idx_out;
  int tid = threadIdx.x;
  // the fallback runs one row after another in a loop: an opaque copy of the
  // thread index keeps its per-thread addresses inside the row instead of
  // hoisted out of the loop and held (they spilled)
  if constexpr (MODE == kFallback) asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;

  // ---- row geometry
  int n, base = 0;
  const float* vals = nullptr;
  const int32_t* vpos = nullptr;  // merge mode: candidate positions
  if (MODE == kSegment) {
    base = seg * kSeg;
    const int vis = min(a.tok_pos[t], max_ctx - 1) + 1;
    n = max(0, min(vis - base, kSeg));
    vals = scores + int64_t(t) * ld + base;
  } else if (MODE == kMerge) {
    n = nseg * kc;
    vals = cand_val + int64_t(t) * n;
    vpos = cand_pos + int64_t(t) * n;
  } else {
    n = max(0, min(a.tok_pos[t], max_ctx - 1) + 1);
    if (MODE == kDirect) vals = scores + int64_t(t) * ld;
  }

  for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
  if (tid == 0) sm.cand_n = 0;
  __syncthreads();

  // ---- load keys and build the coarse histogram.  Loads are unconditional
  // (clamped into the row, which always holds an element) so all are in flight.
  uint32_t key[kEPT];
  const int cnt = n > tid ? (n - tid + kThreads - 1) / kThreads : 0;
  const int last = max(n - 1, 0);
  if constexpr (MODE == kFallback) {
    fallback_scores(key, f, t, n, tid);
  } else {
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
      const int e = min(kThreads * i + tid, last);
      key[i] = __float_as_uint(vals[e]);
    }
  }
  uint32_t my_valid = 0;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    bool ok = i < cnt;
    if (MODE == kMerge) ok = ok && key[i] != kEmptyBits;   // an empty segment slot
    key[i] = ok ? dsa::float_key(__uint_as_float(key[i])) : 0u;
    my_valid += ok ? 1u : 0u;
    if (ok) atomicAdd(&sm.hist[key[i] >> (32 - kCoarseBits)], 1u);
  }
  {
    const uint32_t a = wave_sum(my_valid);
    if (lane == 0) sm.wave_tmp[wave] = a;
    __syncthreads();
    if (tid == 0) {
      uint32_t tot = 0;
      for (int i = 0; i < kWaves; ++i) tot += sm.wave_tmp[i];
      sm.red[0] = tot;
    }
    __syncthreads();
  }
  const uint32_t n_valid = sm.red[0];

  // ---- threshold key tau (the k-th largest key), the number r of tau-equal
  // keys to keep, and the bitmaps of kept keys above tau / equal to tau
  uint32_t tau = 0, r = 0;   // tau = 0, r = 0 keeps every valid key
  bool bitmaps_done = false;
  if (n_valid > uint32_t(k)) {
    uint32_t k_rem = uint32_t(k);
    select_bin(sm, k_rem, kBins, tid);
    const uint32_t dsel = sm.sel_digit;
    const uint32_t nsel = sm.hist[dsel];
    k_rem -= sm.sel_above;
    uint32_t prefix = dsel;            // decided high bits of the threshold key
    int hi = 32 - kCoarseBits;         // bits still undecided
    __syncthreads();
    if (nsel <= uint32_t(kCap)) {
      // keys above the bin are kept; the bin's keys become LDS candidates
      for (int i = tid; i < kWords; i += kThreads) {
        sm.gt_bits[i] = 0;
        sm.eq_bits[i] = 0;
      }
      __syncthreads();
      // element 1024e + tid: bitmap word 32e + tid/32, bit tid%32
      uint32_t* gt_word = &sm.gt_bits[tid >> 5];
      const uint32_t bit = 1u << (tid & 31);
#pragma unroll
      for (int e = 0; e < kEPT; ++e) {
        const uint32_t d = key[e] >> hi;
        if (key[e] != 0 && d >= dsel) {
          if (d > dsel) {
            atomicOr(gt_word + 32 * e, bit);
          } else {
            const uint32_t slot = atomicAdd(&sm.cand_n, 1u);
            sm.cand_key[slot] = key[e];
            sm.cand_idx[slot] = uint32_t(kThreads * e + tid);
          }
        }
      }
      __syncthreads();
      // refine among the candidates only
      while (hi > 0) {
        const int sh = hi - kFineBits;
        for (int i = tid; i < (1 << kFineBits); i += kThreads) sm.hist[i] = 0;
        __syncthreads();
        for (uint32_t j = tid; j < nsel; j += kThreads) {
          const uint32_t c = sm.cand_key[j];
          if ((c >> hi) == prefix) atomicAdd(&sm.hist[(c >> sh) & ((1u << kFineBits) - 1u)], 1u);
        }
        __syncthreads();
        select_bin(sm, k_rem, 1 << kFineBits, tid);
        prefix = (prefix << kFineBits) | sm.sel_digit;
        k_rem -= sm.sel_above;
        hi = sh;
        __syncthreads();
      }
      // mark the candidates kept: above the exact threshold, or equal to it
      for (uint32_t j = tid; j < nsel; j += kThreads) {
        const uint32_t c = sm.cand_key[j], ei = sm.cand_idx[j];
        if (c > prefix) atomicOr(&sm.gt_bits[ei >> 5], 1u << (ei & 31));
        else if (c == prefix) atomicOr(&sm.eq_bits[ei >> 5], 1u << (ei & 31));
      }
      bitmaps_done = true;
    } else {
      // wide threshold bin (heavy ties): refine over the registers
      while (hi > 0) {
        const int sh = hi - kFineBits;
        for (int i = tid; i < (1 << kFineBits); i += kThreads) sm.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kEPT; ++e) {
          const uint32_t c = key[e];
          if (c != 0 && (c >> hi) == prefix) atomicAdd(&sm.hist[(c >> sh) & ((1u << kFineBits) - 1u)], 1u);
        }
        __syncthreads();
        select_bin(sm, k_rem, 1 << kFineBits, tid);
        prefix = (prefix << kFineBits) | sm.sel_digit;
        k_rem -= sm.sel_above;
        hi = sh;
        __syncthreads();
      }
    }
    tau = prefix;
    r = k_rem;
  }

  if (!bitmaps_done) {
    // bitmaps straight from the registers: one ballot per 64 consecutive
    // elements, written by lane 0 (no atomics)
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
      const uint32_t kk = key[i];
      const uint64_t mg = __ballot(kk > tau);
      const uint64_t me = __ballot(r > 0 && kk == tau);
      if (lane == 0) {
        const int wd = (kThreads * i + 64 * wave) >> 5;
        sm.gt_bits[wd] = uint32_t(mg);
        sm.gt_bits[wd + 1] = uint32_t(mg >> 32);
        sm.eq_bits[wd] = uint32_t(me);
        sm.eq_bits[wd + 1] = uint32_t(me >> 32);
      }
    }
  }
  __syncthreads();

  // ---- thread i owns elements [64i, 64i+64): keep the lowest-position equal keys
  const uint32_t w0 = 2 * tid, w1 = 2 * tid + 1;
  uint64_t gtm = uint64_t(sm.gt_bits[w0]) | (uint64_t(sm.gt_bits[w1]) << 32);
  uint64_t eqm = uint64_t(sm.eq_bits[w0]) | (uint64_t(sm.eq_bits[w1]) << 32);
  uint32_t tot_eq;
  const uint32_t eq_before = block_excl_scan(uint32_t(__popcll(eqm)), sm, &tot_eq);
  uint64_t kept = 0;
  if (eq_before < r) {
    uint32_t take = r - eq_before;
    uint64_t x = eqm;
    while (take > 0 && x) {
      const uint64_t low = x & (~x + 1);
      kept |= low;
      x ^= low;
      --take;
    }
  }
  const uint64_t sel = gtm | kept;
  uint32_t total;
  uint32_t out = block_excl_scan(uint32_t(__popcll(sel)), sm, &total);

  // ---- write selected positions ascending, then -1 padding
  const int limit = (MODE == kSegment) ? kc : k;
  uint64_t x = sel;
  while (x && int(out) < limit) {
    const int bit = __ffsll((unsigned long long)x) - 1;
    x &= x - 1;
    const int e = 64 * tid + bit;
    if (MODE == kSegment) {
      const int64_t o = (int64_t(t) * nseg + seg) * kc + out;
      cand_val[o] = vals[e];
      cand_pos[o] = base + e;
    } else if (MODE == kMerge) {
      idx_out[int64_t(t) * k + out] = vpos[e];
    } else {
      idx_out[int64_t(t) * k + out] = e;
    }
    ++out;
  }
  for (int i = int(total) + tid; i < limit; i += kThreads) {
    if (MODE == kSegment) {
      const int64_t o = (int64_t(t) * nseg + seg) * kc + i;
      cand_val[o] = __uint_as_float(kEmptyBits);
      cand_pos[o] = -1;
    } else {
      idx_out[int64_t(t) * k + i] = -1;
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void topk_kernel(RowArgs a) {
  __shared__ Smem sm;
  const IndexIn none{nullptr, 0, nullptr, 0, nullptr, 0, nullptr, nullptr};
  topk_row<MODE>(sm, a, MODE == kSegment ? int(blockIdx.y) : int(blockIdx.x), blockIdx.x, none);
}

// ===================================================================== fused
// Fused indexer + top-k for rows of at most 65,536 positions (no score
// matrix):
//   1. the indexer's sample pass scores logical pages 0, 32, 64, ...;
//   2. threshold_kernel: per token, the r-th largest sampled score, r chosen
//      so that about `target` positions of the row should reach it;
//   3. the indexer's emit pass keeps only positions scoring at least the
//      threshold, in position order, in fixed slots per (token, 512-chunk);
//   4. select_kernel: when no chunk overflowed and at least k candidates
//      exist, the exact top-k of the row lies among them (every other
//      position scores strictly below every candidate, so it cannot beat or
//      tie the k-th largest), and selecting among them under the same rule
//      (score desc, position asc) gives the same answer; otherwise the token
//      is listed;
//   5. fallback_kernel: listed tokens recompute their row into registers and
//      run the one-workgroup selection above.

constexpr int kSmallThreads = 256;
constexpr int kMaxSamples = 2048;     // sample columns of a 65,536-position row
constexpr int kSelMax = 6144;         // candidates one selection workgroup holds
constexpr int kMaxChunks = kSeg / dsa::kIndexChunk;
constexpr int kRankSlack = 8;         // extra sample rank: fewer short-of-k rows

// Block-level helpers for an NT-thread workgroup (NT a multiple of 64, at
// least 256).
template <int NT>
struct SelT {
  uint32_t hist[2][256];
  uint32_t wtmp[NT / 64][4];
  uint32_t digit, above;
};
using Sel = SelT<kSmallThreads>;

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, uint32_t(__shfl_xor(v, off)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, uint32_t(__shfl_xor(v, off)));
  return v;
}

// Exclusive scan over the workgroup; *total gets the sum.  Barriers.
template <int NT>
__device__ __forceinline__ uint32_t scan_block(uint32_t v, SelT<NT>& s, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v, lane);
  if (lane == 63) s.wtmp[wave][0] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t x = s.wtmp[i][0];
    before += i < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}
__device__ __forceinline__ uint32_t scan256(uint32_t v, Sel& s, uint32_t* total) {
  return scan_block<kSmallThreads>(v, s, total);
}

// Minimum and maximum of keys (lo/hi per thread) and a count sum over the
// workgroup.  Barriers.
template <int NT>
__device__ __forceinline__ void minmax_block(SelT<NT>& s, uint32_t lo, uint32_t hi, uint32_t n,
                                             uint32_t* glo, uint32_t* ghi, uint32_t* gn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lo = wave_min(lo);
  hi = wave_max(hi);
  n = wave_sum(n);
  if (lane == 0) {
    s.wtmp[wave][1] = lo;
    s.wtmp[wave][2] = hi;
    s.wtmp[wave][3] = n;
  }
  __syncthreads();
  lo = s.wtmp[0][1];
  hi = s.wtmp[0][2];
  n = s.wtmp[0][3];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) {
    lo = min(lo, s.wtmp[i][1]);
    hi = max(hi, s.wtmp[i][2]);
    n += s.wtmp[i][3];
  }
  __syncthreads();
  *glo = lo;
  *ghi = hi;
  *gn = n;
}
__device__ __forceinline__ void minmax256(Sel& s, uint32_t lo, uint32_t hi, uint32_t n,
                                          uint32_t* glo, uint32_t* ghi, uint32_t* gn) {
  minmax_block<kSmallThreads>(s, lo, hi, n, glo, ghi, gn);
}

// k-th largest of a key multiset spread over the workgroup (1 <= k <= its
// size; every key in [kmin, kmax]).  Radix selection on d = key - kmin, in
// digits of 8 bits taken from the top bit of kmax - kmin down (the last digit
// takes what is left), so the first digit already spreads the keys over the
// histogram instead of piling them into a few bins.  `each(f)` calls f on
// every key the calling thread holds.  Returns the key; *r_out gets how many
// keys equal to it belong to the k largest.  Barriers.
template <int NT, class Each>
__device__ __forceinline__ uint32_t radix_select_block(SelT<NT>& s, uint32_t k_rem, uint32_t kmin,
                                                       uint32_t kmax, Each each, uint32_t* r_out) {
  const int tid = threadIdx.x;
  const uint32_t span = kmax - kmin;
  if (span == 0) {
    *r_out = k_rem;
    return kmin;
  }
  const int bits = 32 - __clz(span);
  const int passes = (bits + 7) / 8;
  uint32_t prefix = 0;   // decided high bits of d: bits [top, bits)
  int top = bits;
  if (tid < 256) s.hist[0][tid] = 0;
  __syncthreads();
  for (int pass = 0; pass < passes; ++pass) {
    const int sh = max(top - 8, 0);                  // this digit: bits [sh, top)
    const uint32_t dmask = (1u << (top - sh)) - 1u;
    uint32_t* h = s.hist[pass & 1];
    if (tid < 256) s.hist[(pass + 1) & 1][tid] = 0;   // the next pass's histogram
    each([&](uint32_t key) {
      const uint32_t d = key - kmin;
      const uint32_t hi = top >= 32 ? 0u : d >> top;
      if (hi == prefix) atomicAdd(&h[(d >> sh) & dmask], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      // lane l scans bins 255-4l .. 252-4l (top down)
      uint32_t hb[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hb[j] = h[255 - 4 * tid - j];
        local += hb[j];
      }
      const uint32_t inc = wave_incl_scan(local, tid);
      uint32_t acc = inc - local;
      if (acc < k_rem && k_rem <= inc) {
        for (int j = 0; j < 4; ++j) {
          if (acc + hb[j] >= k_rem) {
            s.digit = uint32_t(255 - 4 * tid - j);
            s.above = acc;
            break;
          }
          acc += hb[j];
        }
      }
    }
    __syncthreads();
    prefix = (prefix << (top - sh)) | s.digit;
    k_rem -= s.above;
    top = sh;
  }
  *r_out = k_rem;
  return kmin + prefix;
}
template <class Each>
__device__ __forceinline__ uint32_t radix_select256(Sel& s, uint32_t k_rem, uint32_t kmin,
                                                    uint32_t kmax, Each each, uint32_t* r_out) {
  return radix_select_block<kSmallThreads>(s, k_rem, kmin, kmax, each, r_out);
}

// One workgroup per token.  Sample column q lies at position
// 2048*(q/64) + q%64.  Writes the token's threshold score (-inf: keep every
// position).  Also resets the fallback list (block 0).
__global__ __launch_bounds__(kSmallThreads) void threshold_kernel(
    const float* __restrict__ samples, int ls, const int32_t* __restrict__ tok_pos, int max_ctx,
    int k, int target, float* __restrict__ thr, int32_t* __restrict__ nflag) {
  __shared__ Sel s;
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t == 0 && tid == 0) *nflag = 0;
  const int vis = max(0, min(tok_pos[t], max_ctx - 1) + 1);
  if (vis <= k) {          // the selection keeps the whole row
    if (tid == 0) thr[t] = -__builtin_inff();
    return;
  }
  constexpr int kPer = kMaxSamples / kSmallThreads;
  uint32_t key[kPer];
  bool ok[kPer];
  uint32_t nv = 0, lo = 0xFFFFFFFFu, hi = 0u;
  // loads unconditional (a column past the row reads column 0) so all are in
  // flight at once
  float sv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + kSmallThreads * i;
    sv[i] = samples[int64_t(t) * ls + (q < ls ? q : 0)];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = tid + kSmallThreads * i;
    const int p = dsa::kIndexSampleStride * DSA_PAGE_TOKENS * (q >> 6) + (q & 63);
    ok[i] = q < ls && p < vis;
    key[i] = ok[i] ? dsa::float_key(sv[i]) : 0u;
    nv += ok[i] ? 1u : 0u;
    lo = ok[i] ? min(lo, key[i]) : lo;
    hi = ok[i] ? max(hi, key[i]) : hi;
  }
  uint32_t kmin, kmax, ns;
  minmax256(s, lo, hi, nv, &kmin, &kmax, &ns);
  const int64_t r = (int64_t(target) * ns + vis - 1) / vis + kRankSlack;
  if (r >= int64_t(ns)) {  // too few samples to cut anything: keep every position
    if (tid == 0) thr[t] = -__builtin_inff();
    return;
  }
  uint32_t rr;
  const uint32_t tau = radix_select256(
      s, uint32_t(r), kmin, kmax,
      [&](auto&& f) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (ok[i]) f(key[i]);
      },
      &rr);
  if (tid == 0) thr[t] = dsa::key_float(tau);
}

struct SelSmem {
  uint32_t key[kSelMax];
  uint16_t pos[kSelMax];      // rows are at most 65,536 positions
  int32_t off[kMaxChunks];
  Sel s;
};

// One workgroup per token: compacts its candidates into LDS (in position
// order), selects exactly, writes the k positions ascending.  Rows of at
// most k positions are written whole.  Tokens whose candidates cannot be
// trusted go to the fallback list.
__global__ __launch_bounds__(kSmallThreads) void select_kernel(
    const int32_t* __restrict__ tok_pos, int max_ctx, int k,
    const int2* __restrict__ cand, int nch, int cap, int capr, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ nflag, int32_t* __restrict__ flag_list) {
  __shared__ SelSmem sm;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int vis = max(0, min(tok_pos[t], max_ctx - 1) + 1);
  int32_t* out = idx_out + int64_t(t) * k;
  if (vis <= k) {
    for (int i = tid; i < k; i += kSmallThreads) out[i] = i < vis ? i : -1;
    return;
  }
  const int nch_t = (vis + dsa::kIndexChunk - 1) / dsa::kIndexChunk;
  int c = 0;
  bool over = false;
  if (tid < nch_t) {
    c = cand[(int64_t(t) * nch + tid) * capr].x;   // the region's count pair
    over = c > cap || c < 0;
  }
  uint32_t n;
  const uint32_t o = scan256(over ? 0u : uint32_t(c), sm.s, &n);
  if (tid < nch_t) sm.off[tid] = int32_t(o);
  const bool bad = __syncthreads_or(over) || n < uint32_t(k) || n > uint32_t(kSelMax);
  if (bad) {
    if (tid == 0) flag_list[atomicAdd(nflag, 1)] = t;
    return;
  }
  const int N = int(n);
  // compaction, all loads of a thread in flight together: candidate q is slot
  // q - off[j] of the chunk j holding it.  The chunk of every candidate is
  // first written into pos[] (its slots, by the chunk's thread), so each
  // candidate takes two independent LDS reads (a binary search over the
  // offsets is seven dependent ones per candidate, and they ran one after
  // another).
  if (tid < nch_t)
    for (int s2 = 0; s2 < c; ++s2) sm.pos[o + s2] = uint16_t(tid);
  __syncthreads();
  constexpr int kPer = kSelMax / kSmallThreads;
  int chunk_of[kPer], first_of[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int j = sm.pos[kSmallThreads * u + tid];   // stale past N: clamped below
    chunk_of[u] = j < nch_t ? j : 0;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) first_of[u] = sm.off[chunk_of[u]];
  int64_t src[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int q = kSmallThreads * u + tid;
    src[u] = q < N ? (int64_t(t) * nch + chunk_of[u]) * capr + 1 + (q - first_of[u]) : -1;
  }
  // loads unconditional (an unused slot reads the token's first slot) so all
  // are in flight at once; LDS writes after
  float v[kPer];
  int32_t pv[kPer];
  const int64_t first = int64_t(t) * nch * capr + 1;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int2 x = cand[src[u] >= 0 ? src[u] : first];
    v[u] = __int_as_float(x.x);
    pv[u] = x.y;
  }
  // the keys stay in registers for the radix passes (read back from LDS they
  // were one dependent read per key and pass)
  uint32_t lo = 0xFFFFFFFFu, hi = 0u, held = 0u;
  uint32_t kreg[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    kreg[u] = dsa::float_key(v[u]);
    if (src[u] >= 0) {
      const int q = kSmallThreads * u + tid;
      sm.key[q] = kreg[u];
      sm.pos[q] = uint16_t(pv[u]);
      lo = min(lo, kreg[u]);
      hi = max(hi, kreg[u]);
      held |= 1u << u;
    }
  }
  uint32_t kmin, kmax, unused;
  minmax256(sm.s, lo, hi, 0u, &kmin, &kmax, &unused);   // its barriers publish sm.key/pos
  uint32_t r;
  const uint32_t tau = radix_select256(
      sm.s, uint32_t(k), kmin, kmax,
      [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if ((held >> u) & 1u) f(kreg[u]);
      },
      &r);
  // thread i owns candidates [E*i, E*i + E): equal keys kept lowest position first
  const int E = (N + kSmallThreads - 1) / kSmallThreads;
  const int q0 = min(tid * E, N), q1 = min(q0 + E, N);
  uint32_t gt = 0, eq = 0;
  for (int q = q0; q < q1; ++q) {
    const uint32_t key = sm.key[q];
    gt += key > tau ? 1u : 0u;
    eq += key == tau ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t eq_before = scan256(eq, sm.s, &tot);
  uint32_t take = eq_before < r ? min(eq, r - eq_before) : 0u;
  uint32_t w = scan256(gt + take, sm.s, &tot);
  for (int q = q0; q < q1; ++q) {
    const uint32_t key = sm.key[q];
    bool keep = key > tau;
    if (key == tau && take > 0) {
      keep = true;
      --take;
    }
    if (keep && w < uint32_t(k)) out[w++] = int32_t(sm.pos[q]);   // exactly k are kept
  }
}

// ================================================================ DCP merge
// Round-robin KV shards (position p lives on shard p % G at local position
// p / G): each shard selects its local top-k; the global top-k is contained in
// the union of those lists (a position outside its shard's list is beaten by k
// positions of that shard already), so one exact selection over at most G*k
// candidates under the same rule gives it.  One 1024-thread workgroup per token.
constexpr int kMergeMax = dsa::kDcpMergeMax;     // G*k candidates held in LDS

constexpr int kMergeThreads = 1024;
using MSel = SelT<kMergeThreads>;

struct MergeSmem {
  // pass A: candidate keys (0: empty slot); afterwards the kept positions:
  // those above the threshold from 0, the ties after them, then sorted
  uint32_t buf[kMergeMax];
  MSel s;
  uint32_t n_gt, n_eq;
};

// Loads candidate e (entry e % k of shard e / k): its key (0 when empty) and
// global position.  Loads are issued for 8 candidates at once.
struct MergeIn {
  int G, T, k, n;
  const int32_t* local_idx;
  const float* local_scores;
  int64_t ld;
};

template <class F>
__device__ __forceinline__ void merge_for_each(const MergeIn& in, int t, F f) {
  for (int base = 0; base < in.n; base += kMergeThreads * 8) {
    int32_t j[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + kMergeThreads * u + threadIdx.x;
      j[u] = -1;
      if (e < in.n) j[u] = in.local_idx[(int64_t(e / in.k) * in.T + t) * in.k + e % in.k];
    }
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + kMergeThreads * u + threadIdx.x;
      const int r = e < in.n ? e / in.k : 0;
      v[u] = in.local_scores[(int64_t(r) * in.T + t) * in.ld + (j[u] >= 0 ? j[u] : 0)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = base + kMergeThreads * u + threadIdx.x;
      const bool ok = e < in.n && j[u] >= 0;
      f(e, ok ? dsa::float_key(v[u]) : 0u, ok ? j[u] * in.G + e / in.k : -1);
    }
  }
}

// Appends `val` at list position base + (count so far) for the lanes with
// `cond`, one LDS atomic per wave.
__device__ __forceinline__ void wave_append(bool cond, uint32_t val, uint32_t* counter,
                                            uint32_t base, uint32_t* list) {
  const uint64_t m = __ballot(cond);
  if (m == 0ull) return;
  const int lane = threadIdx.x & 63;
  uint32_t first = 0;
  if (lane == 0) first = atomicAdd(counter, uint32_t(__popcll((long long)m)));
  first = __shfl(first, 0);
  if (cond) {
    const uint32_t below = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
    list[base + first + below] = val;
  }
}

__global__ __launch_bounds__(kMergeThreads) void dcp_merge_kernel(
    int G, int T, int k, const int32_t* __restrict__ local_idx, const float* __restrict__ local_scores,
    int64_t ld, int32_t* __restrict__ idx_out, int32_t* __restrict__ shard_idx) {
  __shared__ MergeSmem sm;
  const int t = blockIdx.x, tid = threadIdx.x;
  const MergeIn in{G, T, k, G * k, local_idx, local_scores, ld};
  // ---- pass A: keys into LDS, count / range, the threshold key
  uint32_t nv = 0, lo = 0xFFFFFFFFu, hi = 0u;
  merge_for_each(in, t, [&](int e, uint32_t key, int32_t) {
    if (e < in.n) sm.buf[e] = key;
    if (key != 0u) {
      ++nv;
      lo = min(lo, key);
      hi = max(hi, key);
    }
  });
  if (tid == 0) {
    sm.n_gt = 0;
    sm.n_eq = 0;
  }
  uint32_t kmin, kmax, N;
  minmax_block<kMergeThreads>(sm.s, lo, hi, nv, &kmin, &kmax, &N);   // barriers publish buf
  const bool all = N <= uint32_t(k);
  uint32_t tau = 0, r_eq = 0;
  if (!all) {
    tau = radix_select_block<kMergeThreads>(
        sm.s, uint32_t(k), kmin, kmax,
        [&](auto&& f) {
          for (int e = tid; e < in.n; e += kMergeThreads)
            if (sm.buf[e] != 0u) f(sm.buf[e]);
        },
        &r_eq);
  }
  __syncthreads();   // buf is reused below
  // ---- pass B: positions above the threshold from 0, the ties after them
  const uint32_t eq_base = all ? 0u : uint32_t(k) - r_eq;
  merge_for_each(in, t, [&](int, uint32_t key, int32_t p) {
    const bool gt = key != 0u && (all || key > tau);
    const bool eq = key != 0u && !all && key == tau;
    wave_append(gt, uint32_t(p), &sm.n_gt, 0u, sm.buf);
    wave_append(eq, uint32_t(p), &sm.n_eq, eq_base, sm.buf);
  });
  __syncthreads();
  const uint32_t n_eq = sm.n_eq;
  if (!all && n_eq > r_eq) {
    // keep the r_eq lowest positions among the ties: the r_eq-th largest of ~pos
    uint32_t rr;
    const uint32_t inv = radix_select_block<kMergeThreads>(
        sm.s, r_eq, 0x80000000u, 0xFFFFFFFFu,
        [&](auto&& f) {
          for (uint32_t e = tid; e < n_eq; e += kMergeThreads) f(~sm.buf[eq_base + e]);
        },
        &rr);
    const uint32_t p_cut = ~inv;
    // compact the kept ties to the front of their region (each thread first
    // reads its entries, then the scan's barriers order the writes after)
    uint32_t mine[kMergeMax / kMergeThreads];
    uint32_t c = 0;
    for (uint32_t e = tid, i = 0; e < n_eq; e += kMergeThreads, ++i) {
      const uint32_t p = sm.buf[eq_base + e];
      if (p <= p_cut) mine[c++] = p;
    }
    uint32_t tot;
    const uint32_t o = scan_block<kMergeThreads>(c, sm.s, &tot);
    for (uint32_t i = 0; i < c; ++i) sm.buf[eq_base + o + i] = mine[i];
  }
  // ---- bitonic sort of the kept positions (padded to a power of two)
  const int m = all ? int(N) : k;
  int P = 1;
  while (P < m) P <<= 1;
  for (int e = m + tid; e < P; e += kMergeThreads) sm.buf[e] = 0x7FFFFFFFu;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int e = tid; e < P / 2; e += kMergeThreads) {
        const int a = 2 * e - (e & (stride - 1));   // lower index of the pair
        const int b = a + stride;
        const bool up = (a & size) == 0;
        const uint32_t x = sm.buf[a], y = sm.buf[b];
        if ((x > y) == up) {
          sm.buf[a] = y;
          sm.buf[b] = x;
        }
      }
      __syncthreads();
    }
  }
  // ---- global list, then each shard's local list (ascending, -1 padded)
  int32_t* out = idx_out + int64_t(t) * k;
  for (int i = tid; i < k; i += kMergeThreads) out[i] = i < m ? int32_t(sm.buf[i]) : -1;
  if (shard_idx) {
    const int E = (m + kMergeThreads - 1) / kMergeThreads;
    const int q0 = min(tid * E, m), q1 = min(q0 + E, m);
    for (int r = 0; r < G; ++r) {
      uint32_t c = 0;
      for (int q = q0; q < q1; ++q) c += (int(sm.buf[q]) % G == r) ? 1u : 0u;
      uint32_t tot;
      uint32_t o = scan_block<kMergeThreads>(c, sm.s, &tot);
      int32_t* dst = shard_idx + (int64_t(r) * T + t) * k;
      for (int q = q0; q < q1; ++q) {
        const int p = int(sm.buf[q]);
        if (p % G == r) dst[o++] = p / G;
      }
      for (int i = int(tot) + tid; i < k; i += kMergeThreads) dst[i] = -1;
    }
  }
}

// Persistent over the fallback list (every workgroup leaves once the list is
// exhausted).
__global__ __launch_bounds__(kThreads) void fallback_kernel(RowArgs a, IndexIn f,
                                                            const int32_t* __restrict__ nflag,
                                                            const int32_t* __restrict__ flag_list) {
  __shared__ Smem sm;
  const int n = *nflag;
  for (int li = blockIdx.x; li < n; li += gridDim.x) {
    topk_row<kFallback>(sm, a, flag_list[li], 0, f);
    __syncthreads();
  }
}

}  // namespace

namespace {

// The launches of one top-k call; the long-row staging (candidate scores and
// positions of every token and segment) is at cand, already checked to hold
// dsa_topk_workspace_bytes(num_tokens, max_ctx, k) bytes.
dsa_status launch_topk(const char* who, const float* scores, int64_t ld, const int32_t* tok_pos,
                       int32_t num_tokens, int32_t max_ctx, int32_t k, int32_t* idx, void* cand,
                       void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (max_ctx <= kSeg) {
    const RowArgs a{scores, ld, tok_pos, max_ctx, k, 1, k, nullptr, nullptr, idx};
    hipLaunchKernelGGL(topk_kernel<kDirect>, dim3(num_tokens), dim3(kThreads), 0, st, a);
  } else {
    const int nseg = dsa::topk_num_segments(max_ctx);
    const int kc = (k + 3) & ~3;
    float* cv = static_cast<float*>(cand);
    int32_t* cp = reinterpret_cast<int32_t*>(static_cast<char*>(cand) +
                                             size_t(num_tokens) * nseg * kc * 4);
    const RowArgs a{scores, ld, tok_pos, max_ctx, k, nseg, kc, cv, cp, idx};
    hipLaunchKernelGGL(topk_kernel<kSegment>, dim3(nseg, num_tokens), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(topk_kernel<kMerge>, dim3(num_tokens), dim3(kThreads), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
  return dsa::ok();
}

}  // namespace

extern "C" dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* tok_pos,
                               int32_t num_tokens, int32_t max_ctx, int32_t k, int32_t* idx,
                               void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status s = dsa::check_topk("dsa_topk", scores, ld, tok_pos, num_tokens, max_ctx, k, idx);
  if (s != DSA_OK) return s;
  if (num_tokens == 0) return dsa::ok();
  s = dsa::check_workspace("dsa_topk", workspace, workspace_bytes,
                           dsa_topk_workspace_bytes(num_tokens, max_ctx, k));
  if (s != DSA_OK) return s;
  return launch_topk("dsa_topk", scores, ld, tok_pos, num_tokens, max_ctx, k, idx, workspace,
                     stream);
}

// ---------------------------------------------------------------------------
// Allocation-free top-k: the long-row staging lives in this library-owned
// device array (one copy per GPU, held until the process ends) instead of a
// caller workspace.  Host code never uses the array's name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device on its first call and kept.
static __device__ __align__(256) unsigned char scratch[DSA_TOPK_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_address(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string(who) + ": hipGetDevice failed: " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return dsa::fail(DSA_ERR_UNSUPPORTED, std::string(who) + ": device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dsa::fail(DSA_ERR_HIP, std::string(who) + ": hipGetSymbolAddress(scratch) failed: " +
                                        hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" dsa_status dsa_topk_noalloc(const float* scores, int64_t ld, const int32_t* tok_pos,
                                       int32_t num_tokens, int32_t max_ctx, int32_t k, int32_t* idx,
                                       void* stream) {
  const char* who = "dsa_topk_noalloc";
  dsa_status s = dsa::check_topk(who, scores, ld, tok_pos, num_tokens, max_ctx, k, idx);
  if (s != DSA_OK) return s;
  if (num_tokens == 0) return dsa::ok();
  const size_t need = dsa_topk_workspace_bytes(num_tokens, max_ctx, k);
  if (need > DSA_TOPK_SCRATCH_BYTES)
    return dsa::fail(DSA_ERR_WORKSPACE, std::string(who) + ": the long-row staging needs " +
                                            std::to_string(need) + " bytes, above the " +
                                            std::to_string(DSA_TOPK_SCRATCH_BYTES) +
                                            "-byte library scratch");
  void* cand = nullptr;
  if (need > 0) {
    s = scratch_address(who, &cand);
    if (s != DSA_OK) return s;
  }
  return launch_topk(who, scores, ld, tok_pos, num_tokens, max_ctx, k, idx, cand, stream);
}

extern "C" size_t dsa_index_topk_workspace_bytes(int32_t num_tokens, int32_t max_ctx, int32_t cap) {
  if (num_tokens <= 0 || max_ctx < 0 || max_ctx > kSeg || cap < 1 || cap > dsa::kIndexMaxCap) return 0;
  return dsa::fused_layout(num_tokens, max_ctx, cap).total;
}

extern "C" dsa_status dsa_index_topk(const dsa_pool* pool, const int32_t* page_table,
                                     int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                                     int32_t max_q, const int32_t* tok_pos, int32_t num_tokens,
                                     int32_t max_ctx, const uint16_t* q_idx, const float* w,
                                     int32_t k, int32_t cap, int32_t cand_target, int32_t* idx,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status s = dsa::check_index_topk(pool, page_table, pt_stride, q_offsets, num_reqs, max_q,
                                       tok_pos, num_tokens, max_ctx, q_idx, w, k, cap, cand_target,
                                       idx, workspace, workspace_bytes);
  if (s != DSA_OK || num_tokens == 0) return s == DSA_OK ? dsa::ok() : s;
  s = dsa::deep_check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens,
                            "dsa_index_topk", stream);
  if (s != DSA_OK) return s;
  const dsa::FusedLayout L = dsa::fused_layout(num_tokens, max_ctx, cap);
  char* ws = static_cast<char*>(workspace);
  int32_t* nflag = reinterpret_cast<int32_t*>(ws + L.nflag);
  int32_t* list = reinterpret_cast<int32_t*>(ws + L.list);
  float* samples = reinterpret_cast<float*>(ws + L.samples);
  float* thr = reinterpret_cast<float*>(ws + L.thr);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + L.cand);
  // default: about 2k candidates (within what one selection workgroup holds)
  const int target = cand_target > 0 ? cand_target : std::min(2 * k, kSelMax - 1024);
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (max_ctx > 0) {
    s = dsa::launch_index(1, pool, page_table, pt_stride, q_offsets, num_reqs, max_q, tok_pos,
                          num_tokens, max_ctx, q_idx, w, samples, L.ls, nullptr, stream);
    if (s != DSA_OK) return s;
  }
  hipLaunchKernelGGL(threshold_kernel, dim3(num_tokens), dim3(kSmallThreads), 0, st, samples, L.ls,
                     tok_pos, max_ctx, k, target, thr, nflag);
  if (max_ctx > 0) {
    const dsa::IndexEmit em{thr, cand, L.nch, cap, L.capr};
    s = dsa::launch_index(2, pool, page_table, pt_stride, q_offsets, num_reqs, max_q, tok_pos,
                          num_tokens, max_ctx, q_idx, w, nullptr, 0, &em, stream);
    if (s != DSA_OK) return s;
  }
  hipLaunchKernelGGL(select_kernel, dim3(num_tokens), dim3(kSmallThreads), 0, st, tok_pos, max_ctx,
                     k, reinterpret_cast<const int2*>(cand), L.nch, cap, L.capr, idx, nflag,
                     list);
  const RowArgs a{nullptr, 0, tok_pos, max_ctx, k, 1, k, nullptr, nullptr, idx};
  const IndexIn f{reinterpret_cast<const uint16_t*>(pool->base + pool->layout.index_plane_offset),
                  pool->num_pages, page_table, pt_stride, q_offsets, num_reqs, q_idx, w};
  hipLaunchKernelGGL(fallback_kernel, dim3(std::min(num_tokens, 256)), dim3(kThreads), 0, st, a, f,
                     nflag, list);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_index_topk: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}

extern "C" dsa_status dsa_dcp_merge(int32_t num_shards, int32_t num_tokens, int32_t k,
                                    const int32_t* local_idx, const float* local_scores,
                                    int64_t ld, int32_t* idx, int32_t* shard_idx, void* stream) {
  const dsa_status s = dsa::check_dcp_merge(num_shards, num_tokens, k, local_idx, local_scores, ld,
                                            idx, shard_idx);
  if (s != DSA_OK || num_tokens == 0) return s == DSA_OK ? dsa::ok() : s;
  hipLaunchKernelGGL(dcp_merge_kernel, dim3(num_tokens), dim3(kMergeThreads), 0,
                     static_cast<hipStream_t>(stream), num_shards, num_tokens, k, local_idx,
                     local_scores, ld, idx, shard_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_dcp_merge: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
