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

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kEPT = 64;                       // elements per thread
constexpr int kSeg = kThreads * kEPT;          // 65536
constexpr int kWords = kSeg / 32;              // bitmap words
constexpr int kCoarseBits = 12;                // top key bits of the first histogram
constexpr int kBins = 1 << kCoarseBits;        // 4096
constexpr int kFineBits = 10;                  // 32 - 12 = 20 remaining bits = 2 x 10
constexpr int kCap = 4096;                     // threshold-bin candidates kept in LDS

static_assert(kSeg == dsa::kTopkSeg, "segment size must match the host side");

enum Mode { kDirect = 0, kSegment = 1, kMerge = 2 };

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

template <int MODE>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ tok_pos,
    int max_ctx, int k, int nseg, int kc, float* __restrict__ cand_val,
    int32_t* __restrict__ cand_pos, int32_t* __restrict__ idx_out) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- row geometry
  int t, n, base = 0;
  const float* vals;
  const int32_t* vpos = nullptr;  // merge mode: candidate positions
  if (MODE == kSegment) {
    t = blockIdx.y;
    base = blockIdx.x * kSeg;
    const int vis = min(tok_pos[t], max_ctx - 1) + 1;
    n = max(0, min(vis - base, kSeg));
    vals = scores + int64_t(t) * ld + base;
  } else if (MODE == kMerge) {
    t = blockIdx.x;
    n = nseg * kc;
    vals = cand_val + int64_t(t) * n;
    vpos = cand_pos + int64_t(t) * n;
  } else {
    t = blockIdx.x;
    n = max(0, min(tok_pos[t], max_ctx - 1) + 1);
    vals = scores + int64_t(t) * ld;
  }

  for (int i = tid; i < kBins; i += kThreads) sm.hist[i] = 0;
  if (tid == 0) sm.cand_n = 0;
  __syncthreads();

  // ---- load keys and build the coarse histogram.  Loads are unconditional
  // (clamped into the row, which always holds an element) so all are in flight.
  uint32_t key[kEPT];
  const int cnt = n > tid ? (n - tid + kThreads - 1) / kThreads : 0;
  const int last = max(n - 1, 0);
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    const int e = min(kThreads * i + tid, last);
    key[i] = __float_as_uint(vals[e]);
  }
  uint32_t my_valid = 0;
#pragma unroll
  for (int i = 0; i < kEPT; ++i) {
    bool ok = i < cnt;
    if (MODE == kMerge) ok = ok && vpos[min(kThreads * i + tid, last)] >= 0;
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
      const int64_t o = (int64_t(t) * nseg + blockIdx.x) * kc + out;
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
      const int64_t o = (int64_t(t) * nseg + blockIdx.x) * kc + i;
      cand_val[o] = 0.f;
      cand_pos[o] = -1;
    } else {
      idx_out[int64_t(t) * k + i] = -1;
    }
  }
}

}  // namespace

extern "C" dsa_status dsa_topk(const float* scores, int64_t ld, const int32_t* tok_pos,
                               int32_t num_tokens, int32_t max_ctx, int32_t k, int32_t* idx,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (num_tokens < 0 || max_ctx < 0) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: negative size");
  if (k < 1) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: k must be >= 1");
  if (k > dsa::kTopkMaxK) return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_topk: k above 16384");
  if (num_tokens == 0) return dsa::ok();
  if (!scores || !tok_pos || !idx)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: scores, tok_pos and idx must be non-null");
  if (!dsa::aligned(scores, 16) || !dsa::aligned(tok_pos, 4) || !dsa::aligned(idx, 4))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: scores must be 16-byte aligned");
  if (ld < max_ctx || ld % 4 != 0)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: need ld >= max_ctx and ld % 4 == 0");
  if (num_tokens > 65535 && max_ctx > kSeg)
    return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_topk: too many long rows for one launch");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (max_ctx <= kSeg) {
    hipLaunchKernelGGL(topk_kernel<kDirect>, dim3(num_tokens), dim3(kThreads), 0, st, scores, ld,
                       tok_pos, max_ctx, k, 1, k, nullptr, nullptr, idx);
  } else {
    const int nseg = dsa::topk_num_segments(max_ctx);
    const int kc = (k + 3) & ~3;
    if (int64_t(nseg) * kc > kSeg)
      return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_topk: segments x k exceeds one merge workgroup");
    const size_t need = size_t(num_tokens) * nseg * kc * 8;
    if (!workspace || workspace_bytes < need)
      return dsa::fail(DSA_ERR_WORKSPACE, "dsa_topk: workspace of " + std::to_string(need) +
                                              " bytes required");
    if (!dsa::aligned(workspace, 256))
      return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_topk: workspace must be 256-byte aligned");
    float* cv = static_cast<float*>(workspace);
    int32_t* cp = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             size_t(num_tokens) * nseg * kc * 4);
    hipLaunchKernelGGL(topk_kernel<kSegment>, dim3(nseg, num_tokens), dim3(kThreads), 0, st, scores,
                       ld, tok_pos, max_ctx, k, nseg, kc, cv, cp, nullptr);
    hipLaunchKernelGGL(topk_kernel<kMerge>, dim3(num_tokens), dim3(kThreads), 0, st, scores, ld,
                       tok_pos, max_ctx, k, nseg, kc, cv, cp, idx);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_topk: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
