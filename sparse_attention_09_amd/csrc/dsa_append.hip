// Writing new tokens into the cache on gfx950: quantize + append.
//
// "GLM-5.3-Flash" SGLang cookbook, section 2 ("Size both memory pools"): the
// paged KV pool holds the latent rows - FP8 by default on MI355X - and the DSA
// indexer pool the indexer keys.  The pages do not spell the quantizer out;
// the reading used here (and by the oracle): per group of 64 consecutive
// elements the scale is the smallest power of two 2^k with amax <= 448 * 2^k
// (1 for an all-zero group), stored as fp32, and code = E4M3FN(x / scale),
// rounded to the nearest finite value with ties to the even code (x / scale
// is exact and within +-448); the row's 28 pad bytes are written as 0.
// Power-of-two scales are what gfx950's FP8 conversions and scaled MFMAs
// apply in hardware, so the attention kernels never multiply by them.
//
// One wave per row.  Lane l holds elements 64g + l of the nine groups, so a
// group's amax is one wave reduction and its 64 codes one coalesced 64-byte
// store.  The E4M3 rounding is done with integer operations on the fp32 bits
// (exact, independent of any hardware conversion mode).
#include <hip/hip_runtime.h>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

using dsa::u32x4;

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;
constexpr int kGroups = DSA_D_QK / 64;         // 9
constexpr int kFp8Stride = 640;
constexpr int kBf16Stride = 2 * DSA_D_QK;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return dsa::rows4_max(v);
}

template <int KV>
__global__ __launch_bounds__(kThreads) void append_kernel(
    uint8_t* __restrict__ latent, uint8_t* __restrict__ key_plane, int num_pages,
    const int32_t* __restrict__ page_table, int pt_stride, int num_reqs,
    const int32_t* __restrict__ req, const int32_t* __restrict__ pos, int n,
    const uint16_t* __restrict__ src, const uint16_t* __restrict__ ksrc) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= n) return;
  const int b = req[i], p = pos[i];
  if (b < 0 || b >= num_reqs || p < 0 || (p >> 6) >= pt_stride) return;
  const int page = page_table[int64_t(b) * pt_stride + (p >> 6)];
  if (page < 0 || page >= num_pages) return;
  const int64_t phys = int64_t(page) * DSA_PAGE_TOKENS + (p & (DSA_PAGE_TOKENS - 1));
  const uint16_t* x = src + int64_t(i) * DSA_D_QK;

  if constexpr (KV == DSA_KV_FP8_E4M3_S64) {
    uint8_t* row = latent + phys * kFp8Stride;
    float v[kGroups], scale[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) v[g] = dsa::bf16_bits_to_f32(x[64 * g + lane]);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const float amax = wave_max(fabsf(v[g]));
      scale[g] = dsa::fp8_group_scale(amax);
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) row[64 * g + lane] = uint8_t(dsa::e4m3_encode(v[g] / scale[g]));
    // scales at byte 576 (lanes 0..8), zero padding up to byte 640 (lanes 9..15)
    float sv = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) sv = lane == g ? scale[g] : sv;
    if (lane < 16) reinterpret_cast<float*>(row + DSA_D_QK)[lane] = sv;
  } else {
    u32x4* row = reinterpret_cast<u32x4*>(latent + phys * kBf16Stride);
    const u32x4* s16 = reinterpret_cast<const u32x4*>(x);
    row[lane] = s16[lane];
    if (lane < kBf16Stride / 16 - 64) row[64 + lane] = s16[64 + lane];
  }
  if (ksrc && lane < 16) {
    reinterpret_cast<u32x4*>(key_plane + phys * (2 * DSA_IDX_DIM))[lane] =
        reinterpret_cast<const u32x4*>(ksrc + int64_t(i) * DSA_IDX_DIM)[lane];
  }
}

// Q8 query quantizer [LMSYS page, section 4 "Prefill dataflow optimization":
// the prefill attention takes an FP8 query against the FP8 cache; the
// quantizer is not spelled out].  One fp32 scale per (token, head) over its
// 576 elements, scale = amax / 448 (1 for an all-zero head), codes by the
// cache's rule.  One wave per (token, head), lane l holding elements 64g + l,
// so the amax is one wave reduction and each group's codes one 64-byte store.
__global__ __launch_bounds__(kThreads) void quantize_q8_kernel(const uint16_t* __restrict__ q,
                                                              int64_t rows,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (i >= rows) return;
  const uint16_t* x = q + i * DSA_D_QK;
  float v[kGroups];
  float amax = 0.f;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    v[g] = dsa::bf16_bits_to_f32(x[64 * g + lane]);
    amax = fmaxf(amax, fabsf(v[g]));
  }
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  uint8_t* row = codes + i * DSA_D_QK;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) row[64 * g + lane] = uint8_t(dsa::e4m3_encode(v[g] / scale));
  if (lane == 0) scales[i] = scale;
}

}  // namespace

extern "C" dsa_status dsa_quantize_q8(const uint16_t* q, int32_t num_tokens, uint8_t* q_codes,
                                      float* q_scales, void* stream) {
  const dsa_status s = dsa::check_quantize_q8(q, num_tokens, q_codes, q_scales);
  if (s != DSA_OK || num_tokens == 0) return s == DSA_OK ? dsa::ok() : s;
  const int64_t rows = int64_t(num_tokens) * DSA_HEADS;
  hipLaunchKernelGGL(quantize_q8_kernel, dim3(unsigned((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kThreads), 0, static_cast<hipStream_t>(stream), q, rows, q_codes, q_scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_quantize_q8: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}

extern "C" dsa_status dsa_kv_append(const dsa_pool* pool, const int32_t* page_table,
                                    int32_t pt_stride, int32_t num_reqs, const int32_t* req,
                                    const int32_t* pos, int32_t n, const uint16_t* latent,
                                    const uint16_t* keys, void* stream) {
  const dsa_status s =
      dsa::check_kv_append(pool, page_table, pt_stride, num_reqs, req, pos, n, latent, keys);
  if (s != DSA_OK || n == 0) return s == DSA_OK ? dsa::ok() : s;
  uint8_t* lat = reinterpret_cast<uint8_t*>(pool->base + pool->layout.latent_plane_offset);
  uint8_t* kp = reinterpret_cast<uint8_t*>(pool->base + pool->layout.index_plane_offset);
  const dim3 grid{unsigned((n + kRowsPerBlock - 1) / kRowsPerBlock)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pool->kv_dtype == DSA_KV_FP8_E4M3_S64)
    hipLaunchKernelGGL(append_kernel<DSA_KV_FP8_E4M3_S64>, grid, dim3(kThreads), 0, st, lat, kp,
                       pool->num_pages, page_table, pt_stride, num_reqs, req, pos, n, latent, keys);
  else
    hipLaunchKernelGGL(append_kernel<DSA_KV_BF16>, grid, dim3(kThreads), 0, st, lat, kp,
                       pool->num_pages, page_table, pt_stride, num_reqs, req, pos, n, latent, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_kv_append: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
