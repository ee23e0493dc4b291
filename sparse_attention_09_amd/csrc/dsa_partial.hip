// DSA Partial (sparse MLA over selected rows, split-KV) and Combine on gfx950.
//
// "Accelerating GLM-5.3-Flash on H200", section 3, "Larger KV tiles for DSA
// Partial": Partial loads the KV rows the indexer selected, computes Q K^T, an
// online softmax and the weighted value sum; KV splits write intermediates that
// Combine merges; the loop over the index tensor runs in KV tiles, the last one
// virtually padded (Figure 4).  "A million-token context on 16 H200s":
// MLA's latent row is shared by all 64 heads, so one row read from HBM serves
// 64 heads - which makes QK^T and PV dense enough for the matrix cores.
//
// One workgroup = one (token, split), 4 waves, wave w owns heads 16w..16w+15.
// Per KV tile of TILE rows:
//   * the selected rows are gathered through the page table with coalesced
//     loads (each wave instruction reads 512 contiguous bytes of one row), FP8
//     codes are dequantized in registers (exact E4M3->fp32, times the row's
//     per-64 scale, rounded to bf16) and written to LDS twice: row-major K
//     (576 wide, QK^T operand) and transposed V (512 x TILE, PV operand);
//   * the next tile's rows are prefetched into registers while the current
//     tile is computed;
//   * S^T = K Q^T and O += P V run on the 16x16x32 bf16 MFMA with fp32
//     accumulation; Q stays in registers for the whole split, the softmax
//     state (running max and sum, log2 domain) in registers per head, and
//     P goes from the S^T accumulators to the PV operand without leaving
//     registers.
#include <hip/hip_runtime.h>

#include <cmath>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

using dsa::bf16x8;
using dsa::f32x4;
using dsa::u32x2;
using dsa::u32x4;

constexpr int kThreads = 256;
constexpr int kKStride = DSA_D_QK + 8;   // LDS row stride of K in bf16 (pad against bank conflicts)
constexpr int kRowChunk = 2048;          // index columns whose row addresses are resolved at once
constexpr float kNegInf = -INFINITY;

struct PartialArgs {
  const uint8_t* latent;
  int num_pages;
  const int32_t* page_table;
  int pt_stride;
  const int32_t* q_offsets;
  int num_reqs;
  const int32_t* tok_pos;
  const uint16_t* q;
  const int32_t* idx;
  int width;
  float scale_log2;      // sm_scale * log2(e)
  int cols_per_split;
  int splits;
  float* o_part;
  float* lse_part;
};

template <int TILE>
struct TileSmem {
  uint16_t k[TILE * kKStride];
  uint16_t vt[DSA_D_LATENT * TILE];
  int32_t rows[kRowChunk];
};

// XOR swizzle of the 8-row chunks inside one transposed-V row (column d), so
// that both the transposed writes (consecutive lanes -> d, d+8, ...) and the
// MFMA operand reads (consecutive lanes -> d, d+1, ...) spread over the banks.
template <int TILE>
__device__ __forceinline__ int vt_swizzle(int d) {
  return (d ^ (d >> 3)) & (TILE / 8 - 1);
}

// Register staging of one tile's rows for one thread.
template <int KV, int TILE>
struct Stage;

// FP8 rows: 576 codes, 9 fp32 scales at byte 576, stride 640.
template <int TILE>
struct Stage<DSA_KV_FP8_E4M3_S64, TILE> {
  static constexpr int kStride = 640;
  static constexpr int kVU = TILE / 32;                 // V units (8 rows x 8 cols) per thread
  static constexpr int kRU = (TILE * 4 + kThreads - 1) / kThreads;  // rope units (1 row x 16 cols)
  u32x2 vcode[kVU][8];
  float vscale[kVU][8];
  u32x4 rcode[kRU];
  float rscale[kRU];

  __device__ __forceinline__ void load(const uint8_t* latent, const int32_t* rows, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < kVU; ++i) {
      const int rg = wave + 4 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int phys = rows[8 * rg + e];
        if (phys >= 0) {
          const uint8_t* row = latent + int64_t(phys) * kStride;
          vcode[i][e] = *reinterpret_cast<const u32x2*>(row + 8 * lane);
          vscale[i][e] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * (lane >> 3));
        } else {
          vcode[i][e] = u32x2{0, 0};
          vscale[i][e] = 0.f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kRU; ++i) {
      const int u = tid + kThreads * i;
      rcode[i] = u32x4{0, 0, 0, 0};
      rscale[i] = 0.f;
      if (u < TILE * 4) {
        const int phys = rows[u >> 2];
        if (phys >= 0) {
          const uint8_t* row = latent + int64_t(phys) * kStride;
          rcode[i] = *reinterpret_cast<const u32x4*>(row + DSA_D_LATENT + 16 * (u & 3));
          rscale[i] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * 8);
        }
      }
    }
  }

  // bf16 pairs of the 8 rows of V unit i: bits[e][m] holds cols 2m, 2m+1 of row e
  __device__ __forceinline__ void vbits(int i, uint32_t bits[8][4]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f[8];
      dsa::fp8x4_to_f32(vcode[i][e][0], f);
      dsa::fp8x4_to_f32(vcode[i][e][1], f + 4);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        bits[e][m] = dsa::pack_bf16x2(f[2 * m] * vscale[i][e], f[2 * m + 1] * vscale[i][e]);
    }
  }
  __device__ __forceinline__ void rbits(int i, uint32_t bits[8]) const {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float f[4];
      dsa::fp8x4_to_f32(rcode[i][h], f);
      bits[2 * h] = dsa::pack_bf16x2(f[0] * rscale[i], f[1] * rscale[i]);
      bits[2 * h + 1] = dsa::pack_bf16x2(f[2] * rscale[i], f[3] * rscale[i]);
    }
  }
};

// BF16 rows: 576 bf16, stride 1152.
template <int TILE>
struct Stage<DSA_KV_BF16, TILE> {
  static constexpr int kStride = 2 * DSA_D_QK;
  static constexpr int kVU = TILE / 32;
  static constexpr int kRU = (TILE * 4 + kThreads - 1) / kThreads;
  u32x4 vraw[kVU][8];
  u32x4 rraw[kRU][2];

  __device__ __forceinline__ void load(const uint8_t* latent, const int32_t* rows, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < kVU; ++i) {
      const int rg = wave + 4 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int phys = rows[8 * rg + e];
        vraw[i][e] = phys >= 0
            ? *reinterpret_cast<const u32x4*>(latent + int64_t(phys) * kStride + 16 * lane)
            : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < kRU; ++i) {
      const int u = tid + kThreads * i;
      rraw[i][0] = rraw[i][1] = u32x4{0, 0, 0, 0};
      if (u < TILE * 4) {
        const int phys = rows[u >> 2];
        if (phys >= 0) {
          const u32x4* src = reinterpret_cast<const u32x4*>(latent + int64_t(phys) * kStride +
                                                            2 * DSA_D_LATENT + 32 * (u & 3));
          rraw[i][0] = src[0];
          rraw[i][1] = src[1];
        }
      }
    }
  }
  __device__ __forceinline__ void vbits(int i, uint32_t bits[8][4]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int m = 0; m < 4; ++m) bits[e][m] = vraw[i][e][m];
  }
  __device__ __forceinline__ void rbits(int i, uint32_t bits[8]) const {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      bits[m] = rraw[i][0][m];
      bits[4 + m] = rraw[i][1][m];
    }
  }
};

template <int KV, int TILE>
__device__ __forceinline__ void stage_store(const Stage<KV, TILE>& st, TileSmem<TILE>& sm, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < Stage<KV, TILE>::kVU; ++i) {
    const int rg = wave + 4 * i;
    uint32_t bits[8][4];
    st.vbits(i, bits);
    // row-major K: row 8rg+e, cols 8*lane .. +8
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<u32x4*>(&sm.k[(8 * rg + e) * kKStride + 8 * lane]) =
          u32x4{bits[e][0], bits[e][1], bits[e][2], bits[e][3]};
    // transposed V: column d = 8*lane + dd, rows 8rg .. +8
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int m = dd >> 1;
      const bool hi = dd & 1;
      uint32_t v[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t a = bits[2 * pr][m], b = bits[2 * pr + 1][m];
        v[pr] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      const int d = 8 * lane + dd;
      *reinterpret_cast<u32x4*>(&sm.vt[d * TILE + 8 * (rg ^ vt_swizzle<TILE>(d))]) =
          u32x4{v[0], v[1], v[2], v[3]};
    }
  }
#pragma unroll
  for (int i = 0; i < Stage<KV, TILE>::kRU; ++i) {
    const int u = tid + kThreads * i;
    if (u < TILE * 4) {
      uint32_t bits[8];
      st.rbits(i, bits);
      uint16_t* dst = &sm.k[(u >> 2) * kKStride + DSA_D_LATENT + 16 * (u & 3)];
      *reinterpret_cast<u32x4*>(dst) = u32x4{bits[0], bits[1], bits[2], bits[3]};
      *reinterpret_cast<u32x4*>(dst + 8) = u32x4{bits[4], bits[5], bits[6], bits[7]};
    }
  }
}

template <int KV, int TILE>
__global__ __launch_bounds__(kThreads) void partial_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) TileSmem<TILE> sm;
  constexpr int kMB = TILE / 16;   // 16-row MFMA blocks per tile
  constexpr int kKS = TILE / 32;   // PV k-steps per tile

  const int t = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int c0 = s * a.cols_per_split;
  const int c1 = min(a.width, c0 + a.cols_per_split);

  int lo = 0, hi = a.num_reqs - 1;   // request of token t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.q_offsets[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int req = lo;
  const int pos = a.tok_pos[t];

  // Q of head 16*wave + c, dims 32ks + 8g .. +8 (MFMA B operand)
  u32x4 qf[DSA_D_QK / 32];
  {
    const u32x4* qsrc =
        reinterpret_cast<const u32x4*>(a.q + (int64_t(t) * DSA_HEADS + 16 * wave + c) * DSA_D_QK);
#pragma unroll
    for (int ks = 0; ks < DSA_D_QK / 32; ++ks) qf[ks] = qsrc[ks * 4 + g];
  }
  f32x4 o[DSA_D_LATENT / 16];
#pragma unroll
  for (int nb = 0; nb < DSA_D_LATENT / 16; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  Stage<KV, TILE> st;
  for (int cc = c0; cc < c1; cc += kRowChunk) {
    const int cend = min(c1, cc + kRowChunk);
    __syncthreads();
    for (int i = tid; i < kRowChunk; i += kThreads) {
      const int col = cc + i;
      int phys = -1;
      if (col < cend) {
        const int p = a.idx[int64_t(t) * a.width + col];
        if (p >= 0 && p <= pos) {
          const int j = p >> 6;
          if (j < a.pt_stride) {
            int pg = a.page_table[int64_t(req) * a.pt_stride + j];
            pg = min(max(pg, 0), a.num_pages - 1);
            phys = pg * DSA_PAGE_TOKENS + (p & 63);
          }
        }
      }
      sm.rows[i] = phys;
    }
    __syncthreads();
    const int ntile = (cend - cc + TILE - 1) / TILE;
    st.load(a.latent, sm.rows, tid);
    stage_store<KV, TILE>(st, sm, tid);
    __syncthreads();
    for (int it = 0; it < ntile; ++it) {
      const bool more = it + 1 < ntile;
      if (more) st.load(a.latent, sm.rows + (it + 1) * TILE, tid);

      // ---- S^T = K Q^T for this wave's 16 heads
      f32x4 sacc[kMB];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* krow = &sm.k[(16 * mb + c) * kKStride + 8 * g];
#pragma unroll
        for (int ks = 0; ks < DSA_D_QK / 32; ++ks) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 32 * ks);
          sacc[mb] = dsa::mfma16x16x32(dsa::as_bf16x8(kf), dsa::as_bf16x8(qf[ks]), sacc[mb]);
        }
      }

      // ---- online softmax (log2 domain); lane holds rows 16mb+4g+j of head c
      const int32_t* rows = sm.rows + it * TILE;
      float z[kMB][4];
      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool valid = rows[16 * mb + 4 * g + j] >= 0;
          z[mb][j] = valid ? sacc[mb][j] * a.scale_log2 : kNegInf;
          tmax = fmaxf(tmax, z[mb][j]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const bool none = (m_new == kNegInf);
      const float alpha = none ? 1.f : exp2f(m_run - m_new);
      float psum = 0.f;
      float p[kMB][4];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[mb][j] = none ? 0.f : exp2f(z[mb][j] - m_new);
          psum += p[mb][j];
        }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      float aj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) aj[j] = __shfl(alpha, 4 * g + j);
#pragma unroll
      for (int nb = 0; nb < DSA_D_LATENT / 16; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[nb][j] *= aj[j];

      // ---- O += P V : P straight from the S^T accumulators
      u32x4 pa[kKS];
#pragma unroll
      for (int k2 = 0; k2 < kKS; ++k2)
        pa[k2] = u32x4{dsa::pack_bf16x2(p[2 * k2][0], p[2 * k2][1]),
                       dsa::pack_bf16x2(p[2 * k2][2], p[2 * k2][3]),
                       dsa::pack_bf16x2(p[2 * k2 + 1][0], p[2 * k2 + 1][1]),
                       dsa::pack_bf16x2(p[2 * k2 + 1][2], p[2 * k2 + 1][3])};
#pragma unroll
      for (int nb = 0; nb < DSA_D_LATENT / 16; ++nb) {
        const int d = 16 * nb + c;
        const int sw = vt_swizzle<TILE>(d);
        const uint16_t* vrow = &sm.vt[d * TILE + 4 * (g & 1)];
#pragma unroll
        for (int k2 = 0; k2 < kKS; ++k2) {
          const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vrow + 8 * ((4 * k2 + (g >> 1)) ^ sw));
          const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vrow + 8 * ((4 * k2 + 2 + (g >> 1)) ^ sw));
          const u32x4 vb = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          o[nb] = dsa::mfma16x16x32(dsa::as_bf16x8(pa[k2]), dsa::as_bf16x8(vb), o[nb]);
        }
      }
      __syncthreads();
      if (more) {
        stage_store<KV, TILE>(st, sm, tid);
        __syncthreads();
      }
    }
  }

  // ---- normalize and write this split's partial
  const int64_t ts = int64_t(t) * a.splits + s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lj = __shfl(l_run, 4 * g + j);
    const float inv = lj > 0.f ? 1.f / lj : 0.f;
    float* dst = a.o_part + (ts * DSA_HEADS + 16 * wave + 4 * g + j) * DSA_D_LATENT + c;
#pragma unroll
    for (int nb = 0; nb < DSA_D_LATENT / 16; ++nb) dst[16 * nb] = o[nb][j] * inv;
  }
  if (g == 0)
    a.lse_part[ts * DSA_HEADS + 16 * wave + c] =
        l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994530942f : kNegInf;
}

template <int KV, int TILE>
hipError_t launch_partial(const PartialArgs& a, int T, int S, hipStream_t st) {
  hipLaunchKernelGGL((partial_kernel<KV, TILE>), dim3(T, S), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one thread per (token, head, 8 columns).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int T,
                                                      int S, uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // token*64 + head
  if (row >= T * DSA_HEADS) return;
  const int lane = threadIdx.x & 63;
  const int t = row / DSA_HEADS, h = row % DSA_HEADS;
  float m = kNegInf;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse_part[(int64_t(t) * S + s) * DSA_HEADS + h]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const float ls = lse_part[(int64_t(t) * S + s) * DSA_HEADS + h];
      if (ls == kNegInf) continue;
      const float wgt = expf(ls - m);
      tot += wgt;
      const float4* src = reinterpret_cast<const float4*>(
          o_part + ((int64_t(t) * S + s) * DSA_HEADS + h) * DSA_D_LATENT + 8 * lane);
      const float4 x0 = src[0], x1 = src[1];
      acc[0] += wgt * x0.x; acc[1] += wgt * x0.y; acc[2] += wgt * x0.z; acc[3] += wgt * x0.w;
      acc[4] += wgt * x1.x; acc[5] += wgt * x1.y; acc[6] += wgt * x1.z; acc[7] += wgt * x1.w;
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  u32x4 packed;
#pragma unroll
  for (int i = 0; i < 4; ++i) packed[i] = dsa::pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *reinterpret_cast<u32x4*>(out + int64_t(row) * DSA_D_LATENT + 8 * lane) = packed;
  if (lane == 0) lse_out[row] = tot > 0.f ? m + logf(tot) : kNegInf;
}

}  // namespace

extern "C" dsa_status dsa_sparse_mla_partial(const dsa_pool* pool, const int32_t* page_table,
                                             int32_t pt_stride, const int32_t* q_offsets,
                                             int32_t num_reqs, const int32_t* tok_pos,
                                             int32_t num_tokens, const uint16_t* q,
                                             const int32_t* idx, int32_t width, float sm_scale,
                                             int32_t kv_tile, int32_t num_splits, float* o_part,
                                             float* lse_part, void* stream) {
  dsa_status s = dsa::check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos,
                                  num_tokens, "dsa_sparse_mla_partial");
  if (s != DSA_OK) return s;
  if (width < 1) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: width must be >= 1");
  if (kv_tile != 32 && kv_tile != 64 && kv_tile != 128)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: kv_tile must be 32, 64 or 128");
  if (num_splits < 1 || num_splits > 65535)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: num_splits must be in [1, 65535]");
  if (!std::isfinite(sm_scale))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: sm_scale must be finite");
  if (num_tokens == 0) return dsa::ok();
  if (!q || !idx || !o_part || !lse_part)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: q, idx, o_part, lse_part must be non-null");
  if (!dsa::aligned(q, 16) || !dsa::aligned(idx, 4) || !dsa::aligned(o_part, 16) ||
      !dsa::aligned(lse_part, 4))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_sparse_mla_partial: q and o_part must be 16-byte aligned");
  if (kv_tile == 128)
    return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_sparse_mla_partial: kv_tile 128 is not built yet");
  dsa_partial_plan plan;
  if (dsa_plan_partial(num_tokens, width, kv_tile, num_splits, 0, &plan) != DSA_OK)
    return DSA_ERR_INVALID_ARG;
  PartialArgs a;
  a.latent = reinterpret_cast<const uint8_t*>(pool->base + pool->layout.latent_plane_offset);
  a.num_pages = pool->num_pages;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.q_offsets = q_offsets;
  a.num_reqs = num_reqs;
  a.tok_pos = tok_pos;
  a.q = q;
  a.idx = idx;
  a.width = width;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.cols_per_split = plan.cols_per_split;
  a.splits = num_splits;
  a.o_part = o_part;
  a.lse_part = lse_part;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool fp8 = pool->kv_dtype == DSA_KV_FP8_E4M3_S64;
  if (kv_tile == 32)
    e = fp8 ? launch_partial<DSA_KV_FP8_E4M3_S64, 32>(a, num_tokens, num_splits, st)
            : launch_partial<DSA_KV_BF16, 32>(a, num_tokens, num_splits, st);
  else
    e = fp8 ? launch_partial<DSA_KV_FP8_E4M3_S64, 64>(a, num_tokens, num_splits, st)
            : launch_partial<DSA_KV_BF16, 64>(a, num_tokens, num_splits, st);
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_sparse_mla_partial: launch failed: ") +
                                      hipGetErrorString(e));
  return dsa::ok();
}

extern "C" dsa_status dsa_combine(const float* o_part, const float* lse_part, int32_t num_tokens,
                                  int32_t num_splits, uint16_t* out, float* lse, void* stream) {
  if (num_tokens < 0) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_combine: num_tokens < 0");
  if (num_splits < 1) return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_combine: num_splits must be >= 1");
  if (num_tokens == 0) return dsa::ok();
  if (!o_part || !lse_part || !out || !lse)
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_combine: pointers must be non-null");
  if (!dsa::aligned(o_part, 16) || !dsa::aligned(out, 16) || !dsa::aligned(lse_part, 4) ||
      !dsa::aligned(lse, 4))
    return dsa::fail(DSA_ERR_INVALID_ARG, "dsa_combine: o_part and out must be 16-byte aligned");
  const int64_t rows = int64_t(num_tokens) * DSA_HEADS;
  if ((rows + 3) / 4 > 0x7fffffff)
    return dsa::fail(DSA_ERR_UNSUPPORTED, "dsa_combine: too many tokens for one launch");
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), o_part, lse_part, num_tokens, num_splits,
                     out, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string("dsa_combine: launch failed: ") + hipGetErrorString(e));
  return dsa::ok();
}
