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
// One workgroup = one (token, split).  Per KV tile of TILE rows:
//   * the selected rows are gathered through the page table in 16-byte chunks,
//     the lanes of a wave instruction covering whole 128-byte lines; FP8 codes
//     are dequantized in registers (the scaled FP8 -> bf16 conversion, exact
//     for the cache's power-of-two group scales) and written once to LDS as a
//     row-major K tile (576 wide, swizzled against bank conflicts);
//   * the next tile's rows are prefetched into registers while the current
//     tile is computed (gather loads are unconditional so nothing waits on them
//     before the tile's stores);
//   * S^T = K Q^T runs on the 16x16x32 bf16 MFMA with Q held in registers for
//     the whole split; O += P V reads V = K[:, :512] from the same LDS tile with
//     the gfx950 transpose read (ds_read_b64_tr_b16), so no transposed copy is
//     made.
// Kernels:
//   * tiles of 32 and 128 index columns (partial_ws_kernel): 12 waves (8 for
//     BF16 rows) in a score role and a value role one 32-row tile apart, a
//     running reference max that rescales O only when it grows by more than
//     2^8 (described at the kernel); a 128-column tile is four of its 32-row
//     LDS steps;
//   * tiles of 64 (partial_v2_kernel, split batches): 8 waves, 2 per SIMD,
//     each owning 32 heads, with a softmax whose per-head reference is fixed
//     once (described at the kernel);
//   * the Q8 variant (partial_q8_kernel): FP8 query codes against the raw FP8
//     rows on the scaled f8f6f4 MFMA.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <utility>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace {

using dsa::bf16x8;
using dsa::f32x4;
using dsa::u32x2;
using dsa::u32x4;

constexpr int kKStride = DSA_D_QK + 16;  // LDS row stride of the K tile in bf16 (296 dwords)
constexpr int kRowChunk = 2048;          // index columns whose row addresses are resolved at once
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleThreshold = 8.f; // log2 units
constexpr float kLn2 = 0.69314718055994530942f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// K-tile layout.  Rows at a 296-dword stride; logical 16-byte chunk x of a
// row sits at physical chunk k_phys(x) = x ^ bit3(x) (chunks 8..15 of every
// 16 swap with their neighbour).  Bank behaviour of gfx950's LDS, measured
// with conflict counters over single access patterns: 16-byte reads are
// served 32 lanes at a time over 512 bytes of banks (lanes 0..15 with
// 48..63, then 16..47), 16-byte writes 8 lanes at a time over 128 bytes,
// 8-byte transpose reads 32 lanes at a time over 256 bytes.  With this
// stride and chunk map
//   * MFMA operand reads (16 consecutive rows, one chunk each; the lane
//     groups read chunks of opposite parity),
//   * transpose reads (4 rows x 32 bytes per 16 lanes),
//   * staging writes (8 lanes writing the even chunks 2l of one row: the
//     bit-3 swap moves half of them to odd chunks)
// all hit distinct banks.  The map depends only on the chunk index, so every
// lane-dependent choice is an address, computed once per lane.
__device__ __forceinline__ constexpr int k_phys(int x) { return x ^ ((x >> 3) & 1); }
__device__ __forceinline__ int k_chunk_off(int r, int chunk) { return r * kKStride + (k_phys(chunk) << 3); }

// Transposed 4x16-bit read: lane i of each 16-lane group receives element i%4
// of the 8-byte chunks addressed by lanes 4j + i/4 of its group, j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

struct PartialArgs {
  const uint8_t* latent;
  int num_pages;
  const int32_t* page_table;
  int pt_stride;
  const int32_t* q_offsets;
  int num_reqs;
  const int32_t* tok_pos;
  const uint16_t* q;
  const uint8_t* q8;     // Q8 path: E4M3 query codes [T,64,576]
  const float* q8_scale; // and one scale per (token, head)
  const int32_t* idx;
  int width;
  float scale_log2;      // sm_scale * log2(e)
  int cols_per_split;
  int splits;
  float* o_part;
  float* lse_part;
  uint16_t* out;         // single-split form: final bf16 output [T,64,512]
  float* lse_out;        // and its lse [T,64]
};

// Output of one (token, split, head, column) value.  With kFinal (one split,
// no Combine) the normalized value is written in bf16 to the final output;
// that is bit for bit what Combine makes of a single split (weight exp(0) = 1).
template <bool kFinal>
__device__ __forceinline__ void put_out(const PartialArgs& a, int64_t ts, int head, int col, float v) {
  if constexpr (kFinal)
    a.out[(ts * DSA_HEADS + head) * DSA_D_LATENT + col] = __builtin_bit_cast(uint16_t, (__bf16)v);
  else
    a.o_part[(ts * DSA_HEADS + head) * DSA_D_LATENT + col] = v;
}
template <bool kFinal>
__device__ __forceinline__ void put_lse(const PartialArgs& a, int64_t ts, int head, float v) {
  if constexpr (kFinal)
    a.lse_out[ts * DSA_HEADS + head] = v;
  else
    a.lse_part[ts * DSA_HEADS + head] = v;
}

// Register staging of NR rows of a tile, spread over NT threads.  Chunk q of
// the tile (16 bytes of a row) goes to thread q % NT, so the lanes of one
// wave instruction read whole 128-byte lines of one or two rows.
template <int KV, int NR, int NT>
struct Stage;

// 4 E4M3 codes times their group scale -> 4 bf16 (two dwords) with gfx950's
// scaled conversion, two values per instruction.  It applies the exponent of
// the fp32 scale (a block scale); the cache's group scales are powers of two,
// so the result is the exact product (4 significant bits fit bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 dq4_bf16(uint32_t codes, float scale) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// FP8 rows: 576 codes, 9 fp32 scales at byte 576, stride 640.  Latent chunk
// q (16 codes) is row q/32, columns 16(q%32)..+16, with the scale of group
// (q%32)/4.  The rope (64 codes per row) is cut into NT equal pieces of
// kRP = NR*64/NT bytes when that is 4 or 8 (tiles of 32 and 64 rows over 512
// threads), so every thread stages the same number of latent chunks and one
// rope piece and the staging has no per-thread branch; otherwise rope chunk q
// (16 codes) is row q/4, rope columns 16(q%4)..+16.
template <int NR, int NT>
struct Stage<DSA_KV_FP8_E4M3_S64, NR, NT> {
  static constexpr int kStride = 640;
  static constexpr int kLC = (NR * 32 + NT - 1) / NT;
  static constexpr bool kLExact = kLC * NT == NR * 32;
  static constexpr int kRP = (NR * 64) % NT == 0 ? NR * 64 / NT : 0;
  static constexpr bool kRPiece = kRP == 4 || kRP == 8;
  static constexpr int kRC = kRPiece ? 1 : (NR * 4 + NT - 1) / NT;
  using RopeT = std::conditional_t<kRP == 4, uint32_t, std::conditional_t<kRP == 8, u32x2, u32x4>>;
  u32x4 lcode[kLC];
  float lscale[kLC];
  RopeT rcode[kRC];
  float rscale[kRC];
  uint32_t lok, rok;   // bit i: chunk i holds a valid row

  // Latent chunk i of this thread (row (tid + NT*i)/32) into registers.
  __device__ __forceinline__ void load_latent(const uint8_t* latent, const int32_t* rows, int tid, int i) {
    const int q = tid + NT * i;
    const int phys = (kLExact || q < NR * 32) ? rows[q >> 5] : -1;
    lok = (lok & ~(1u << i)) | (uint32_t(phys >= 0) << i);
    const uint8_t* row = latent + int64_t(max(phys, 0)) * kStride;
    lcode[i] = *reinterpret_cast<const u32x4*>(row + 16 * (q & 31));
    lscale[i] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * ((q & 31) >> 2));
  }
  // This thread's rope piece (piece layout only).
  __device__ __forceinline__ void load_rope_piece(const uint8_t* latent, const int32_t* rows, int tid) {
    constexpr int kPerRow = 64 / kRP;
    const int phys = rows[tid / kPerRow];
    rok = uint32_t(phys >= 0);
    const uint8_t* row = latent + int64_t(max(phys, 0)) * kStride;
    rcode[0] = *reinterpret_cast<const RopeT*>(row + DSA_D_LATENT + kRP * (tid % kPerRow));
    rscale[0] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * 8);
  }

  // Unconditional loads: invalid rows read row 0 and are zeroed when stored.
  __device__ __forceinline__ void load(const uint8_t* latent, const int32_t* rows, int tid) {
#pragma unroll
    for (int i = 0; i < kLC; ++i) load_latent(latent, rows, tid, i);
    if constexpr (kRPiece) {
      load_rope_piece(latent, rows, tid);
    } else {
      rok = 0;
#pragma unroll
      for (int i = 0; i < kRC; ++i) {
        const int q = tid + NT * i;
        const int phys = q < NR * 4 ? rows[q >> 2] : -1;
        rok |= uint32_t(phys >= 0) << i;
        const uint8_t* row = latent + int64_t(max(phys, 0)) * kStride;
        rcode[i] = *reinterpret_cast<const u32x4*>(row + DSA_D_LATENT + 16 * (q & 3));
        rscale[i] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * 8);
      }
    }
  }

  __device__ __forceinline__ static u32x2 dq4(uint32_t codes, float scale) { return dq4_bf16(codes, scale); }

  // 16 codes -> 16 bf16 = logical chunks `chunk` (even) and `chunk`+1 of
  // row r (physically k_phys(chunk) and k_phys(chunk) ^ 1)
  __device__ __forceinline__ static void put16(uint16_t* k, int r, int chunk, const u32x4& codes,
                                               float scale) {
    const int c0 = k_phys(chunk);
    uint16_t* row = k + r * kKStride;
    const u32x2 a0 = dq4(codes[0], scale), a1 = dq4(codes[1], scale);
    *reinterpret_cast<u32x4*>(row + 8 * c0) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    const u32x2 b0 = dq4(codes[2], scale), b1 = dq4(codes[3], scale);
    *reinterpret_cast<u32x4*>(row + 8 * (c0 ^ 1)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
  }

  // piece p of row r: rope codes kRP*p..; bf16 chunk 64 + kRP*p/8, and
  // within it 4*(p&1) values for 4-byte pieces
  __device__ __forceinline__ void store_rope_piece(uint16_t* k, int r0, int tid) const {
    constexpr int kPerRow = 64 / kRP;
    const int r = r0 + tid / kPerRow, p = tid % kPerRow;
    const bool ok = rok & 1u;
    const float sc = ok ? rscale[0] : 0.f;
    if constexpr (kRP == 4) {
      const u32x2 v = dq4(ok ? rcode[0] : 0u, sc);
      *reinterpret_cast<u32x2*>(k + k_chunk_off(r, DSA_D_LATENT / 8 + (p >> 1)) + 4 * (p & 1)) = v;
    } else {
      const u32x2 lo = dq4(ok ? rcode[0][0] : 0u, sc), hi = dq4(ok ? rcode[0][1] : 0u, sc);
      *reinterpret_cast<u32x4*>(k + k_chunk_off(r, DSA_D_LATENT / 8 + p)) =
          u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }

  // rows are stored at r0 + (tile row)
  __device__ __forceinline__ void store(uint16_t* k, int r0, int tid) const {
    const u32x4 z = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kLC; ++i) {
      const int q = tid + NT * i;
      const bool ok = (lok >> i) & 1u;
      if (kLExact || q < NR * 32)
        put16(k, r0 + (q >> 5), 2 * (q & 31), ok ? lcode[i] : z, ok ? lscale[i] : 0.f);
    }
    if constexpr (kRPiece) {
      store_rope_piece(k, r0, tid);
    } else {
#pragma unroll
      for (int i = 0; i < kRC; ++i) {
        const int q = tid + NT * i;
        const bool ok = (rok >> i) & 1u;
        if (q < NR * 4)
          put16(k, r0 + (q >> 2), DSA_D_LATENT / 8 + 2 * (q & 3), ok ? rcode[i] : z,
                ok ? rscale[i] : 0.f);
      }
    }
  }
};

// BF16 rows: 576 bf16, stride 1152.  Latent chunk q (8 values) is row q/64,
// columns 8(q%64)..+8; rope chunk q is row q/8, rope columns 8(q%8)..+8.
template <int NR, int NT>
struct Stage<DSA_KV_BF16, NR, NT> {
  static constexpr int kStride = 2 * DSA_D_QK;
  static constexpr int kLC = (NR * 64 + NT - 1) / NT;
  static constexpr int kRC = (NR * 8 + NT - 1) / NT;
  u32x4 lraw[kLC];
  u32x4 rraw[kRC];
  uint32_t lok, rok;

  __device__ __forceinline__ void load(const uint8_t* latent, const int32_t* rows, int tid) {
    lok = rok = 0;
#pragma unroll
    for (int i = 0; i < kLC; ++i) {
      const int q = tid + NT * i;
      const int phys = q < NR * 64 ? rows[q >> 6] : -1;
      lok |= uint32_t(phys >= 0) << i;
      lraw[i] = *reinterpret_cast<const u32x4*>(latent + int64_t(max(phys, 0)) * kStride +
                                                16 * (q & 63));
    }
#pragma unroll
    for (int i = 0; i < kRC; ++i) {
      const int q = tid + NT * i;
      const int phys = q < NR * 8 ? rows[q >> 3] : -1;
      rok |= uint32_t(phys >= 0) << i;
      rraw[i] = *reinterpret_cast<const u32x4*>(latent + int64_t(max(phys, 0)) * kStride +
                                                2 * DSA_D_LATENT + 16 * (q & 7));
    }
  }
  __device__ __forceinline__ void store(uint16_t* k, int r0, int tid) const {
    const u32x4 z = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kLC; ++i) {
      const int q = tid + NT * i;
      const bool ok = (lok >> i) & 1u;
      if (q < NR * 64) {
        const int r = r0 + (q >> 6);
        *reinterpret_cast<u32x4*>(k + k_chunk_off(r, q & 63)) = ok ? lraw[i] : z;
      }
    }
#pragma unroll
    for (int i = 0; i < kRC; ++i) {
      const int q = tid + NT * i;
      const bool ok = (rok >> i) & 1u;
      if (q < NR * 8) {
        const int r = r0 + (q >> 3);
        *reinterpret_cast<u32x4*>(k + k_chunk_off(r, DSA_D_LATENT / 8 + (q & 7))) = ok ? rraw[i] : z;
      }
    }
  }
};

// Physical rows (page*64 + slot, or -1 when masked) of index columns
// [cc, cc + N) of token t, written to rows[]; with a bias array, also
// 0 for a valid row and -inf for a masked one.  *last (reset to -1 by the
// caller) receives the largest chunk-relative column with a valid row.
// nthreads must divide N (the column count, kRowChunk by default).
// Physical rows of index columns [cc, cend) of token t (-1 where the entry is
// masked), written to rows[0..N) (and bias: 0 or -inf); *last gets the largest
// slot holding a valid row.  NT threads; each thread takes its columns in
// batches of kB, the batch's index loads in flight together, then its
// page-table loads (the plain loop, kB = 0, waits for each column's two loads
// in turn: six memory latencies at 2,048 columns over 768 threads).
template <int N, int NT, int kB = (N + NT - 1) / NT>
__device__ __forceinline__ void resolve_rows(const PartialArgs& a, int t, int req, int pos, int cc,
                                             int cend, int32_t* rows, int tid, int* last,
                                             float* bias = nullptr) {
  static_assert(N % 64 == 0 && NT % 64 == 0, "whole waves per pass");
  constexpr int kIt = (N + NT - 1) / NT;
  const int lane = tid & 63;
  if constexpr (kB == 0) {
    for (int i = tid; i < N; i += NT) {
      const int col = cc + i;
      int phys = -1;
      if (col < cend) {
        const int p = a.idx[int64_t(t) * a.width + col];
        if (p >= 0 && p <= pos && (p >> 6) < a.pt_stride) {
          const int pg = a.page_table[int64_t(req) * a.pt_stride + (p >> 6)];
          phys = min(max(pg, 0), a.num_pages - 1) * DSA_PAGE_TOKENS + (p & 63);
        }
      }
      rows[i] = phys;
      if (bias) bias[i] = phys >= 0 ? 0.f : kNegInf;
      const uint64_t m = __ballot(phys >= 0);
      if (m != 0ull && lane == 0) atomicMax(last, i + 63 - __clzll((long long)m));
    }
    return;
  }
  // loads unconditional (a column past the range reads the range's last one
  // or column 0, a masked entry page 0 of the request) and masked afterwards:
  // a conditional load compiles to a branch that waits for it, one load at a
  // time
  const int32_t* idx_row = a.idx + int64_t(t) * a.width;
  const int32_t* pt = a.page_table + int64_t(req) * a.pt_stride;
  const int col_max = max(cend - 1, 0);
#pragma unroll
  for (int u0 = 0; u0 < kIt; u0 += (kB > 0 ? kB : 1)) {
    int p[kB > 0 ? kB : 1], pg[kB > 0 ? kB : 1];
#pragma unroll
    for (int v = 0; v < kB; ++v) p[v] = idx_row[min(cc + tid + NT * (u0 + v), col_max)];
#pragma unroll
    for (int v = 0; v < kB; ++v) {
      const int i = tid + NT * (u0 + v);
      if (!(u0 + v < kIt && i < N && cc + i < cend)) p[v] = -1;
    }
#pragma unroll
    for (int v = 0; v < kB; ++v) {
      const bool ok = p[v] >= 0 && p[v] <= pos && (p[v] >> 6) < a.pt_stride;
      pg[v] = pt[ok ? (p[v] >> 6) : 0];
    }
#pragma unroll
    for (int v = 0; v < kB; ++v) {
      const bool ok = p[v] >= 0 && p[v] <= pos && (p[v] >> 6) < a.pt_stride;
      pg[v] = ok ? min(max(pg[v], 0), a.num_pages - 1) : -1;
    }
#pragma unroll
    for (int v = 0; v < kB; ++v) {
      const int i = tid + NT * (u0 + v);
      if (u0 + v < kIt && i < N) {   // wave-uniform
        const int phys = pg[v] >= 0 ? pg[v] * DSA_PAGE_TOKENS + (p[v] & 63) : -1;
        rows[i] = phys;
        if (bias) bias[i] = phys >= 0 ? 0.f : kNegInf;
        const uint64_t m = __ballot(phys >= 0);
        if (m != 0ull && lane == 0) atomicMax(last, i + 63 - __clzll((long long)m));
      }
    }
  }
}

// Request of token t: q_offsets is nondecreasing with q_offsets[0] = 0, so the
// request is (the number of requests r with q_offsets[r] <= t) - 1, counted
// by every wave with ballots over one vector load per lane and request block
// (a binary search was one dependent load per halving, ~7 latencies at 128
// requests, before anything else could start).  Whole waves, uniform flow.
__device__ __forceinline__ int request_of(const PartialArgs& a, int t) {
  constexpr int kFirst = 4;   // 256 requests in the first round trip
  const int lane = dsa::fresh_lane();
  int below = 0;
  bool more = true;
  int le[kFirst];
#pragma unroll
  for (int i = 0; i < kFirst; ++i) {
    const int r = 64 * i + lane;
    le[i] = r < a.num_reqs ? a.q_offsets[r] : 0x7fffffff;
  }
#pragma unroll
  for (int i = 0; i < kFirst; ++i) {
    const uint64_t m = __ballot(le[i] <= t);
    if (more) below += __popcll(m);
    more = more && m == ~0ull;
  }
  for (int base = 64 * kFirst; more && base < a.num_reqs; base += 64) {
    const int r = base + lane;
    const uint64_t m = __ballot(r < a.num_reqs && a.q_offsets[r] <= t);
    below += __popcll(m);
    more = m == ~0ull;
  }
  // clamped into [0, num_reqs) like any request index (malformed offsets
  // then read a wrong request's pages, never out of the page table)
  return min(max(below - 1, 0), a.num_reqs - 1);
}

// ---------------------------------------------------------------------------
// Eight-wave kernel with 32-head waves, tiles of 32 and 64 rows.  Wave w has
// hp = w&1 (heads 32hp..+32), dh = (w>>1)&1 and rh = w>>2:
//   * S^T: rows (TILE/2)rh..+TILE/2 of the tile, dims 288dh..+288, 32 heads -
//     every K fragment read from LDS feeds two head blocks (half the reads of
//     16-head waves) and Q of 32 heads x 288 dims stays in registers;
//   * the dh pair swaps one head block of partial sums through LDS, so wave
//     dh holds the whole S^T of head block dh on its rows and exponentiates
//     only those (no softmax work is duplicated);
//   * P goes to LDS in the PV operand's row order; wave w then accumulates
//     O for its 32 heads on output columns 128(2rh+dh)..+128 over all rows
//     of the tile (each V fragment read by transpose feeds two head blocks).
// Softmax: the reference max of each head is fixed by the first tile with a
// valid row (all heads at once: masking is per row), so O is never rescaled;
// a tile sum above 2^52 (or not finite) sends the split through a second pass
// whose reference is the exact max of the first.  Masked rows enter S^T as an
// accumulator bias of -inf.
constexpr int kThreadsV2 = 512;
constexpr float kOverflowSum = 4503599627370496.f;   // 2^52

template <int TILE>
struct SmemV2 {
  static constexpr int kPStride = TILE + 8;     // bf16 per head in the P buffer
  uint16_t k[TILE * kKStride];
  int32_t rows[kRowChunk];
  float bias[kRowChunk];                        // 0 for a valid row, -inf for a masked one
  f32x4 xs[8][TILE / 32][64];                   // partial S^T sent to the dh partner
  uint16_t p[DSA_HEADS * kPStride];             // P[head][row in PV operand order]
  float red[2][2][2][16];                       // [rh][hp][dh][head]: max / l partials
  int last;                                     // last valid column of the row chunk
};

template <int KV, int TILE, bool kFinal>
__global__ __launch_bounds__(kThreadsV2) void partial_v2_kernel(PartialArgs a) {
  static_assert(TILE == 64, "tiles of 64 rows (32-row tiles run partial_ws_kernel)");
  __shared__ __attribute__((aligned(16))) SmemV2<TILE> sm;
  constexpr int kPS = SmemV2<TILE>::kPStride;
  constexpr int kOMB = TILE / 32;            // own 16-row blocks per wave
  constexpr int kKS = TILE / 32;             // PV k-steps
  constexpr int kQS = DSA_D_QK / 64;         // QK k-steps per half of the dims (9)
  constexpr int kNB = DSA_D_LATENT / 64;     // 16-column blocks per quarter of the 512 (8)

  const int t = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hp = wave & 1, dh = (wave >> 1) & 1, rh = wave >> 2;
  const int cq = (wave >> 1) & 3;            // output column quarter (2rh + dh)
  const int g = lane >> 4, c = lane & 15;
  const int c0 = s * a.cols_per_split;
  const int c1 = min(a.width, c0 + a.cols_per_split);
  const int req = request_of(a, t);
  const int pos = a.tok_pos[t];

  // Q of heads 32hp + 16hb + c, dims 288dh + 32ks + 8g .. +8 (MFMA B operand)
  u32x4 qf[2][kQS];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(
        a.q + (int64_t(t) * DSA_HEADS + 32 * hp + 16 * hb + c) * DSA_D_QK + (DSA_D_QK / 2) * dh);
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) qf[hb][ks] = qsrc[ks * 4 + g];
  }
  __builtin_amdgcn_s_waitcnt(0);   // Q resident before the tile loop

  f32x4 o[2][kNB];
  float m_ref, l_run;               // head 32hp + 16dh + c (lane column c)
  float m_run = kNegInf;            // exact running max over this wave's rows
  bool overflow = false;
  bool ref_set = false;             // workgroup-uniform: the references are fixed

  // K operand: rows (TILE/2)rh + 16mb + c, dims 288dh + 32ks + 8g = logical
  // chunk 36dh + 4ks + g, physical 36dh + 4ks + (g ^ bit3(36dh + 4ks))
  const int krow = ((TILE / 2) * rh + c) * kKStride + 8 * (DSA_D_QK / 16) * dh;
  const int klane0 = krow + 8 * g, klane1 = krow + 8 * (g ^ 1);
  const int kb = (DSA_D_QK / 64) * dh;       // bit3(36dh + 4ks) = bit1(9dh + ks)
  // V transpose read: rows 32k2 + 4g + c/4 (+16), columns 128cq + 16nb: logical
  // chunk 16cq + 2nb + (c%4)/2, whose bit 3 (bit 2 of nb) selects the base
  const int vrow = (4 * g + (c >> 2)) * kKStride + (DSA_D_LATENT / 4) * cq + 4 * (c & 1);
  const int vlane0 = vrow + 8 * ((c & 3) >> 1), vlane1 = vrow + 8 * (((c & 3) >> 1) ^ 1);
  // P: written at head 32hp + 16dh + c, read as the A operand of head 32hp + 16hb + c
  uint16_t* pw = sm.p + (32 * hp + 16 * dh + c) * kPS;

  auto compute_tile = [&](int it, const uint16_t* kt) {
    // S^T over this wave's rows and half of the dims, starting at the row bias
    f32x4 sacc[kOMB][2];
#pragma unroll
    for (int mb = 0; mb < kOMB; ++mb) {
      const f32x4 b =
          *reinterpret_cast<const f32x4*>(sm.bias + it * TILE + (TILE / 2) * rh + 16 * mb + 4 * g);
      sacc[mb][0] = b;
      sacc[mb][1] = b;
    }
#pragma unroll
    for (int ks = 0; ks < kQS; ++ks) {
      const uint16_t* kq = kt + (((kb + ks) >> 1) & 1 ? klane1 : klane0);
      u32x4 kf[kOMB];
#pragma unroll
      for (int mb = 0; mb < kOMB; ++mb)
        kf[mb] = *reinterpret_cast<const u32x4*>(kq + 16 * mb * kKStride + 32 * ks);
#pragma unroll
      for (int mb = 0; mb < kOMB; ++mb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          sacc[mb][hb] = dsa::mfma16x16x32(dsa::as_bf16x8(kf[mb]), dsa::as_bf16x8(qf[hb][ks]),
                                           sacc[mb][hb]);
    }
    // keep head block dh, send head block 1-dh to the partner (wave ^ 2)
    f32x4 sv[kOMB];
#pragma unroll
    for (int mb = 0; mb < kOMB; ++mb) {
      sm.xs[wave][mb][lane] = dh ? sacc[mb][0] : sacc[mb][1];
      sv[mb] = dh ? sacc[mb][1] : sacc[mb][0];
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < kOMB; ++mb) sv[mb] += sm.xs[wave ^ 2][mb][lane];   // float + commutes

    // tile max of the head over this wave's rows (log2 units, scale > 0)
    float tmax = kNegInf;
#pragma unroll
    for (int mb = 0; mb < kOMB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) tmax = fmaxf(tmax, sv[mb][j]);
    tmax = dsa::rows4_max(tmax) * a.scale_log2;
    m_run = fmaxf(m_run, tmax);
    // the first tile with a valid row fixes every head's reference (the
    // condition reads only shared row data, so all waves take the branch)
    if (!ref_set &&
        __ballot(lane < TILE && sm.rows[it * TILE + min(lane, TILE - 1)] >= 0) != 0ull) {
      if (g == 0) sm.red[rh][hp][dh][c] = tmax;
      __syncthreads();
      m_ref = fmaxf(sm.red[0][hp][dh][c], sm.red[1][hp][dh][c]);
      __syncthreads();
      ref_set = true;
    }
    const float neg_m = m_ref == kNegInf ? 0.f : -m_ref;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < kOMB; ++mb) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(fmaf(sv[mb][j], a.scale_log2, neg_m));   // exp2(-inf) = 0
        psum += p[j];
      }
      // rows (TILE/2)rh + 16mb + 4g + j -> position 32k2 + 8g + 4h + j
      const int blk = kOMB * rh + mb;
      *reinterpret_cast<u32x2*>(pw + 32 * (blk >> 1) + 8 * g + 4 * (blk & 1)) =
          u32x2{dsa::pack_bf16x2(p[0], p[1]), dsa::pack_bf16x2(p[2], p[3])};
    }
    psum = dsa::rows4_sum(psum);
    l_run += psum;
    overflow = overflow || !(psum <= kOverflowSum);
    __syncthreads();

    // O[32 heads x 128 columns] += P V over the tile's rows
    u32x4 pa[2][kKS];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int k2 = 0; k2 < kKS; ++k2)
        pa[hb][k2] = *reinterpret_cast<const u32x4*>(sm.p + (32 * hp + 16 * hb + c) * kPS + 32 * k2 + 8 * g);
#pragma unroll
    for (int k2 = 0; k2 < kKS; ++k2)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const uint16_t* vp = kt + ((nb >> 2) & 1 ? vlane1 : vlane0) + 32 * k2 * kKStride + 16 * nb;
        const u32x2 lo2 = lds_read_tr16(vp);
        const u32x2 hi2 = lds_read_tr16(vp + 16 * kKStride);
        const u32x4 vb = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          o[hb][nb] = dsa::mfma16x16x32(dsa::as_bf16x8(pa[hb][k2]), dsa::as_bf16x8(vb), o[hb][nb]);
      }
  };

  Stage<KV, TILE, kThreadsV2> st;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    if (pass == 0) {
      m_ref = kNegInf;
      ref_set = false;
    } else {
      // exact max of the first pass, over both row halves
      if (g == 0) sm.red[rh][hp][dh][c] = m_run;
      __syncthreads();
      m_ref = fmaxf(sm.red[0][hp][dh][c], sm.red[1][hp][dh][c]);
      overflow = false;
      ref_set = true;
    }
    for (int cc = c0; cc < c1; cc += kRowChunk) {
      const int cend = min(c1, cc + kRowChunk);
      if (tid == 0) sm.last = -1;
      __syncthreads();
      // the plain loop: with the accumulators live here, the batched form
      // spilled 3-4 VGPRs in this 256-register kernel
      resolve_rows<kRowChunk, kThreadsV2, 0>(a, t, req, pos, cc, cend, sm.rows, tid, &sm.last, sm.bias);
      __syncthreads();
      // tiles up to the last valid row (trailing -1 padding is skipped: its
      // rows would contribute exactly nothing)
      const int ntile = (sm.last + TILE) / TILE;
      if (ntile == 0) continue;
      st.load(a.latent, sm.rows, tid);
      st.store(sm.k, 0, tid);
      __syncthreads();
      for (int it = 0; it < ntile; ++it) {
        const bool more = it + 1 < ntile;
        if (more) st.load(a.latent, sm.rows + (it + 1) * TILE, tid);
        compute_tile(it, sm.k);
        __syncthreads();
        if (more) {
          st.store(sm.k, 0, tid);
          __syncthreads();
        }
      }
    }
    if (!__syncthreads_or(overflow)) break;
  }

  // l of each head = the two row halves' sums; then normalize and write.  The
  // lane's indices are taken afresh here rather than held through the tile
  // loop (where they spilled).
  const int le = dsa::fresh_lane(), ge = le >> 4, ce = le & 15;
  __syncthreads();
  if (ge == 0) sm.red[rh][hp][dh][ce] = l_run;
  __syncthreads();
  const int64_t ts = int64_t(t) * a.splits + s;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = 4 * ge + j;
      const float lj = sm.red[0][hp][hb][hh] + sm.red[1][hp][hb][hh];
      const float inv = lj > 0.f ? 1.f / lj : 0.f;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        put_out<kFinal>(a, ts, 32 * hp + 16 * hb + hh, (DSA_D_LATENT / 4) * cq + 16 * nb + ce,
                        o[hb][nb][j] * inv);
    }
  }
  if (rh == 0 && ge == 0) {
    const float l = sm.red[0][hp][dh][ce] + sm.red[1][hp][dh][ce];
    put_lse<kFinal>(a, ts, 32 * hp + 16 * dh + ce, l > 0.f ? (m_ref + log2f(l)) * kLn2 : kNegInf);
  }
}

// ---------------------------------------------------------------------------
// Warp-specialized kernel, tiles of 32 rows: one workgroup per (token,
// split), two roles, every SIMD running one score wave beside its value waves.
//   * Score waves 0..3: wave w computes S^T for heads 16w..+16 over all 576
//     dims and the tile's 32 rows (the Q of its heads stays in registers, so
//     no partial sums are exchanged between waves), runs the online softmax
//     with a running per-head max (O is rescaled only when a head's max grows
//     by more than 2^8) and writes P and the per-head rescale factor to LDS.
//   * Value waves: O for all 64 heads on a slice of the output columns, 8
//     waves of 64 columns for FP8 rows (12 waves, three per SIMD) or 4 of 128
//     for BF16 rows (8 waves); each transposed V fragment read feeds four
//     head blocks.
// The roles run one tile apart: in iteration j the score waves work on tile
// j while the value waves run PV of tile j-1, so on each SIMD one wave's
// MFMAs can overlap the other waves' softmax and staging work instead of
// every wave passing through the same phase between barriers.  K tiles are a
// ring of three bf16 buffers (score waves read tile j, value waves tile j-1,
// tile j+1 is staged into the third) and P a ring of two: one barrier per
// tile.  The selected rows are gathered two tiles ahead into registers and
// dequantized and stored to LDS after the role work: by the value waves for
// FP8 rows (the score waves' registers hold their Q), by every thread for
// the wider BF16 rows.
constexpr int kTileWS = 32;
// Value waves of the warp-specialized kernel: 8 of 64 columns for FP8 rows
// (12 waves, three per SIMD); 4 of 128 columns for BF16 rows, whose staging
// (twice the bytes per row) does not fit beside the accumulators in the
// three-wave register budget.
template <int KV>
constexpr int ws_value_waves() { return KV == DSA_KV_FP8_E4M3_S64 ? 8 : 4; }
constexpr int kWSKLook = 2;                 // k-steps ahead the score waves read K fragments
constexpr int kPStrideWS = kTileWS;         // bf16 per head in a P buffer (64 bytes)

// 16-byte chunk of a P row: logical chunk g (PV operand positions 8g..8g+7)
// of head h sits at g ^ p_swz(h), p_swz(h) = bits 1-2 of h.  A 64-lane
// 16-byte LDS read is served in four passes of 16 lanes: lanes 0-31 and
// 32-63 apart, and within a half the lanes whose bits 2, 3 and 4 have even
// parity apart from those with odd parity (measured: a probe that makes two
// lanes l and l^m hit the same banks conflicts exactly for m in {1-3, 12-15,
// 20-27}).  With heads h = lane & 15 and chunk groups g = lane >> 4, every
// pass then meets 16 distinct 16-byte slots of its 256 bytes, for the value
// waves' operand reads and for the score waves' writes of the same layout
// (8 consecutive lanes, or the passes above).  The previous XOR (bit 0 =
// bit 1 ^ bit 3 of h, bit 1 = bit 2) gave every P read 2-way conflicts:
// 8.4M conflict cycles per verify-batch launch, 9% of its LDS activity.
__device__ __forceinline__ int p_swz(int h) { return (h >> 1) & 3; }

struct SmemWS {
  uint16_t k[3][kTileWS * kKStride];          // bf16 K tiles (ring of three)
  uint16_t p[2][DSA_HEADS * kPStrideWS];      // P of a tile in the PV operand's row order
  float alpha[2][DSA_HEADS];                  // O *= alpha before PV of that tile
  uint32_t resc[2][4];                        // score wave w: a head of its tile moved its max
  int32_t rows[kRowChunk];
  float bias[kRowChunk];                      // 0 for a valid row, -inf for a masked one
  float fin_l[DSA_HEADS];
  int last;
};

// Tiles gathered ahead into registers: two.  A load then has two tile steps
// to arrive instead of one (verify batch -2 to -4%, prefill chunk -2%, BF16
// -1%); a third tile measured no faster for FP8 rows and spills for BF16.
template <int KV, int NV>
constexpr int ws_depth() { return 2; }

// Waves that stage nothing (the score waves of the 12-wave form).
struct NoStage {
  __device__ __forceinline__ void load(const uint8_t*, const int32_t*, int) {}
  __device__ __forceinline__ void store(uint16_t*, int, int) const {}
};


// The tile pipeline shared by both roles, so that both execute exactly the
// same barriers: per row chunk the rows are resolved, tiles 0..kD-1 are
// fetched and tile 0 staged; iteration j = 0, 1, ... (at least through ntile,
// in whole groups of three) calls work(j, ntile, P) (P = j % 3 at compile
// time; work contains no barrier and does no role work past ntile), stages
// tile j+1 (held in register set (j+1) % kD) into K buffer (j+1) % 3,
// fetches tile j+1+kD into that set and waits at the barrier.  The staging
// follows the role work (spread between the score waves' MFMAs, done by the
// score waves alone, or done before PV, it measured slower or no faster).
// Loads and stores run unconditionally (row indices clamped to the chunk's
// last tile): past the last tile they refill a buffer nobody reads.
template <int KV, int NV, class Stager, class Work>
__device__ __forceinline__ void ws_pipeline(const PartialArgs& a, SmemWS& sm, int t, int req,
                                            int pos, int c0, int c1, int wave, int sid,
                                            Work&& work) {
  constexpr int TILE = kTileWS;
  constexpr int NT = (4 + NV) * 64;
  constexpr int kD = ws_depth<KV, NV>();
  Stager st[kD];
  for (int cc = c0; cc < c1; cc += kRowChunk) {
    const int cend = min(c1, cc + kRowChunk);
    const int tid = 64 * wave + dsa::fresh_lane();   // not held through the tile loop
    __syncthreads();                            // every thread has read the last chunk's state
    if (tid == 0) sm.last = -1;
    __syncthreads();
    resolve_rows<kRowChunk, NT>(a, t, req, pos, cc, cend, sm.rows, tid, &sm.last, sm.bias);
    __syncthreads();
    const int ntile = (sm.last + TILE) / TILE;
    if (ntile == 0) continue;
    auto tile_rows = [&](int i) { return sm.rows + min(i, ntile - 1) * TILE; };
    dsa::static_for<kD>([&](auto D) { st[decltype(D)::value].load(a.latent, tile_rows(D), sid); });
    st[0].store(sm.k[0], 0, sid);
    st[0].load(a.latent, tile_rows(kD), sid);
    __syncthreads();
    // Whole groups of three iterations, every one staging and fetching: the
    // fetches then form one straight-line stream whose in-order completion
    // counts the compiler can track (a conditional iteration makes it wait
    // for every load in flight).  work() skips iterations past ntile.  The
    // loop body holds two groups so that the register set of every
    // iteration is known at compile time (kD divides six); an odd last group
    // runs after the loop (an exit between the two groups spilled).
    static_assert(6 % kD == 0, "register sets cycle within two groups of three");
    auto group = [&](int j0, auto H) {
      dsa::static_for<3>([&](auto P) {
        constexpr int p = decltype(P)::value;
        const int j = j0 + p;
        constexpr int si = (3 * decltype(H)::value + p + 1) % kD;
        work(j, ntile, P);
        st[si].store(sm.k[(p + 1) % 3], 0, sid);
        st[si].load(a.latent, tile_rows(j + 1 + kD), sid);
        __syncthreads();
      });
    };
    const int ngroups = ntile / 3 + 1;
    for (int j0 = 0; j0 < 3 * (ngroups & ~1); j0 += 6) {
      group(j0, std::integral_constant<int, 0>{});
      group(j0 + 3, std::integral_constant<int, 1>{});
    }
    if (ngroups & 1) group(3 * (ngroups - 1), std::integral_constant<int, 0>{});
  }
}

template <int KV, bool kFinal, int NV>
__global__ __launch_bounds__((4 + NV) * 64) void partial_ws_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) SmemWS sm;
  constexpr int TILE = kTileWS;
  // 4 value waves: every thread stages (Stage over 512 threads); 8: the score
  // waves hold the Q of their heads and stage nothing, the 512 value threads
  // stage the whole tile
  using ScoreStage = std::conditional_t<NV == 4, Stage<KV, TILE, 512>, NoStage>;
  using ValueStage = Stage<KV, TILE, 512>;
  constexpr int kSidValue0 = NV == 4 ? 256 : 0;   // stage index of the first value thread
  constexpr int kQS = DSA_D_QK / 32;           // 18 QK k-steps
  constexpr int kNB = DSA_D_LATENT / (16 * NV);   // 16-column blocks of a value wave
  constexpr int kVCols = DSA_D_LATENT / NV;        // output columns of a value wave

  const int t = blockIdx.x, s = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c0 = s * a.cols_per_split;
  const int c1 = min(a.width, c0 + a.cols_per_split);
  const int req = request_of(a, t);
  const int pos = a.tok_pos[t];
  const int64_t ts = int64_t(t) * a.splits + s;

  // Each role derives its thread indices itself: the two roles' code is laid
  // out one after the other, and an index taken before the branch would be
  // held through the first role's tile loop for the second.
  if (wave < 4) {
    // ---- score wave: heads 16*wave + c (lane column c)
    const int lane = dsa::fresh_lane(), tid = 64 * wave + lane;
    const int g = lane >> 4, c = lane & 15;
    const int head = 16 * wave + c;
    u32x4 qf[kQS];   // Q of heads 16*wave..+16, dims 32ks + 8g .. +8 (MFMA B operand)
    {
      const u32x4* qsrc = reinterpret_cast<const u32x4*>(a.q + (int64_t(t) * DSA_HEADS + head) * DSA_D_QK);
#pragma unroll
      for (int ks = 0; ks < kQS; ++ks) qf[ks] = qsrc[ks * 4 + g];
    }
    // running max of the head and this lane's share of its sum (rows 4g..+4
    // of every block), summed over the lanes once at the end
    float m_run = kNegInf, l_lane = 0.f;
    // K operand: rows 16mb + c, dims 32ks + 8g = logical chunk 4ks + g, physical
    // 4ks + (g ^ bit1(ks))
    const int klane0 = c * kKStride + 8 * g;
    const int klane1 = c * kKStride + 8 * (g ^ 1);
    ws_pipeline<KV, NV, ScoreStage>(a, sm, t, req, pos, c0, c1, wave, tid, [&](int j, int ntile, auto P) {
      constexpr int p = decltype(P)::value;
      if (j < ntile) {
        const uint16_t* kq0 = sm.k[p] + klane0;
        const uint16_t* kq1 = sm.k[p] + klane1;
        f32x4 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          sacc[mb] = *reinterpret_cast<const f32x4*>(sm.bias + j * TILE + 16 * mb + 4 * g);
        // K fragments of k-step ks (rows 16mb + c) in a ring of kWSKLook + 1
        auto kread = [&](int ks, int mb) {
          const uint16_t* kq = (ks >> 1) & 1 ? kq1 : kq0;
          return *reinterpret_cast<const u32x4*>(kq + 16 * mb * kKStride + 32 * ks);
        };
        u32x4 kr[kWSKLook + 1][2];
        dsa::static_for<kWSKLook>([&](auto L) {
          constexpr int l = decltype(L)::value;
          kr[l][0] = kread(l, 0);
          kr[l][1] = kread(l, 1);
        });
        dsa::static_for<kQS>([&](auto KS) {
          constexpr int ks = decltype(KS)::value;
          if constexpr (ks + kWSKLook < kQS) {
            kr[(ks + kWSKLook) % (kWSKLook + 1)][0] = kread(ks + kWSKLook, 0);
            kr[(ks + kWSKLook) % (kWSKLook + 1)][1] = kread(ks + kWSKLook, 1);
          }
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            sacc[mb] = dsa::mfma16x16x32(dsa::as_bf16x8(kr[ks % (kWSKLook + 1)][mb]),
                                         dsa::as_bf16x8(qf[ks]), sacc[mb]);
        });
        // tile max of the head (log2 units; -inf when every row is masked)
        float tmax = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) tmax = fmaxf(tmax, sacc[mb][jj]);
        tmax = dsa::rows4_max(tmax) * a.scale_log2;
        float alpha = 1.f;
        if (tmax > m_run + kRescaleThreshold) {
          if (m_run != kNegInf) alpha = __builtin_amdgcn_exp2f(m_run - tmax);
          l_lane *= alpha;
          m_run = tmax;
        }
        // masked rows: -inf * scale - m = -inf, exp2 gives 0; while no row has
        // been valid m is -inf and every row so far is masked
        const float neg_m = m_run == kNegInf ? 0.f : -m_run;
        // rows 16mb + 4g + jj -> PV operand position 8g + 4mb + jj: this lane's
        // eight values are logical chunk g of the head's P row
        float psum = l_lane;
        uint32_t pk[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          float pr[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            pr[jj] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][jj], a.scale_log2, neg_m));
            psum += pr[jj];
          }
          pk[2 * mb] = dsa::pack_bf16x2(pr[0], pr[1]);
          pk[2 * mb + 1] = dsa::pack_bf16x2(pr[2], pr[3]);
        }
        *reinterpret_cast<u32x4*>(sm.p[j & 1] + head * kPStrideWS + 8 * (g ^ p_swz(c))) =
            u32x4{pk[0], pk[1], pk[2], pk[3]};
        l_lane = psum;
        if (g == 0) sm.alpha[j & 1][head] = alpha;
        // one word per wave for the value waves: does PV of this tile start
        // with a rescale of O
        const bool any_resc = __any(alpha != 1.f);
        if (g == 0 && c == 0) sm.resc[j & 1][wave] = any_resc;
      }
    });
    const float l_run = dsa::rows4_sum(l_lane);
    if (g == 0) {
      sm.fin_l[head] = l_run;
      put_lse<kFinal>(a, ts, head, l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf);
    }
    __syncthreads();
  } else {
    // ---- value wave: all 64 heads, output columns kVCols*q..+kVCols
    const int q = wave - 4;
    const int sid = 64 * q + dsa::fresh_lane() + kSidValue0;
    f32x4 o[4][kNB];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // V transpose read: rows 4g + c/4 (+16), columns kVCols*q + 16nb: logical
    // chunk x = (kVCols/8)q + 2nb + (c%4)/2; bit 3 of the even chunk selects
    // the lane base, and as kVCols/8 is a multiple of 8 it flips with nb at
    // compile time relative to nb = 0.  The lane offsets are computed once;
    // each tile takes laundered copies, so the compiler cannot derive and
    // hold per-ring-slot addresses from them (that spilled).
    static_assert((kVCols / 8) % 8 == 0, "V lane base depends on q and nb only");
    int v_even, v_odd, p_off;
    {
      const int ln = dsa::fresh_lane();
      const int g = ln >> 4, c = ln & 15;
      const int vrow = (4 * g + (c >> 2)) * kKStride + kVCols * q + 4 * (c & 1);
      const int vlane0 = vrow + 8 * ((c & 3) >> 1);
      const int vlane1 = vrow + 8 * (((c & 3) >> 1) ^ 1);
      const bool hi0 = (((kVCols / 8) * q) >> 3) & 1;
      v_even = hi0 ? vlane1 : vlane0;
      v_odd = hi0 ? vlane0 : vlane1;
      p_off = c * kPStrideWS + 8 * (g ^ p_swz(c));
    }
    ws_pipeline<KV, NV, ValueStage>(a, sm, t, req, pos, c0, c1, wave, sid,
                                    [&](int j, int ntile, auto P) {
      constexpr int p = decltype(P)::value;
      if (j >= 1 && j <= ntile) {
        const int jp = j - 1;   // PV of the previous tile, in K buffer (p + 2) % 3
        int ve = v_even, vo = v_odd, po = p_off;
        asm volatile("" : "+v"(ve), "+v"(vo), "+v"(po));
        // O *= alpha of the heads this lane holds (rows 4g + jj of each head
        // block), only in the rare tiles where some score wave moved a head's
        // reference: one LDS word per score wave says so, instead of every
        // lane testing its 16 factors (that test's VALU work, on the SIMDs
        // the score waves share, cost 4-5%)
        const u32x4 rf = *reinterpret_cast<const u32x4*>(sm.resc[jp & 1]);
        if (__builtin_amdgcn_readfirstlane(rf[0] | rf[1] | rf[2] | rf[3]) != 0) {
          const float* alp = sm.alpha[jp & 1] + 4 * (dsa::fresh_lane() >> 4);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(alp + 16 * hb);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) o[hb][nb][jj] *= al[jj];
          }
        }
        const uint16_t* pb = sm.p[jp & 1];
        u32x4 pa[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          pa[hb] = *reinterpret_cast<const u32x4*>(pb + 16 * hb * kPStrideWS + po);
        // V fragments read one column block ahead; one staging step of the
        // next tile after each block's four MFMAs
        const uint16_t* vt = sm.k[(p + 2) % 3];
        auto vread = [&](int nb) {
          const uint16_t* vp = vt + (((2 * nb) >> 3) & 1 ? vo : ve) + 16 * nb;
          const u32x2 lo2 = lds_read_tr16(vp);
          const u32x2 hi2 = lds_read_tr16(vp + 16 * kKStride);
          return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        };
        u32x4 vb = vread(0);
        dsa::static_for<kNB>([&](auto NB) {
          constexpr int nb = decltype(NB)::value;
          u32x4 vn;
          if constexpr (nb + 1 < kNB) vn = vread(nb + 1);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb)
            o[hb][nb] = dsa::mfma16x16x32(dsa::as_bf16x8(pa[hb]), dsa::as_bf16x8(vb), o[hb][nb]);
          if constexpr (nb + 1 < kNB) vb = vn;
        });
      }
    });
    __syncthreads();   // the score waves have written each head's sum
    // the output addresses are derived from a fresh lane index, so the
    // compiler computes them here instead of keeping them live through the
    // tile loop (where they spilled)
    const int lane_e = dsa::fresh_lane();
    const int ge = lane_e >> 4, ce = lane_e & 15;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int hh = 16 * hb + 4 * ge + jj;
        const float l = sm.fin_l[hh];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
          put_out<kFinal>(a, ts, hh, kVCols * q + 16 * nb + ce, o[hb][nb][jj] * inv);
      }
  }
}

// ---------------------------------------------------------------------------
// Q8 prefill ["Accelerating GLM-5.3-Flash on H200", section 4 "Prefill
// dataflow optimization": the prefill attention multiplies an FP8 query with
// the FP8 cache].  S = K Q^T runs on gfx950's scaled 32x32x64 f8f6f4 MFMA, the
// FP8 form with twice the bf16 rate.  Its 64-deep contraction is exactly one
// scale group of a cache row and each lane's 32 codes one block, so the
// MFMA applies every row's power-of-two group scale itself (E8M0 block
// scale = the exponent byte of the stored fp32 scale) and the nine group
// products accumulate in one chain; the query's one scale per head multiplies
// the finished score.  The value product stays on bf16 with V dequantized
// once per tile, as in the bf16 path.
//
// One workgroup per token, 8 waves (wave w runs on SIMD w % 4), tiles of 32
// rows:
//   * score waves 0, 1: heads 32w..+32 against the tile's 32 rows; lane l holds
//     head 32w + l%32 and rows 8q + 4(l/32) + j (q, j < 4), the query codes of
//     its head stay in registers; online softmax with the running reference
//     max of the bf16 kernels;
//   * value waves: O for all 64 heads on a slice of the output columns; waves
//     2, 3, 6, 7 (SIMDs 2 and 3, which hold no score wave) take 96 columns
//     each, waves 4 and 5 (beside the score waves) 64, so each SIMD gets a
//     similar share of matrix work;
//   * after its role work every thread gathers and dequantizes two latent
//     chunks of a coming tile (waves 4 and 5 also the rope codes).
// Per tile the raw codes go to a ring of two buffers (score waves read tile j
// while tile j+1 is written) with their scale exponents beside them, the dequantized
// latent to a ring of three (value waves read tile j-1) and P to a ring of
// two; one barrier per tile.
constexpr int kTileQ8 = 32;
constexpr int kRowChunkQ8 = 1024;              // index columns resolved at once (LDS budget)
constexpr int kK8Stride = DSA_D_QK + 16;       // bytes per raw-code row: 37 16-byte chunks
constexpr int kVStrideQ8 = DSA_D_LATENT + 16;  // bf16 per V row: 1056 bytes = 33 x 32
constexpr int kQ8Groups = DSA_D_QK / 64;       // 9 scale groups = 9 MFMA k-steps

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Raw-code tile: rows 37 16-byte chunks apart (odd).  A score lane (row
// m = l%32, half h = l/32) reads chunks 4g + h and 4g + 2 + h of group g; a
// 16-byte read is served in passes of 16 lanes of one half whose lane bits
// 2-4 share a parity, so a pass holds one of rows m and m + 16 for each m
// mod 16, and the odd stride puts those 16 rows on 16 distinct bank slots.
// (A flip of the chunk by bit 4 of the row, made for a wrongly assumed pass
// grouping, put two rows of every pass on the same banks.)  Staging writes
// (8 lanes on 8 consecutive chunks of a row) are conflict-free as well.
// V tile: logical bf16 chunk x (8 values) of row r at k_phys(x), rows 33
// 32-byte units apart (odd), which keeps the transpose reads and the staging
// writes conflict-free, as in the bf16 K tile.
struct SmemQ8 {
  uint8_t k8[2][kTileQ8 * kK8Stride];          // raw E4M3 codes
  uint8_t sc8[2][kTileQ8][16];                 // E8M0 exponents of the 9 group scales per row
  uint16_t v[3][kTileQ8 * kVStrideQ8];         // dequantized latent (V), bf16
  uint16_t p[2][DSA_HEADS * kPStrideWS];       // P in the PV operand's row order
  float alpha[2][DSA_HEADS];
  uint32_t resc[2][2];                        // score wave w: a head of its tile moved its max
  int32_t rows[kRowChunkQ8];
  float bias[kRowChunkQ8];
  float fin_l[DSA_HEADS];
  int last;
};
static_assert(sizeof(SmemQ8) <= 160 * 1024, "Q8 tiles exceed the LDS");

// acc += (A * 2^(ea - 127)) (B), E4M3 operands (format 0); A's block scale is
// byte S of sa in each lane, B's is 2^0 (E8M0 127).
template <int S>
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(const i32x8& a, const i32x8& b, int sa,
                                                   const f32x16& acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, S, sa, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Max / sum of lanes l and l ^ 32, every lane receiving the result: after
// v_permlane32_swap one result holds lane l % 32's value and the other lane
// l % 32 + 32's, in every lane.
__device__ __forceinline__ float halves_max(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Tile gather, spread over all 512 threads by chunk index cid: latent chunk
// q = cid + 256i (i < NC) is row q / 32, codes 16(q % 32)..+16, group
// (q % 32) / 4.  Every thread takes two chunks; the wide value waves (cid
// 0..511), whose registers hold the 96-column accumulators, gather one tile
// ahead, the score and narrow value waves three (measured 3% faster than
// loading the wide waves less).  With kRope the thread (waves 4 and 5,
// r = tid - 256) also gathers rope chunk r: row r / 4, rope codes
// 16(r % 4)..+16, and the r % 4 == 0 thread the rope group's scale.  Invalid
// rows load row 0 and store zero codes and scales.
template <int NC, bool kRope, int kDepthT>
struct Q8Stage {
  static constexpr int kDepth = kDepthT;     // tiles gathered ahead (1 or 3)
  u32x4 code[NC];
  float scale[NC];
  u32x4 rcode;
  float rscale;
  uint32_t ok;
  __device__ __forceinline__ void load(const uint8_t* latent, const int32_t* rows, int cid, int tid) {
    ok = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int q = cid + 256 * i;
      const int phys = rows[q >> 5];
      ok |= uint32_t(phys >= 0) << i;
      const uint8_t* row = latent + int64_t(max(phys, 0)) * 640;
      code[i] = *reinterpret_cast<const u32x4*>(row + 16 * (q & 31));
      scale[i] = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * ((q & 31) >> 2));
    }
    if constexpr (kRope) {
      const int r = tid - 256;
      const int phys = rows[r >> 2];
      ok |= uint32_t(phys >= 0) << NC;
      const uint8_t* row = latent + int64_t(max(phys, 0)) * 640;
      rcode = *reinterpret_cast<const u32x4*>(row + DSA_D_LATENT + 16 * (r & 3));
      rscale = *reinterpret_cast<const float*>(row + DSA_D_QK + 4 * 8);
    }
  }
  __device__ __forceinline__ void store(uint8_t* k8, uint8_t* sc8, uint16_t* v, int cid,
                                        int tid) const {
    // the LDS addresses are computed at each store from opaque copies of the
    // indices, not hoisted out of the loops and held (they spilled)
    asm volatile("" : "+v"(cid), "+v"(tid));
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int q = cid + 256 * i, r = q >> 5, c = q & 31;
      const bool okb = (ok >> i) & 1u;
      const u32x4 cd = okb ? code[i] : u32x4{0, 0, 0, 0};
      const float s = okb ? scale[i] : 0.f;
      *reinterpret_cast<u32x4*>(k8 + r * kK8Stride + 16 * c) = cd;
      // bf16 chunks 2c, 2c + 1 at k_phys(2c), k_phys(2c) ^ 1
      const u32x2 a0 = dq4_bf16(cd[0], s), a1 = dq4_bf16(cd[1], s);
      *reinterpret_cast<u32x4*>(v + r * kVStrideQ8 + 8 * k_phys(2 * c)) =
          u32x4{a0[0], a0[1], a1[0], a1[1]};
      const u32x2 b0 = dq4_bf16(cd[2], s), b1 = dq4_bf16(cd[3], s);
      *reinterpret_cast<u32x4*>(v + r * kVStrideQ8 + 8 * (k_phys(2 * c) ^ 1)) =
          u32x4{b0[0], b0[1], b1[0], b1[1]};
      if ((c & 3) == 0) sc8[r * 16 + (c >> 2)] = uint8_t(__float_as_uint(s) >> 23);
    }
    if constexpr (kRope) {
      const int rr = tid - 256, r = rr >> 2, c = DSA_D_LATENT / 16 + (rr & 3);
      const bool okb = (ok >> NC) & 1u;
      *reinterpret_cast<u32x4*>(k8 + r * kK8Stride + 16 * c) = okb ? rcode : u32x4{0, 0, 0, 0};
      if ((rr & 3) == 0) sc8[r * 16 + 8] = okb ? uint8_t(__float_as_uint(rscale) >> 23) : 0;
    }
  }
};

// The tile loop shared by all roles (identical barriers): per chunk of
// kRowChunkQ8 index columns the rows are resolved, tiles 0..kD-1
// gathered and tile 0 stored; iteration j (in whole groups of three, so the
// gathers form one straight-line stream) calls work(j, ntile, P), stores tile
// j + 1 (codes and scale exponents into buffer (j + 1) % 2, V into (j + 1) % 3),
// gathers tile j + 1 + kD and waits at the barrier (kD = the role's
// Stager::kDepth, 1 or 3, so a role's register stages divide the group of
// three iterations).  Past the last tile
// the row indices are clamped and the stores refill buffers nobody reads.
template <class Stager, class Work>
__device__ __forceinline__ void q8_pipeline(const PartialArgs& a, SmemQ8& sm, int t, int req,
                                            int pos, int tid, int cid, Work&& work) {
  constexpr int kD = Stager::kDepth;
  Stager st[kD];
  for (int cc = 0; cc < a.width; cc += kRowChunkQ8) {
    const int cend = min(a.width, cc + kRowChunkQ8);
    __syncthreads();
    if (tid == 0) sm.last = -1;
    __syncthreads();
    resolve_rows<kRowChunkQ8, kThreadsV2>(a, t, req, pos, cc, cend, sm.rows, tid, &sm.last, sm.bias);
    __syncthreads();
    const int ntile = (sm.last + kTileQ8) / kTileQ8;
    if (ntile == 0) continue;
    auto tile_rows = [&](int i) { return sm.rows + min(i, ntile - 1) * kTileQ8; };
    dsa::static_for<kD>([&](auto D) { st[decltype(D)::value].load(a.latent, tile_rows(D), cid, tid); });
    st[0].store(sm.k8[0], &sm.sc8[0][0][0], sm.v[0], cid, tid);
    st[0].load(a.latent, tile_rows(kD), cid, tid);
    __syncthreads();
    for (int j0 = 0; j0 <= ntile; j0 += 3) {
      dsa::static_for<3>([&](auto P) {
        constexpr int p = decltype(P)::value;
        const int j = j0 + p;
        constexpr int si = (p + 1) % kD;
        work(j, ntile, P);
        const int kn = (j + 1) & 1;
        st[si].store(sm.k8[kn], &sm.sc8[kn][0][0], sm.v[(p + 1) % 3], cid, tid);
        st[si].load(a.latent, tile_rows(j + 1 + kD), cid, tid);
        __syncthreads();
      });
    }
  }
}

// Value role: O for all 64 heads on columns d0..d0 + 16NB (PV of tile j - 1 in
// iteration j, as in the bf16 warp-specialized kernel).
template <int NB, class Stager>
__device__ __forceinline__ void q8_value(const PartialArgs& a, SmemQ8& sm, int t, int req, int pos,
                                         int tid, int cid, int d0) {
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  f32x4 o[4][NB];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transpose read of rows 4g + c/4 (+16), columns d0 + 16nb + 4(c%4): logical
  // chunk x = d0/8 + 2nb + (c%4)/2, physical k_phys(x) (bit 3 of the even
  // chunk, the same for the wave, picks the lane base)
  const int vrow = (4 * g + (c >> 2)) * kVStrideQ8 + d0 + 4 * (c & 1);
  const int vlane0 = vrow + 8 * ((c & 3) >> 1);
  const int vlane1 = vrow + 8 * (((c & 3) >> 1) ^ 1);
  const int xb = d0 >> 3;
  q8_pipeline<Stager>(a, sm, t, req, pos, tid, cid, [&](int j, int ntile, auto P) {
    constexpr int p = decltype(P)::value;
    if (j >= 1 && j <= ntile) {
      const int jp = j - 1;
      // O *= alpha only in the rare tiles where a score wave moved a head's
      // reference (one word per score wave)
      const u32x2 rf = *reinterpret_cast<const u32x2*>(sm.resc[jp & 1]);
      if (__builtin_amdgcn_readfirstlane(rf[0] | rf[1]) != 0) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const f32x4 al = *reinterpret_cast<const f32x4*>(sm.alpha[jp & 1] + 16 * hb + 4 * g);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[hb][nb][jj] *= al[jj];
        }
      }
      const uint16_t* pb = sm.p[jp & 1];
      u32x4 pa[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        pa[hb] = *reinterpret_cast<const u32x4*>(pb + (16 * hb + c) * kPStrideWS + 8 * (g ^ p_swz(c)));
      const uint16_t* vt = sm.v[(p + 2) % 3];
      auto vread = [&](int nb) {
        const int x = xb + 2 * nb;
        const uint16_t* vp = vt + ((x >> 3) & 1 ? vlane1 : vlane0) + 16 * nb;
        const u32x2 lo2 = lds_read_tr16(vp);
        const u32x2 hi2 = lds_read_tr16(vp + 16 * kVStrideQ8);
        return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      };
      u32x4 vb = vread(0);
      dsa::static_for<NB>([&](auto NBI) {
        constexpr int nb = decltype(NBI)::value;
        u32x4 vn;
        if constexpr (nb + 1 < NB) vn = vread(nb + 1);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
          o[hb][nb] = dsa::mfma16x16x32(dsa::as_bf16x8(pa[hb]), dsa::as_bf16x8(vb), o[hb][nb]);
        if constexpr (nb + 1 < NB) vb = vn;
      });
    }
  });
  __syncthreads();   // the score waves have written each head's sum
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int hh = 16 * hb + 4 * g + jj;
      const float l = sm.fin_l[hh];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) put_out<true>(a, t, hh, d0 + 16 * nb + c, o[hb][nb][jj] * inv);
    }
}

__global__ __launch_bounds__(kThreadsV2) void partial_q8_kernel(PartialArgs a) {
  __shared__ __attribute__((aligned(16))) SmemQ8 sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int req = request_of(a, t);
  const int pos = a.tok_pos[t];

  if (wave < 2) {
    // ---- score wave: heads 32w + n; MFMA A = code rows (row m = lane % 32),
    // B = query codes (head n = lane % 32), both halves h = lane / 32 holding
    // logical chunks 4g + h and 4g + 2 + h of group g
    const int n = lane & 31, h = lane >> 5;
    const int head = 32 * wave + n;
    i32x8 qf[kQ8Groups];
    {
      const uint8_t* qs = a.q8 + (int64_t(t) * DSA_HEADS + head) * DSA_D_QK + 16 * h;
#pragma unroll
      for (int g = 0; g < kQ8Groups; ++g)
        qf[g] = cat8(*reinterpret_cast<const u32x4*>(qs + 64 * g),
                     *reinterpret_cast<const u32x4*>(qs + 64 * g + 32));
    }
    const float cq = a.q8_scale[int64_t(t) * DSA_HEADS + head] * a.scale_log2;
    const int ka = n * kK8Stride + 16 * h;
    const int sw = p_swz(head & 15);
    float m_run = kNegInf, l_run = 0.f;
    q8_pipeline<Q8Stage<2, false, 3>>(a, sm, t, req, pos, tid, 512 + tid, [&](int j, int ntile, auto) {
      if (j < ntile) {
        const uint8_t* k8 = sm.k8[j & 1];
        auto aread = [&](int g) {
          return cat8(*reinterpret_cast<const u32x4*>(k8 + ka + 64 * g),
                      *reinterpret_cast<const u32x4*>(k8 + ka + 64 * g + 32));
        };
        // the nine scale exponents of row m (bytes 0..8)
        const u32x4 se = *reinterpret_cast<const u32x4*>(&sm.sc8[j & 1][n][0]);
        // acc[4q + jj] = score of row 8q + 4h + jj over the nine groups
        f32x16 acc = {};
        i32x8 af[2];
        af[0] = aread(0);
        dsa::static_for<kQ8Groups>([&](auto G) {
          constexpr int g = decltype(G)::value;
          if constexpr (g + 1 < kQ8Groups) af[(g + 1) & 1] = aread(g + 1);
          acc = mfma32x32x64_fp8<g & 3>(af[g & 1], qf[g], int(se[g >> 2]), acc);
        });
        // log2-domain scores (-inf on masked rows) and the tile max of the head
        float z[16];
        float tmax = kNegInf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(sm.bias + j * kTileQ8 + 8 * q + 4 * h);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            z[4 * q + jj] = fmaf(acc[4 * q + jj], cq, b[jj]);
            tmax = fmaxf(tmax, z[4 * q + jj]);
          }
        }
        tmax = halves_max(tmax);
        float alpha = 1.f;
        if (tmax > m_run + kRescaleThreshold) {
          if (m_run != kNegInf) alpha = __builtin_amdgcn_exp2f(m_run - tmax);
          l_run *= alpha;
          m_run = tmax;
        }
        const float neg_m = m_run == kNegInf ? 0.f : -m_run;
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(z[r] + neg_m);
          l_run += pr[r];
        }
        // PV operand position 8g' + 4e + jj holds row 16e + 4g' + jj: rows of
        // q = 0 and 2 fill chunk h of the head's P row, q = 1 and 3 chunk 2 + h
        uint16_t* prow = sm.p[j & 1] + head * kPStrideWS;
        *reinterpret_cast<u32x4*>(prow + 8 * (h ^ sw)) =
            u32x4{dsa::pack_bf16x2(pr[0], pr[1]), dsa::pack_bf16x2(pr[2], pr[3]),
                  dsa::pack_bf16x2(pr[8], pr[9]), dsa::pack_bf16x2(pr[10], pr[11])};
        *reinterpret_cast<u32x4*>(prow + 8 * ((2 + h) ^ sw)) =
            u32x4{dsa::pack_bf16x2(pr[4], pr[5]), dsa::pack_bf16x2(pr[6], pr[7]),
                  dsa::pack_bf16x2(pr[12], pr[13]), dsa::pack_bf16x2(pr[14], pr[15])};
        if (h == 0) sm.alpha[j & 1][head] = alpha;
        // one word per wave for the value waves: does PV of this tile start
        // with a rescale of O
        const bool any_resc = __any(alpha != 1.f);
        if (lane == 0) sm.resc[j & 1][wave] = any_resc;
      }
    });
    const float l = halves_sum(l_run);
    if (h == 0) {
      sm.fin_l[head] = l;
      put_lse<true>(a, t, head, l > 0.f ? (m_run + log2f(l)) * kLn2 : kNegInf);
    }
    __syncthreads();
  } else if (wave == 4 || wave == 5) {
    q8_value<4, Q8Stage<2, true, 3>>(a, sm, t, req, pos, tid, tid + 384, 192 + 64 * (wave - 4));
  } else {
    const int hw = wave < 4 ? wave - 2 : wave - 4;   // waves 2, 3, 6, 7 -> 0..3
    const int d0 = hw < 2 ? 96 * hw : 320 + 96 * (hw - 2);
    q8_value<6, Q8Stage<2, false, 1>>(a, sm, t, req, pos, tid, 64 * hw + lane, d0);
  }
}

// Tiles of 32 and of 128 index columns run the warp-specialized kernel: a
// 128-column tile (the plan's loop step and split granularity, Figure 4's
// virtual padding) is streamed through its three-deep ring as four 32-row LDS
// steps.  A kernel holding a whole 128-row bf16 tile (148 KB of the 160 KB
// LDS) had room for neither a second buffer nor more than four waves, spilled
// 85-98 registers and ran at a third of the tile-32 speed.
template <int KV, int TILE, bool kFinal>
hipError_t launch_partial(const PartialArgs& a, int T, int S, hipStream_t st) {
  if constexpr (TILE == kTileWS || TILE == 128)
    hipLaunchKernelGGL((partial_ws_kernel<KV, kFinal, ws_value_waves<KV>()>), dim3(T, S),
                       dim3((4 + ws_value_waves<KV>()) * 64), 0, st, a);
  else
    hipLaunchKernelGGL((partial_v2_kernel<KV, TILE, kFinal>), dim3(T, S), dim3(kThreadsV2), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one thread per (token, head, 8 columns).
// Part s of token t sits at slot t*ts + s*ss (token-major splits: ts = S,
// ss = 1; shard-major parts: ts = 1, ss = T).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int T,
                                                      int S, int64_t ts, int64_t ss,
                                                      uint16_t* __restrict__ out,
                                                      float* __restrict__ lse_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // token*64 + head
  if (row >= T * DSA_HEADS) return;
  const int lane = threadIdx.x & 63;
  const int t = row / DSA_HEADS, h = row % DSA_HEADS;
  // Splits are visited in groups of kU with every load of a group issued
  // before its arithmetic (a split's weight is exp(lse_s - m), 0 for an empty
  // split, so no branch depends on a loaded value); splits past S repeat the
  // last one with weight 0.  The sums run in split order.
  constexpr int kU = 8;
  auto lse_at = [&](int s) { return lse_part[(t * ts + int64_t(s) * ss) * DSA_HEADS + h]; };
  float m = kNegInf;
  for (int s0 = 0; s0 < S; s0 += kU) {
    float ls[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j) ls[j] = lse_at(min(s0 + j, S - 1));
#pragma unroll
    for (int j = 0; j < kU; ++j) m = fmaxf(m, ls[j]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != kNegInf) {
    for (int s0 = 0; s0 < S; s0 += kU) {
      float ls[kU];
      float4 x[kU][2];
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const int sj = min(s0 + j, S - 1);
        ls[j] = s0 + j < S ? lse_at(sj) : kNegInf;
        const float4* src = reinterpret_cast<const float4*>(
            o_part + ((t * ts + int64_t(sj) * ss) * DSA_HEADS + h) * DSA_D_LATENT + 8 * lane);
        x[j][0] = src[0];
        x[j][1] = src[1];
      }
#pragma unroll
      for (int j = 0; j < kU; ++j) {
        const float wgt = expf(ls[j] - m);   // exp(-inf) = 0: empty splits add nothing
        tot += wgt;
        acc[0] += wgt * x[j][0].x; acc[1] += wgt * x[j][0].y;
        acc[2] += wgt * x[j][0].z; acc[3] += wgt * x[j][0].w;
        acc[4] += wgt * x[j][1].x; acc[5] += wgt * x[j][1].y;
        acc[6] += wgt * x[j][1].z; acc[7] += wgt * x[j][1].w;
      }
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

// Validation and launch shared by the split form (o_part/lse_part) and the
// single-split form (out/lse).  `who` names the entry point in messages.
static dsa_status run_partial(const char* who, const dsa_pool* pool, const int32_t* page_table,
                              int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                              const int32_t* tok_pos, int32_t num_tokens, const uint16_t* q,
                              const int32_t* idx, int32_t width, float sm_scale, int32_t kv_tile,
                              int32_t num_splits, float* o_part, float* lse_part, uint16_t* out,
                              float* lse_out, void* stream) {
  const std::string w(who);
  const bool final_out = num_splits == 1 && (out != nullptr || lse_out != nullptr);
  dsa_status s = dsa::check_partial(who, pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos,
                                    num_tokens, q, idx, width, sm_scale, kv_tile, num_splits,
                                    final_out, final_out ? static_cast<const void*>(out) : o_part,
                                    final_out ? static_cast<const void*>(lse_out) : lse_part);
  if (s != DSA_OK) return s;
  if (num_tokens == 0) return dsa::ok();
  s = dsa::deep_check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens,
                            who, stream);
  if (s != DSA_OK) return s;
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
  a.q8 = nullptr;
  a.q8_scale = nullptr;
  a.idx = idx;
  a.width = width;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.cols_per_split = plan.cols_per_split;
  a.splits = num_splits;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.out = out;
  a.lse_out = lse_out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fp8 = pool->kv_dtype == DSA_KV_FP8_E4M3_S64;
  auto launch = [&](auto tile_c, auto final_c) -> hipError_t {
    constexpr int TILE = decltype(tile_c)::value;
    constexpr bool FIN = decltype(final_c)::value;
    return fp8 ? launch_partial<DSA_KV_FP8_E4M3_S64, TILE, FIN>(a, num_tokens, num_splits, st)
               : launch_partial<DSA_KV_BF16, TILE, FIN>(a, num_tokens, num_splits, st);
  };
  using T32 = std::integral_constant<int, 32>;
  using T64 = std::integral_constant<int, 64>;
  using T128 = std::integral_constant<int, 128>;
  hipError_t e;
  if (final_out) {
    if (kv_tile == 32) e = launch(T32{}, std::true_type{});
    else if (kv_tile == 64) e = launch(T64{}, std::true_type{});
    else e = launch(T128{}, std::true_type{});
  } else {
    if (kv_tile == 32) e = launch(T32{}, std::false_type{});
    else if (kv_tile == 64) e = launch(T64{}, std::false_type{});
    else e = launch(T128{}, std::false_type{});
  }
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, w + ": launch failed: " + hipGetErrorString(e));
  return dsa::ok();
}

extern "C" dsa_status dsa_sparse_mla_partial(const dsa_pool* pool, const int32_t* page_table,
                                             int32_t pt_stride, const int32_t* q_offsets,
                                             int32_t num_reqs, const int32_t* tok_pos,
                                             int32_t num_tokens, const uint16_t* q,
                                             const int32_t* idx, int32_t width, float sm_scale,
                                             int32_t kv_tile, int32_t num_splits, float* o_part,
                                             float* lse_part, void* stream) {
  return run_partial("dsa_sparse_mla_partial", pool, page_table, pt_stride, q_offsets, num_reqs,
                     tok_pos, num_tokens, q, idx, width, sm_scale, kv_tile, num_splits, o_part,
                     lse_part, nullptr, nullptr, stream);
}

extern "C" dsa_status dsa_sparse_mla(const dsa_pool* pool, const int32_t* page_table,
                                     int32_t pt_stride, const int32_t* q_offsets, int32_t num_reqs,
                                     const int32_t* tok_pos, int32_t num_tokens, const uint16_t* q,
                                     const int32_t* idx, int32_t width, float sm_scale,
                                     int32_t kv_tile, uint16_t* out, float* lse, void* stream) {
  return run_partial("dsa_sparse_mla", pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos,
                     num_tokens, q, idx, width, sm_scale, kv_tile, 1, nullptr, nullptr, out, lse,
                     stream);
}

extern "C" dsa_status dsa_sparse_mla_q8(const dsa_pool* pool, const int32_t* page_table,
                                        int32_t pt_stride, const int32_t* q_offsets,
                                        int32_t num_reqs, const int32_t* tok_pos,
                                        int32_t num_tokens, const uint8_t* q_codes,
                                        const float* q_scales, const int32_t* idx, int32_t width,
                                        float sm_scale, uint16_t* out, float* lse, void* stream) {
  const char* who = "dsa_sparse_mla_q8";
  dsa_status s = dsa::check_sparse_mla_q8(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos,
                                          num_tokens, q_codes, q_scales, idx, width, sm_scale, out,
                                          lse);
  if (s != DSA_OK) return s;
  if (num_tokens == 0) return dsa::ok();
  s = dsa::deep_check_batch(pool, page_table, pt_stride, q_offsets, num_reqs, tok_pos, num_tokens,
                            who, stream);
  if (s != DSA_OK) return s;
  PartialArgs a;
  a.latent = reinterpret_cast<const uint8_t*>(pool->base + pool->layout.latent_plane_offset);
  a.num_pages = pool->num_pages;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.q_offsets = q_offsets;
  a.num_reqs = num_reqs;
  a.tok_pos = tok_pos;
  a.q = nullptr;
  a.q8 = q_codes;
  a.q8_scale = q_scales;
  a.idx = idx;
  a.width = width;
  a.scale_log2 = sm_scale * 1.44269504088896340736f;
  a.cols_per_split = width;
  a.splits = 1;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.out = out;
  a.lse_out = lse;
  hipLaunchKernelGGL(partial_q8_kernel, dim3(unsigned(num_tokens)), dim3(kThreadsV2), 0,
                     static_cast<hipStream_t>(stream), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
  return dsa::ok();
}

static dsa_status run_combine(const char* who, const float* o_part, const float* lse_part,
                              int32_t num_tokens, int32_t parts, bool shard_major, uint16_t* out,
                              float* lse, void* stream) {
  const std::string w(who);
  const dsa_status s = dsa::check_combine(who, o_part, lse_part, num_tokens, parts, out, lse);
  if (s != DSA_OK || num_tokens == 0) return s == DSA_OK ? dsa::ok() : s;
  const int64_t rows = int64_t(num_tokens) * DSA_HEADS;
  const int64_t ts = shard_major ? 1 : parts, ss = shard_major ? num_tokens : 1;
  hipLaunchKernelGGL(combine_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), o_part, lse_part, num_tokens, parts, ts, ss,
                     out, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return dsa::fail(DSA_ERR_HIP, w + ": launch failed: " + hipGetErrorString(e));
  return dsa::ok();
}

extern "C" dsa_status dsa_combine(const float* o_part, const float* lse_part, int32_t num_tokens,
                                  int32_t num_splits, uint16_t* out, float* lse, void* stream) {
  return run_combine("dsa_combine", o_part, lse_part, num_tokens, num_splits, false, out, lse,
                     stream);
}

extern "C" dsa_status dsa_combine_shards(const float* o_part, const float* lse_part,
                                         int32_t num_tokens, int32_t num_shards, uint16_t* out,
                                         float* lse, void* stream) {
  return run_combine("dsa_combine_shards", o_part, lse_part, num_tokens, num_shards, true, out, lse,
                     stream);
}
