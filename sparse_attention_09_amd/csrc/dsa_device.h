// Device-side helpers for the gfx950 kernels: vector types, MFMA wrappers and
// small conversions.  CDNA4 only (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) + i] and B[8*(l/16) + i][l%16], i = 0..7,
// and holds D[4*(l/16) + j][l%16], j = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Four OCP E4M3FN codes (one dword) -> four fp32 values (exact conversion).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t codes, float out[4]) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Nearest E4M3FN code of a finite fp32 value (ties to even, |y| saturated at
// 448, sign from y), with integer operations on the fp32 bits: exact and
// independent of any hardware conversion mode.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.f);
  uint32_t code;
  if (a < 0.015625f) {
    // below 2^-6 the grid is the subnormals, step 2^-9: a*512 is exact and
    // rint rounds half to even (8 is the smallest normal, code 0x08)
    code = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const uint32_t bits = __float_as_uint(a);
    const uint32_t e = (bits >> 23) - 127u + 7u;   // biased E4M3 exponent, 1..15
    const uint32_t m = bits & 0x7FFFFFu;
    const uint32_t m3 = m >> 20, rem = m & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ? 1u : 0u;
    code = min((e << 3) + m3 + up, 0x7Eu);       // a mantissa carry moves up the exponent
  }
  return sign | code;
}

// FP8 cache group scale: the smallest power of two 2^k (k >= -126) with
// amax <= 448 * 2^k, 1 for amax = 0.  Exact: amax = 1.f * 2^e, and
// 448 * 2^k = 1.75 * 2^(k+8) reaches it at k = e - 8 when f <= 1.75, else
// at k = e - 7.
__device__ __forceinline__ float fp8_group_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const uint32_t b = __float_as_uint(amax);
  const int k = max(int(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0), -126);
  return __uint_as_float(uint32_t(k + 127) << 23);
}

// Lane index (0..63) computed where it is called.  The asm is volatile, so
// two calls are never merged: a value derived from it is recomputed in a loop
// body instead of being held in a register through the loop.
__device__ __forceinline__ int fresh_lane() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// Max / sum over lanes i, i^16, i^32, i^48 (the four 16-lane rows of a
// wave), every lane receiving the result: v_permlane32_swap then
// v_permlane16_swap each pair a lane with its partner in one VALU op (no LDS
// round trip, unlike ds_bpermute).  Both combines commute, so all four lanes
// hold the same bits.
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Indexer epilogue of one 16-position MFMA block (acc holds heads 4g..4g+3 of
// position lane%16, g = lane/16): relu, head weights and the sum over all 16
// heads.  Every lane receives the score of position lane%16; the order of the
// additions is fixed, so every kernel using this gets the same bits.  relu is
// a signed-integer max with 0 on the float bits (one op; -0 and negative
// values give +0; NaN inputs are unsupported).
__device__ __forceinline__ float index_score(const f32x4& acc, const float (&w)[4]) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s = fmaf(w[j], __int_as_float(max(__float_as_int(acc[j]), 0)), s);
  return rows4_sum(s);
}

// The same for two tokens' blocks at once: lanes 0..31 receive token A's score
// of position lane%16, lanes 32..63 token B's.  One permlane32 swap pairs A's
// groups 0+2 / 1+3 in the low half and B's in the high half, one permlane16
// swap adds the pairs: the additions are those of index_score, in the same
// order, so each token's bits equal index_score's.
__device__ __forceinline__ float index_score2(const f32x4& accA, const float (&wA)[4],
                                              const f32x4& accB, const float (&wB)[4]) {
  float a = 0.f, b = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a = fmaf(wA[j], __int_as_float(max(__float_as_int(accA[j]), 0)), a);
    b = fmaf(wB[j], __int_as_float(max(__float_as_int(accB[j]), 0)), b);
  }
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

}  // namespace dsa
