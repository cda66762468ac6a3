// Device helpers shared by the gfx950 kernels: bf16/FP8 conversions, DPP
// row reductions, order-preserving score keys and workgroup scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 values packed in a uint4 -> 8 floats (exact)
__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- FP8 E4M3

// Four OCP E4M3 codes (one per byte, byte 0 first) -> four floats, exact.
// gfx950's packed conversion reads the OCP "fn" encoding.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0]; f[1] = lo[1]; f[2] = hi[0]; f[3] = hi[1];
}

// float64 -> OCP E4M3 code, round to nearest even, saturating to +-448.
// The code's sign is the sign bit of x.  Every step is exact in fp64.
__device__ __forceinline__ uint32_t f64_to_e4m3(double x) {
  const uint32_t sign = signbit(x) ? 0x80u : 0u;
  const double a = fabs(x);
  if (!(a < 448.0)) return sign | 0x7Eu;            // saturate (and NaN)
  if (a < 0x1p-6) {                                  // subnormal: m * 2^-9
    return sign | (uint32_t)rint(a * 512.0);         // m <= 8; 8 == 2^-6 code
  }
  int e;
  const double f = frexp(a, &e);                     // a = f * 2^e, f in [0.5,1)
  int biased = e - 1 + 7;
  int q = (int)rint((2.0 * f - 1.0) * 8.0);          // 0..8
  if (q == 8) { q = 0; biased += 1; }
  if (biased > 15 || (biased == 15 && q == 7)) return sign | 0x7Eu;
  return sign | (uint32_t)(biased << 3) | (uint32_t)q;
}

// ---------------------------------------------------------------- buffer loads

// Raw buffer resource over [base, base + bytes): loads whose lane offset is at
// or past `bytes` return zero (hardware range check over the vector and
// immediate offsets; callers pass the whole offset in the lane offset and 0 as
// the scalar one), so tails and padding need no clamping or branches.
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped) 32-bit element format
typedef unsigned int sa_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  const sa_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- DPP sums

// DPP control words (gfx9 encoding)
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

constexpr int kDppRowShr = 0x110;     // row_shr:n = kDppRowShr + n (n = 1 .. 15)
constexpr int kDppRowBcast15 = 0x142; // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143; // lane 31 to rows 2 and 3

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// x moved by DPP control CTRL; rows outside ROW_MASK keep `old`, and with
// ZERO a lane whose source lies outside its row reads 0.
template <int CTRL, int ROW_MASK, bool ZERO>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, ZERO);
}

// Sum over aligned groups of W lanes (W in 2, 4, 8, 16); every lane of the
// group receives the same bits (the pairings are symmetric).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
  x = x + dpp_f<kDppQuadSwap1>(x);
  if (W >= 4) x = x + dpp_f<kDppQuadSwap2>(x);
  if (W >= 8) x = x + dpp_f<kDppHalfMirror>(x);
  if (W >= 16) x = x + dpp_f<kDppMirror>(x);
  return x;
}

// ---------------------------------------------------------------- keys

// Order-preserving map fp32 score -> uint32 (larger score, larger key).
// Key 0 is reserved for "no position"; the one float that would map to it
// (a negative NaN with every payload bit set) is moved to 1.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k == 0u ? 1u : k;
}

// The score a key stands for (inverse of score_key on keys >= 2).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---------------------------------------------------------------- lanes

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __builtin_popcountll(m); }

// Inclusive prefix sum across the 64 lanes of a wave (uint32).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  // Hillis-Steele shifts inside each 16-lane row, then every row adds the
  // totals of the rows below it (row broadcasts): six DPP adds, no LDS trips
  x += dpp_u32<kDppRowShr + 1, 0xF, true>(0u, x);
  x += dpp_u32<kDppRowShr + 2, 0xF, true>(0u, x);
  x += dpp_u32<kDppRowShr + 4, 0xF, true>(0u, x);
  x += dpp_u32<kDppRowShr + 8, 0xF, true>(0u, x);
  x += dpp_u32<kDppRowBcast15, 0xA, false>(0u, x);   // rows 1, 3 += lane 15 of rows 0, 2
  x += dpp_u32<kDppRowBcast31, 0xC, false>(0u, x);   // rows 2, 3 += lane 31
  return x;
}

// Largest value over the wave (every lane receives it): the scan's steps
// with max (0 is the identity), then lane 63's result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<kDppRowShr + 1, 0xF, true>(0u, x));
  x = max(x, dpp_u32<kDppRowShr + 2, 0xF, true>(0u, x));
  x = max(x, dpp_u32<kDppRowShr + 4, 0xF, true>(0u, x));
  x = max(x, dpp_u32<kDppRowShr + 8, 0xF, true>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast15, 0xA, false>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast31, 0xC, false>(0u, x));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// Sum across a wave (every lane receives it).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

}  // namespace sa
