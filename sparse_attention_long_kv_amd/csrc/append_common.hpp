// Appending one token's row to a (b, KV head) unit: the bf16 K/V copies and
// the FP8 projected key, as one workgroup's work.  Shared by the append
// kernel and the fused decode-step prologue so both write the same bytes.
//
// Projection order: the d products of column j are split into 8 parts of d/8
// consecutive rows of P; each part is a fused multiply-add chain in fp64 from
// +0 (every product bf16 x fp32 is exact in fp64); the parts are added in
// order to +0 and the total is rounded once to E4M3 (nearest-even,
// saturating).  JSSA article (rit.work blog), "How JSSA preserves token
// order": each key's low-rank projection is stored as FP8 beside the cache.
#pragma once

#include "device_common.hpp"

namespace sa {

constexpr int kProjParts = 8;

// Threads [0, 8R) form the partial sums; `part` holds 8R doubles of LDS.
// Every thread of the workgroup must call this (it synchronises once).
// Returns after the row and its code are stored.
template <int D, int R>
__device__ __forceinline__ void append_row(const uint16_t* __restrict__ kr,
                                           const uint16_t* __restrict__ vr,
                                           const float* __restrict__ Ph, size_t row_off,
                                           uint16_t* __restrict__ k_cache,
                                           uint16_t* __restrict__ v_cache,
                                           uint8_t* __restrict__ kp_row, double* part) {
  constexpr int kPer = D / kProjParts;
  const int t = threadIdx.x;
  // bf16 row copies: D/8 threads move 16 bytes of K and of V each
  if (t < D / 8) {
    const size_t off = row_off * D + t * 8;
    *reinterpret_cast<uint4*>(k_cache + off) = *reinterpret_cast<const uint4*>(kr + t * 8);
    *reinterpret_cast<uint4*>(v_cache + off) = *reinterpret_cast<const uint4*>(vr + t * 8);
  }
  const int p = t / R, j = t % R;
  if (t < kProjParts * R) {
    const float* pc = Ph + (size_t)p * kPer * R + j;
    float pv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) pv[k] = pc[k * R];
    float kv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k += 8)
      bf16x8_to_f32(*reinterpret_cast<const uint4*>(kr + p * kPer + k), kv + k);
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc = fma((double)kv[k], (double)pv[k], acc);
    part[t] = acc;
  }
  __syncthreads();
  if (t < R) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kProjParts; ++q) s += part[q * R + t];
    kp_row[t] = (uint8_t)f64_to_e4m3(s);
  }
}

}  // namespace sa
