// LISA-style gated linear-attention branch (one new token).
//
// LISA news items (aikraft.ru "LISA architecture"; opennieuws.be "Hybrid
// architecture for efficiency"): a linear-attention module gives long-term
// memory in linear time, and a gating mechanism merges it with the sparse
// branch.  With phi(x) = x + 1 (x > 0), exp(x) (x <= 0):
//   S += phi(k) v^T,  z += phi(k)                      (update_state != 0)
//   o_lin = (phi(q)^T S) / (phi(q)^T z),  g = sigmoid(w . q)
//   out = g * o_sparse + (1 - g) * o_lin
// An empty memory (phi(q)^T z = 0: with phi > 0 and z a sum of phi values,
// no token was ever added) reads out o_lin = 0 instead of 0 / 0.
// One 1024-thread workgroup per (batch row, KV head).  Thread (row block rb,
// column j) holds rows rb*RPT .. rb*RPT + RPT - 1 of column j of S: it issues
// all of their loads first, then updates and writes them back and forms each
// head's numerator over them in row order; the row blocks' partial
// numerators are then added in block order.  Denominators and gates
// are fixed-order sums over d formed while the loads are in flight.
#include "device_common.hpp"
#include "kernels.h"

namespace sa {

__device__ __forceinline__ float phi(float x) { return x > 0.0f ? x + 1.0f : expf(x); }

__device__ __forceinline__ float bf16_at(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

constexpr int kGateThreads = 1024;

template <int D, int G>
__global__ __launch_bounds__(kGateThreads) void linear_gate_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, float* __restrict__ S, float* __restrict__ z,
    const float* __restrict__ w_gate, const uint16_t* __restrict__ o_sparse,
    uint16_t* __restrict__ out, int Hq, int Hkv, int update) {
  constexpr int NT = kGateThreads;
  constexpr int RB = NT / D;                    // row blocks: 8 (d = 128) or 16 (d = 64)
  constexpr int RPT = D / RB;                   // rows per thread: 16 or 4
  __shared__ float phk[D], vn[D], zs[D];
  __shared__ float phq[G][D];
  __shared__ float num[RB][G][D];
  __shared__ float den[G], gate[G];

  const int u = blockIdx.x;
  const int b = u / Hkv, h = u % Hkv;
  const int tid = threadIdx.x;
  const int j = tid % D, rb = tid / D;
  const uint16_t* qb = q + ((size_t)b * Hq + (size_t)h * G) * D;
  float* Su = S + (size_t)u * D * D;

  float sv[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) sv[r] = Su[(size_t)(rb * RPT + r) * D + j];
  float* zu = z + (size_t)u * D;
  if (tid < D) {
    const float pk = phi(bf16_at(k_new, (size_t)u * D + tid));
    phk[tid] = pk;
    vn[tid] = bf16_at(v_new, (size_t)u * D + tid);
    float zi = zu[tid];
    if (update) {
      zi = zi + pk;
      zu[tid] = zi;
    }
    zs[tid] = zi;
  }
  for (int t = tid; t < G * D; t += NT) phq[t / D][t % D] = phi(bf16_at(qb, t));
  __syncthreads();

  if (tid < G) {                                // denominators, one thread per head
    float dsum = 0.0f;
    for (int i = 0; i < D; ++i) dsum = __builtin_fmaf(phq[tid][i], zs[i], dsum);
    den[tid] = dsum;
  } else if (tid >= 64 && tid < 64 + G) {       // gates
    const int g = tid - 64;
    const float* wg = w_gate + (size_t)(h * G + g) * D;
    float x = 0.0f;
    for (int i = 0; i < D; ++i) x = __builtin_fmaf(wg[i], bf16_at(qb, (size_t)g * D + i), x);
    gate[g] = 1.0f / (1.0f + expf(-x));
  }
  if (update) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = rb * RPT + r;
      sv[r] = __builtin_fmaf(phk[i], vn[j], sv[r]);
      Su[(size_t)i * D + j] = sv[r];
    }
  }
  // one head at a time (its rows in order), so only the rows stay in registers
#pragma unroll 1
  for (int g = 0; g < G; ++g) {
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) acc = __builtin_fmaf(phq[g][rb * RPT + r], sv[r], acc);
    num[rb][g][j] = acc;
  }
  __syncthreads();

  for (int t = tid; t < G * D; t += NT) {
    const int g = t / D, jj = t % D;
    float nsum = 0.0f;
#pragma unroll
    for (int r = 0; r < RB; ++r) nsum += num[r][g][jj];
    const float olin = den[g] != 0.0f ? nsum / den[g] : 0.0f;
    const size_t oi = ((size_t)b * Hq + (size_t)h * G + g) * D + jj;
    const float osp = bf16_at(o_sparse, oi);
    const float gg = gate[g];
    out[oi] = (uint16_t)f32_to_bf16_bits(gg * osp + (1.0f - gg) * olin);
  }
}

template <int D>
static void launch_lin_d(const LaunchCommon& c, const void* q, const void* k_new,
                         const void* v_new, float* S, float* z, const float* w,
                         const void* o_sp, void* out, int update) {
  const dim3 grid(c.units), block(kGateThreads);
  switch (c.G) {
#define SA_CASE(GG)                                                                        \
  case GG:                                                                                 \
    hipLaunchKernelGGL((linear_gate_kernel<D, GG>), grid, block, 0, c.stream,             \
                       (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new, \
                       S, z, w, (const uint16_t*)o_sp, (uint16_t*)out, c.Hq, c.Hkv, update); \
    break;
    SA_CASE(1) SA_CASE(2) SA_CASE(3) SA_CASE(4) SA_CASE(5) SA_CASE(6) SA_CASE(7) SA_CASE(8)
    SA_CASE(9) SA_CASE(10) SA_CASE(11) SA_CASE(12) SA_CASE(13) SA_CASE(14) SA_CASE(15)
    SA_CASE(16)
#undef SA_CASE
    default: break;
  }
}

hipError_t run_linear_gate(const LaunchCommon& c, const void* q, const void* k_new,
                           const void* v_new, float* S, float* z, const float* w_gate,
                           const void* o_sparse, void* out, int update_state) {
  if (c.D == 128) launch_lin_d<128>(c, q, k_new, v_new, S, z, w_gate, o_sparse, out, update_state);
  else launch_lin_d<64>(c, q, k_new, v_new, S, z, w_gate, o_sparse, out, update_state);
  return hipGetLastError();
}

}  // namespace sa
