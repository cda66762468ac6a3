// Projected-key cache: append of new tokens and bulk (re)projection of cached
// keys.  kp[n][j] = e4m3(sum_i k[n][i] * P[h][i][j]) with the sum in fp64.
//
// JSSA article (rit.work blog, Joint Subspace Sparse Attention), "How JSSA
// preserves token order": each key has a low-rank projection onto its KV
// head's basis, kept as FP8 next to the bf16 cache.
//
// Summation order (shared by both kernels, so a row's code is the same
// whichever kernel wrote it): the d products of column j are split into 8
// parts of d/8 consecutive rows of P; each part is a fused multiply-add chain
// in fp64 starting from +0 (every product bf16 x fp32 is exact in fp64); the
// parts are added in order to +0, and the total is rounded once to E4M3.
//
// Append (the decode hot path, one row per (b, KV head) per token) is latency
// bound, so one workgroup serves one new row: 8 parts x r columns of threads
// each form one partial sum straight from global memory, and the row's bf16
// K/V copies go out in parallel.  The bulk projection stages key rows in LDS
// and lets one lane form one code from all 8 parts.
#include "append_common.hpp"
#include "kernels.h"

namespace sa {

// ---------------------------------------------------------------- append

template <int D, int R>
__global__ __launch_bounds__(kBlock) void append_kv_kernel(
    const int32_t* __restrict__ pos, int T, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const float* __restrict__ P, int Hkv, int Ncap,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, uint8_t* __restrict__ kp) {
  static_assert(kProjParts * R <= kBlock, "one thread per (part, column)");
  __shared__ double part[kProjParts * R];
  const int u = blockIdx.x / T, tok = blockIdx.x % T;
  const int b = u / Hkv, h = u % Hkv;
  const long n = (long)pos[b] + tok;
  if (n < 0 || n >= Ncap) return;                    // block-uniform
  const size_t row = (size_t)u * Ncap + n;
  append_row<D, R>(k_new + ((size_t)u * T + tok) * D, v_new + ((size_t)u * T + tok) * D,
                   P + (size_t)h * D * R, row, k_cache, v_cache, kp + row * R, part);
}

// ---------------------------------------------------------------- bulk

template <int D, int R>
struct ProjGeom {
  static constexpr int kRowsPerWavePass = kWave / R;          // 2 (r=32) or 4 (r=16)
  static constexpr int kRowsPerPass = 4 * kRowsPerWavePass;   // per workgroup
};

template <int D, int R>
__device__ __forceinline__ void load_basis(const float* __restrict__ P, int h, float* Ps) {
  const float* src = P + (size_t)h * D * R;
  for (int i = threadIdx.x; i < D * R; i += blockDim.x) Ps[i] = src[i];
}

// Stage one bf16 key row (D values) into LDS as fp32; D/8 lanes cooperate.
template <int D>
__device__ __forceinline__ void stage_row(const uint16_t* __restrict__ src, float* dst, int sub) {
  if (sub < D / 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + sub * 8);
    float f[8];
    bf16x8_to_f32(v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[sub * 8 + e] = f[e];
  }
}

// One code from a staged row, in the shared summation order.
template <int D, int R>
__device__ __forceinline__ uint32_t project_one(const float* krow, const float* Ps, int j) {
  constexpr int kPer = D / kProjParts;
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kProjParts; ++q) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = q * kPer + k;
      acc = fma((double)krow[i], (double)Ps[i * R + j], acc);
    }
    s += acc;
  }
  return f64_to_e4m3(s);
}

constexpr int kPassesPerBlock = 8;

template <int D, int R>
__global__ __launch_bounds__(kBlock) void project_keys_kernel(
    const uint16_t* __restrict__ k_cache, const float* __restrict__ P, int Hkv,
    int Ncap, int n_begin, int n_count, int blocks_per_unit, uint8_t* __restrict__ kp) {
  using Geo = ProjGeom<D, R>;
  __shared__ float Ps[D * R];
  __shared__ float Ks[Geo::kRowsPerPass][D];
  const int u = blockIdx.x / blocks_per_unit;
  const int rb = blockIdx.x % blocks_per_unit;
  const int h = u % Hkv;
  load_basis<D, R>(P, h, Ps);
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int rr = lane / R, j = lane % R;
  const int n_end = n_begin + n_count;
  const uint16_t* ku = k_cache + (size_t)u * Ncap * D;
  uint8_t* kpu = kp + (size_t)u * Ncap * R;
  for (int pass = 0; pass < kPassesPerBlock; ++pass) {
    const int row0 = n_begin + (rb * kPassesPerBlock + pass) * Geo::kRowsPerPass;
    if (row0 >= n_end) break;                         // uniform across the block
    __syncthreads();                                  // Ks reuse / Ps ready
    // stage rows: thread t -> row t / (D/8), 16-byte piece t % (D/8)
    {
      constexpr int kPieces = D / 8;
      const int t = threadIdx.x;
      const int row = t / kPieces, piece = t % kPieces;
      if (row < Geo::kRowsPerPass) {
        const int n = row0 + row;
        if (n < n_end) stage_row<D>(ku + (size_t)n * D, Ks[row], piece);
      }
    }
    __syncthreads();
    const int row = w * Geo::kRowsPerWavePass + rr;
    const int n = row0 + row;
    if (n < n_end) kpu[(size_t)n * R + j] = (uint8_t)project_one<D, R>(Ks[row], Ps, j);
  }
}

template <int D, int R>
static hipError_t launch_project(const LaunchCommon& c, const void* k_cache, const float* P,
                                 int n_begin, int n_count, uint8_t* kp) {
  using Geo = ProjGeom<D, R>;
  const int rows_per_block = Geo::kRowsPerPass * kPassesPerBlock;
  const int bpu = (n_count + rows_per_block - 1) / rows_per_block;
  const long blocks = (long)bpu * c.units;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((project_keys_kernel<D, R>), dim3((unsigned)blocks), dim3(kBlock), 0,
                     c.stream, (const uint16_t*)k_cache, P, c.Hkv, c.Ncap, n_begin, n_count,
                     bpu, kp);
  return hipGetLastError();
}

template <int D, int R>
static hipError_t launch_append(const LaunchCommon& c, const int32_t* pos, int T,
                                const void* k_new, const void* v_new, const float* P,
                                void* k_cache, void* v_cache, uint8_t* kp) {
  const long blocks = (long)T * c.units;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((append_kv_kernel<D, R>), dim3((unsigned)blocks), dim3(kBlock), 0, c.stream,
                     pos, T, (const uint16_t*)k_new, (const uint16_t*)v_new, P, c.Hkv, c.Ncap,
                     (uint16_t*)k_cache, (uint16_t*)v_cache, kp);
  return hipGetLastError();
}

hipError_t run_project_keys(const LaunchCommon& c, const void* k_cache, const float* P,
                            int n_begin, int n_count, uint8_t* kp) {
  if (n_count <= 0) return hipSuccess;
  if (c.D == 128 && c.R == 32) return launch_project<128, 32>(c, k_cache, P, n_begin, n_count, kp);
  if (c.D == 128 && c.R == 16) return launch_project<128, 16>(c, k_cache, P, n_begin, n_count, kp);
  if (c.D == 64 && c.R == 32) return launch_project<64, 32>(c, k_cache, P, n_begin, n_count, kp);
  return launch_project<64, 16>(c, k_cache, P, n_begin, n_count, kp);
}

hipError_t run_append_kv(const LaunchCommon& c, const int32_t* pos, int T, const void* k_new,
                         const void* v_new, const float* P, void* k_cache, void* v_cache,
                         uint8_t* kp) {
  if (T <= 0) return hipSuccess;
  if (c.D == 128 && c.R == 32)
    return launch_append<128, 32>(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp);
  if (c.D == 128 && c.R == 16)
    return launch_append<128, 16>(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp);
  if (c.D == 64 && c.R == 32)
    return launch_append<64, 32>(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp);
  return launch_append<64, 16>(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp);
}

}  // namespace sa
