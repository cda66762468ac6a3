// Gather-free sparse attention over the selected rows of the bf16 KV cache:
// the attention kernel (selected rows read from idx) and the cross-workgroup
// merge of split states.  The per-workgroup machinery, with its layout and
// the pages it follows, is in attend_common.hpp.
#include "attend_common.hpp"
#include "kernels.h"

namespace sa {

// Dynamic LDS: the waves' output tiles, [waves][G][D] floats.
template <int D>
__global__ __launch_bounds__(kAttendThreads) void decode_kernel(const DecodeArgs a) {
  constexpr int W = kAttendWaves;
  constexpr int NT = kAttendThreads;
  static_assert(kDecodeIdxTile % (16 * W) == 0, "staged runs keep the tile -> wave assignment");
  __shared__ float sm[W][kMaxHeads], sl[W][kMaxHeads];
  __shared__ int32_t sidx[kDecodeIdxTile];
  extern __shared__ float so[];       // [W][G][D]

  const int u = blockIdx.x / a.S, split = blockIdx.x % a.S;
  AttendWave<D, W> aw;
  aw.init(a, u);
  const int r0 = split * a.rps;
  const int r1 = min(a.M, r0 + a.rps);
  const int32_t* idx_u = a.idx + (size_t)u * a.M;
  for (int t0 = r0; t0 < r1; t0 += kDecodeIdxTile) {
    const int cnt = min(r1 - t0, kDecodeIdxTile);
    __syncthreads();
    for (int j = threadIdx.x; j < cnt; j += NT) sidx[j] = idx_u[t0 + j];
    __syncthreads();
    aw.rows(a, sidx, cnt);
  }
  aw.finish(a, u, split, sm, sl, so);
}

// Merge the S partial states of one unit (one workgroup per unit).  A separate
// launch orders the partial writes before these reads without device-scope
// fences inside the attention kernel.
template <int D>
__global__ __launch_bounds__(kBlock) void combine_kernel(const DecodeArgs a) {
  __shared__ float fm[kMaxHeads], fl[kMaxHeads];
  const int G = a.G;
  const int u = blockIdx.x;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x;
  const size_t ubase = (size_t)u * a.S * G;
  if (tid < G) {
    const int g = tid;
    float mt = -__builtin_inff();
    for (int s2 = 0; s2 < a.S; ++s2) mt = fmaxf(mt, a.pm[ubase + (size_t)s2 * G + g]);
    float lt = 0.0f;
    for (int s2 = 0; s2 < a.S; ++s2)
      lt += a.pl[ubase + (size_t)s2 * G + g] * merge_scale(a.pm[ubase + (size_t)s2 * G + g], mt);
    fm[g] = mt;
    fl[g] = lt;
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += kBlock) {
    const int g = t / D, dd = t % D;
    const float mt = fm[g], lt = fl[g];
    float ot = 0.0f;
    for (int s2 = 0; s2 < a.S; ++s2) {
      const size_t pi = ubase + (size_t)s2 * G + g;
      ot += a.po[pi * D + dd] * merge_scale(a.pm[pi], mt);
    }
    const int hq = h * G + g;
    const float val = lt > 0.0f ? ot / lt : 0.0f;
    a.out[((size_t)b * a.Hq + hq) * D + dd] = (uint16_t)f32_to_bf16_bits(val);
    if (dd == 0 && a.lse)
      a.lse[(size_t)b * a.Hq + hq] =
          lt > 0.0f ? (mt + log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

template <int D>
static void launch_decode_d(const DecodeArgs& a, dim3 grid, int units, hipStream_t st) {
  const size_t lds = (size_t)kAttendWaves * a.G * D * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<D>), grid, dim3(kAttendThreads), lds, st, a);
  if (a.S > 1) hipLaunchKernelGGL((combine_kernel<D>), dim3(units), dim3(kBlock), 0, st, a);
}

hipError_t run_combine(const LaunchCommon& c, const DecodeArgs& a) {
  if (a.S <= 1) return hipSuccess;
  if (c.D == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3(c.units), dim3(kBlock), 0, c.stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<64>), dim3(c.units), dim3(kBlock), 0, c.stream, a);
  return hipGetLastError();
}

hipError_t run_decode(const LaunchCommon& c, const DecodePlan& plan, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* idx, int M,
                      float scale, void* out, float* lse, void* workspace) {
  DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.idx = idx;
  a.M = M;
  a.Ncap = c.Ncap;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.G = c.G;
  a.S = plan.splits;
  a.rps = plan.rows_per_split;
  a.qscale = scale * 1.4426950408889634f;
  a.out = (uint16_t*)out;
  a.lse = lse;
  char* ws = (char*)workspace;
  a.pm = (float*)(ws + plan.off_m);
  a.pl = (float*)(ws + plan.off_l);
  a.po = (float*)(ws + plan.off_o);
  const long blocks = (long)plan.units * plan.splits;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (c.G < 1 || c.G > kMaxHeads) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (c.D == 128) launch_decode_d<128>(a, grid, plan.units, c.stream);
  else launch_decode_d<64>(a, grid, plan.units, c.stream);
  return hipGetLastError();
}

}  // namespace sa
