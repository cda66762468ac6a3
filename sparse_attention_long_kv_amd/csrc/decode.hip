// Gather-free sparse attention over the selected rows of the bf16 KV cache.
//
// JSSA article (rit.work blog, Joint Subspace Sparse Attention), "How JSSA
// preserves token order": the final attention uses the original full-size
// keys and values of the selected positions; a dedicated kernel reads them
// directly from the cache, builds no contiguous intermediate buffer, and
// serves every head's own index set in one launch.  "Why token selection is
// not enough" explains why: the copy into such a buffer ate more than half of
// the remaining sparse-attention time at large batch.
//
// Layout.  A (batch row, KV head) unit's M selected rows are split over S
// workgroups ("split-K").  Inside a workgroup, a group of d/8 lanes owns one
// row at a time: each lane loads 16 bytes (8 bf16) of the K row and of the V
// row straight from the cache, so one wave instruction fetches whole 256-byte
// (d=128) rows.  The G queries of the GQA group stay in registers, pre-scaled
// by softmax_scale * log2(e).  Logits are reduced across the row's lanes with
// DPP; each lane group keeps its own online-softmax state (m, l, o) in the
// base-2 domain.  States merge across lane groups, waves and finally across
// the S workgroups with the log-sum-exp rule
//   m = max m_s,  l = sum l_s 2^(m_s - m),  o = sum o_s 2^(m_s - m) / l,
// the cross-workgroup merge being a small second launch (none when S = 1).
#include "device_common.hpp"
#include "kernels.h"

namespace sa {

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  int M, Ncap, Hq, Hkv, S, rps;
  float qscale;        // softmax_scale * log2(e)
  uint16_t* out;
  float* lse;
  float* pm;
  float* pl;
  float* po;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, l) merge weights of two base-2 states; -inf states weigh 0.
__device__ __forceinline__ float merge_scale(float m_part, float m_tot) {
  return m_part == -__builtin_inff() ? 0.0f : fast_exp2(m_part - m_tot);
}

template <int D, int G>
struct DecodeGeom {
  static constexpr int kLanesPerRow = D / 8;              // 16 (d=128) or 8 (d=64)
  static constexpr int kGroupsPerWave = kWave / kLanesPerRow;
  static constexpr int kGroups = 4 * kGroupsPerWave;      // rows in flight per pass
  static constexpr int kUnroll = G <= 4 ? 8 : 4;          // rows per group per pass
  static constexpr int kIdxTile = 1024;                   // selected rows staged in LDS
};

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  using Geo = DecodeGeom<D, G>;
  constexpr int LG = Geo::kLanesPerRow;
  constexpr int U = Geo::kUnroll;
  __shared__ float sm[4][G], sl[4][G];
  __shared__ float so[4][G][D];
  __shared__ int32_t sidx[Geo::kIdxTile];

  const int u = blockIdx.x / a.S, split = blockIdx.x % a.S;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int gid = w * Geo::kGroupsPerWave + lane / LG;
  const int sub = lane % LG;

  // queries of the group, this lane's 8 dims, pre-scaled
  float qf[G][8];
  {
    const uint16_t* qb = a.q + ((size_t)b * a.Hq + (size_t)h * G) * D + sub * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qb + (size_t)g * D);
      float f[8];
      bf16x8_to_f32(raw, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[g][e] = f[e] * a.qscale;
    }
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -__builtin_inff();
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.0f;
  }

  const int r0 = split * a.rps;
  const int r1 = min(a.M, r0 + a.rps);
  const int32_t* idx_u = a.idx + (size_t)u * a.M;
  // this unit's K and V rows; a padding entry maps to an offset past the end
  // and loads zeros (masked out of the softmax below)
  const uint32_t unit_bytes = (uint32_t)a.Ncap * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (size_t)u * a.Ncap * D, unit_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (size_t)u * a.Ncap * D, unit_bytes);
  const uint32_t lane_off = (uint32_t)(sub * 16);

  for (int t0 = r0; t0 < r1; t0 += Geo::kIdxTile) {
    const int t1 = min(r1, t0 + Geo::kIdxTile);
    __syncthreads();
    for (int j = t0 + tid; j < t1; j += kBlock) sidx[j - t0] = idx_u[j];
    __syncthreads();
    // Every lane runs the same trip count (rows past t1 are masked), so the
    // DPP reductions always see the whole wave active.  Row loads are
    // unconditional buffer loads.
    for (int j0 = t0; j0 < t1; j0 += Geo::kGroups * U) {
      bool ok[U];
      uint4 kr[U], vr[U];
#pragma unroll
      for (int x = 0; x < U; ++x) {
        const int jj = j0 + gid + x * Geo::kGroups;
        const int n = jj < t1 ? sidx[jj - t0] : -1;
        ok[x] = (unsigned)n < (unsigned)a.Ncap;
        const uint32_t off = ok[x] ? (uint32_t)n * (D * 2) + lane_off : 0xFFFFFFF0u;
        kr[x] = buffer_load16(rk, off, 0);
        vr[x] = buffer_load16(rv, off, 0);
      }
      // logits (base 2), reduced over the row's lanes
      float s[U][G];
#pragma unroll
      for (int x = 0; x < U; ++x) {
        float kf[8];
        bf16x8_to_f32(kr[x], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = qf[g][0] * kf[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) acc = __builtin_fmaf(qf[g][e], kf[e], acc);
          s[x][g] = group_sum<LG>(acc);
        }
      }
      // online softmax update of this lane group's state
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = m[g];
#pragma unroll
        for (int x = 0; x < U; ++x) mx = ok[x] ? fmaxf(mx, s[x][g]) : mx;
        const float alpha = merge_scale(m[g], mx);
        float p[U];
#pragma unroll
        for (int x = 0; x < U; ++x) p[x] = ok[x] ? fast_exp2(s[x][g] - mx) : 0.0f;
        float lsum = l[g] * alpha;
#pragma unroll
        for (int x = 0; x < U; ++x) lsum += p[x];
        l[g] = lsum;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
#pragma unroll
        for (int x = 0; x < U; ++x) {
          float vf[8];
          bf16x8_to_f32(vr[x], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[g][e] = __builtin_fmaf(p[x], vf[e], o[g][e]);
        }
        m[g] = mx;
      }
    }
  }

  // merge the lane groups of this wave (lanes with equal `sub`)
#pragma unroll
  for (int off = LG; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off, kWave);
      const float lo = __shfl_xor(l[g], off, kWave);
      const float mt = fmaxf(m[g], mo);
      const float as = merge_scale(m[g], mt), ao = merge_scale(mo, mt);
      l[g] = l[g] * as + lo * ao;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float oo = __shfl_xor(o[g][e], off, kWave);
        o[g][e] = o[g][e] * as + oo * ao;
      }
      m[g] = mt;
    }
  }
  if (lane < LG) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) { sm[w][g] = m[g]; sl[w][g] = l[g]; }
#pragma unroll
      for (int e = 0; e < 8; ++e) so[w][g][sub * 8 + e] = o[g][e];
    }
  }
  __syncthreads();

  // merge the 4 waves: thread -> (g, dim)
  const size_t part0 = ((size_t)u * a.S + split) * G;
  for (int t = tid; t < G * D; t += kBlock) {
    const int g = t / D, dd = t % D;
    const float mt = fmaxf(fmaxf(sm[0][g], sm[1][g]), fmaxf(sm[2][g], sm[3][g]));
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float sc = merge_scale(sm[ww][g], mt);
      lt += sl[ww][g] * sc;
      ot += so[ww][g][dd] * sc;
    }
    if (a.S == 1) {
      const int hq = h * G + g;
      const float val = lt > 0.0f ? ot / lt : 0.0f;
      a.out[((size_t)b * a.Hq + hq) * D + dd] = (uint16_t)f32_to_bf16_bits(val);
      if (dd == 0 && a.lse)
        a.lse[(size_t)b * a.Hq + hq] =
            lt > 0.0f ? (mt + log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
    } else {
      if (dd == 0) { a.pm[part0 + g] = mt; a.pl[part0 + g] = lt; }
      a.po[(part0 + g) * D + dd] = ot;
    }
  }
}

// Merge the S partial states of one unit (one workgroup per unit).  A separate
// launch orders the partial writes before these reads without device-scope
// fences inside the attention kernel.
template <int D, int G>
__global__ __launch_bounds__(256) void combine_kernel(const DecodeArgs a) {
  __shared__ float fm[G], fl[G];
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
static void launch_decode_d(int G, const DecodeArgs& a, dim3 grid, int units, hipStream_t st) {
  switch (G) {
#define SA_CASE(GG)                                                                    \
  case GG:                                                                             \
    hipLaunchKernelGGL((decode_kernel<D, GG>), grid, dim3(kBlock), 0, st, a);          \
    if (a.S > 1)                                                                       \
      hipLaunchKernelGGL((combine_kernel<D, GG>), dim3(units), dim3(kBlock), 0, st, a); \
    break;
    SA_CASE(1) SA_CASE(2) SA_CASE(3) SA_CASE(4) SA_CASE(5) SA_CASE(6) SA_CASE(7) SA_CASE(8)
    SA_CASE(9) SA_CASE(10) SA_CASE(11) SA_CASE(12) SA_CASE(13) SA_CASE(14) SA_CASE(15)
    SA_CASE(16)
#undef SA_CASE
    default: break;
  }
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
  const dim3 grid((unsigned)blocks);
  if (c.D == 128) launch_decode_d<128>(c.G, a, grid, plan.units, c.stream);
  else launch_decode_d<64>(c.G, a, grid, plan.units, c.stream);
  return hipGetLastError();
}

}  // namespace sa
