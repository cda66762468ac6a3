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

// ------------------------------------------------------------------ baselines
//
// Comparison baselines for the JSSA article's two measurements: full
// attention (its opening paragraph compares decoding throughput against it)
// and the gather-then-attend scheme ("Why token selection is not enough": the
// copy into a contiguous buffer took more than half of the sparse-attention
// time at large batch).  Neither is on the hot path.

// Exact attention over every valid row n < len of the unit (consecutive
// cache rows), split over S workgroups like the sparse kernel.
template <int D>
__global__ __launch_bounds__(kAttendThreads) void dense_decode_kernel(const DecodeArgs a) {
  constexpr int W = kAttendWaves;
  __shared__ float sm[W][kMaxHeads], sl[W][kMaxHeads];
  extern __shared__ float so[];       // [W][G][D]
  const int u = blockIdx.x / a.S, split = blockIdx.x % a.S;
  const int b = u / a.Hkv;
  const int len = a.lens ? min(max(a.lens[b], 0), a.n_max) : a.n_max;
  AttendWave<D, W> aw;
  aw.init(a, u);
  const int r0 = split * a.rps;
  const int r1 = min(len, r0 + a.rps);
  if (r1 > r0) aw.rows_dense(a, r0, r1 - r0);       // block-uniform
  aw.finish(a, u, split, sm, sl, so);
}

// Copy of the selected rows into contiguous [units][M][d] buffers (zero rows
// for idx < 0): the "gather" of gather-then-attend.
constexpr int kGatherPasses = 8;

template <int D>
__global__ __launch_bounds__(kBlock) void gather_rows_kernel(const int32_t* __restrict__ idx,
                                                             int M, int Ncap,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             uint16_t* __restrict__ ko,
                                                             uint16_t* __restrict__ vo,
                                                             int blocks_per_unit) {
  constexpr int kPieces = D / 8;                      // 16-byte pieces per row
  constexpr int kRowsPerPass = kBlock / kPieces;
  const int u = blockIdx.x / blocks_per_unit, blk = blockIdx.x % blocks_per_unit;
  const int piece = threadIdx.x % kPieces;
#pragma unroll
  for (int pass = 0; pass < kGatherPasses; ++pass) {
    const int j = (blk * kGatherPasses + pass) * kRowsPerPass + threadIdx.x / kPieces;
    if (j < M) {
      const int n = idx[(size_t)u * M + j];
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
      if ((unsigned)n < (unsigned)Ncap) {
        const size_t src = ((size_t)u * Ncap + n) * D + piece * 8;
        kv = *reinterpret_cast<const uint4*>(k + src);
        vv = *reinterpret_cast<const uint4*>(v + src);
      }
      const size_t dst = ((size_t)u * M + j) * D + piece * 8;
      *reinterpret_cast<uint4*>(ko + dst) = kv;
      *reinterpret_cast<uint4*>(vo + dst) = vv;
    }
  }
}

// Merge the S partial states of one unit's head: one workgroup of D threads
// per (unit, head), thread dd owning output dimension dd.  A separate launch
// orders the partial writes before these reads without device-scope fences
// inside the attention kernel.  Every state of the head is loaded at once;
// the weights 2^(m_s - m) and l = sum_s l_s 2^(m_s - m) are formed in split
// order, and o = sum_s o_s 2^(m_s - m) / l in split order from loads issued
// eight splits at a time.
constexpr int kMaxSplitsCombine = 256;     // splits per unit the planners produce, at most

template <int D>
__global__ __launch_bounds__(D) void combine_kernel(const DecodeArgs a) {
  __shared__ float sm[kMaxSplitsCombine], sw[kMaxSplitsCombine];
  __shared__ float fm, fl;
  const int G = a.G, S = a.S;
  const int u = blockIdx.x / G, g = blockIdx.x % G;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x;
  const size_t ubase = (size_t)u * S * G;
  float lv[kMaxSplitsCombine / D];
#pragma unroll
  for (int k = 0; k < kMaxSplitsCombine / D; ++k) {
    const int s2 = tid + k * D;
    lv[k] = 0.0f;
    if (s2 < S) {
      sm[s2] = a.pm[ubase + (size_t)s2 * G + g];
      lv[k] = a.pl[ubase + (size_t)s2 * G + g];
    }
  }
  __syncthreads();
  if (tid == 0) {
    float mt = -__builtin_inff();
    for (int s2 = 0; s2 < S; ++s2) mt = fmaxf(mt, sm[s2]);
    fm = mt;
  }
  __syncthreads();
  const float mt = fm;
#pragma unroll
  for (int k = 0; k < kMaxSplitsCombine / D; ++k) {
    const int s2 = tid + k * D;
    if (s2 < S) {
      const float w = merge_scale(sm[s2], mt);
      sw[s2] = w;
      sm[s2] = lv[k] * w;                       // l_s 2^(m_s - m)
    }
  }
  __syncthreads();
  if (tid == 0) {
    float lt = 0.0f;
    for (int s2 = 0; s2 < S; ++s2) lt += sm[s2];
    fl = lt;
  }
  const float* po = a.po + ubase * D + (size_t)g * D + tid;   // split s2 at s2 * G * D
  float ot = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = s0 + k < S ? po[(size_t)(s0 + k) * G * D] : 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < S) ot += v[k] * sw[s0 + k];
  }
  __syncthreads();
  const float lt = fl;
  const int hq = h * G + g;
  const float val = lt > 0.0f ? ot / lt : 0.0f;
  a.out[((size_t)b * a.Hq + hq) * D + tid] = (uint16_t)f32_to_bf16_bits(val);
  if (tid == 0 && a.lse)
    a.lse[(size_t)b * a.Hq + hq] =
        lt > 0.0f ? (mt + log2f(lt)) * 0.69314718055994530942f : -__builtin_inff();
}

template <int D>
static void launch_decode_d(const DecodeArgs& a, dim3 grid, int units, hipStream_t st) {
  const size_t lds = (size_t)kAttendWaves * a.G * D * sizeof(float);
  hipLaunchKernelGGL((decode_kernel<D>), grid, dim3(kAttendThreads), lds, st, a);
  if (a.S > 1) hipLaunchKernelGGL((combine_kernel<D>), dim3(units * a.G), dim3(D), 0, st, a);
}

// Streaming read of a buffer (a measurement helper): workgroup w reads the
// w-th 4 MiB, each wave load 1 KB of contiguous bytes (16 per lane), four
// loads per thread in flight, non-temporal (the pattern that read fastest on
// this GPU in a sweep of workgroup sizes, bytes per workgroup, loads in
// flight and cache policies: ~7 TB/s).
constexpr size_t kStreamBytesPerBlock = 4u << 20;
constexpr int kStreamThreads = 512;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const uint8_t* __restrict__ p,
                                                                     uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(p + (size_t)blockIdx.x * kStreamBytesPerBlock, (uint32_t)kStreamBytesPerBlock);
  constexpr uint32_t kStep = kStreamThreads * 16 * 4;
  uint32_t acc = 0u;
  for (uint32_t base = 0; base < (uint32_t)kStreamBytesPerBlock; base += kStep) {
    sa_u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      v[k] = __builtin_amdgcn_raw_buffer_load_b128(
          r, (int)(base + k * kStreamThreads * 16 + threadIdx.x * 16), 0, kRowLoadPolicy);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k].x + v[k].y + v[k].z + v[k].w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

hipError_t run_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t blocks = bytes / kStreamBytesPerBlock;
  if (blocks == 0 || blocks * kStreamBytesPerBlock != bytes || blocks > INT32_MAX)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, st,
                     (const uint8_t*)buf, sink);
  return hipGetLastError();
}

// Reads of the selected rows alone (a measurement helper): one 16-wave
// workgroup per unit, wave w taking tiles w, w + 16, ... of 16 selected rows,
// every K and V row of a tile read once with the non-temporal policy, and
// nothing computed.  MODE 0: into registers with AttendWave's lane layout;
// MODE 1: straight into LDS (buffer loads to LDS, each wave load a run of
// whole rows, one tile per wave in flight).
template <int D, int MODE>
__global__ __launch_bounds__(kAttendThreads) void row_read_kernel(const int32_t* __restrict__ idx,
                                                                 int M, int Ncap,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 uint32_t* sink) {
  constexpr int W = kAttendWaves;
  constexpr int RB = D * 2;                           // bytes per row
  constexpr int TB = 16 * RB;                         // bytes per 16-row tile (K or V)
  extern __shared__ uint8_t lds_raw[];
  const int u = blockIdx.x;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int q4 = lane >> 4, n16 = lane & 15;
  const int32_t* iu = idx + (size_t)u * M;
  const uint32_t ub = (uint32_t)Ncap * RB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + (size_t)u * Ncap * D, ub);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (size_t)u * Ncap * D, ub);
  const int ntile = (M + 15) >> 4;
  auto row_off = [&](int j) -> uint32_t {
    const int n = j < M ? iu[j] : -1;
    return (unsigned)n < (unsigned)Ncap ? (uint32_t)n * RB : kOffNone;
  };
  uint32_t acc = 0u;
  for (int tt = w; tt < ntile; tt += W) {
    if (MODE == 0) {
      const int tk = 4 * (n16 & 3) + (n16 >> 2);
      const uint32_t kb = row_off(tt * 16 + tk);
      sa_u32x4 kx[D / 32];
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
        kx[i] = __builtin_amdgcn_raw_buffer_load_b128(
            rk, (int)(kb == kOffNone ? kOffNone : kb + 16u * q4 + 64u * i), 0, kRowLoadPolicy);
      typename VRaw<D>::type vx[4];
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const uint32_t vb = row_off(tt * 16 + 4 * vv + q4);
        vx[vv] = load_v_raw<D>(rv, vb == kOffNone ? kOffNone : vb + (uint32_t)(D / 16 * n16) * 2u);
      }
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc ^= kx[i].x + kx[i].w;
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        if constexpr (D == 128) acc ^= vx[vv].x + vx[vv].w;
        else acc ^= vx[vv].x + vx[vv].y;
      }
    } else {
      // each 1 KB wave load covers 1024 / RB whole rows: lane l reads 16
      // bytes of row (l * 16) / RB of its group
      constexpr int RPL = 1024 / RB;                  // rows per wave load
      constexpr int NL = TB / 1024;                   // wave loads per tile (K or V)
      char __attribute__((address_space(3)))* lb =
          (char __attribute__((address_space(3)))*)(lds_raw) + (size_t)w * 2 * TB;
#pragma unroll
      for (int i = 0; i < 2 * NL; ++i) {
        const int row = tt * 16 + (i % NL) * RPL + (lane * 16) / RB;
        const uint32_t rb = row_off(row);
        const uint32_t off = rb == kOffNone ? kOffNone : rb + (uint32_t)((lane * 16) % RB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            i < NL ? rk : rv, (__attribute__((address_space(3))) void*)(lb + i * 1024), 16, off, 0,
            0, kRowLoadPolicy);
      }
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t* lw = reinterpret_cast<const uint32_t*>(lds_raw + (size_t)w * 2 * TB);
#pragma unroll
      for (int i = 0; i < 2 * NL; ++i) acc ^= lw[i * 256 + lane * 4];
    }
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

hipError_t run_row_read(const LaunchCommon& c, const int32_t* idx, int M, const void* k_cache,
                        const void* v_cache, int mode, uint32_t* sink) {
  const dim3 grid((unsigned)c.units), block(kAttendThreads);
  const size_t lds = mode == 1 ? (size_t)kAttendWaves * 2 * 16 * c.D * 2 : 0;
  const uint16_t* kk = (const uint16_t*)k_cache;
  const uint16_t* vv = (const uint16_t*)v_cache;
  if (c.D == 128 && mode == 0)
    hipLaunchKernelGGL((row_read_kernel<128, 0>), grid, block, 0, c.stream, idx, M, c.Ncap, kk, vv, sink);
  else if (c.D == 128)
    hipLaunchKernelGGL((row_read_kernel<128, 1>), grid, block, lds, c.stream, idx, M, c.Ncap, kk, vv, sink);
  else if (mode == 0)
    hipLaunchKernelGGL((row_read_kernel<64, 0>), grid, block, 0, c.stream, idx, M, c.Ncap, kk, vv, sink);
  else
    hipLaunchKernelGGL((row_read_kernel<64, 1>), grid, block, lds, c.stream, idx, M, c.Ncap, kk, vv, sink);
  return hipGetLastError();
}

hipError_t run_combine(const LaunchCommon& c, const DecodeArgs& a) {
  if (a.S <= 1) return hipSuccess;
  if (a.S > kMaxSplitsCombine) return hipErrorInvalidConfiguration;
  if (c.D == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3(c.units * a.G), dim3(128), 0, c.stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<64>), dim3(c.units * a.G), dim3(64), 0, c.stream, a);
  return hipGetLastError();
}

hipError_t run_dense_decode(const LaunchCommon& c, const DecodePlan& plan, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            int n_max, float scale, void* out, float* lse, void* workspace) {
  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.idx = nullptr;
  a.M = n_max;
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
  a.lens = seq_lens;
  a.n_max = n_max;
  const long blocks = (long)plan.units * plan.splits;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (c.G < 1 || c.G > kMaxHeads) return hipErrorInvalidConfiguration;
  if (a.S > kMaxSplitsCombine) return hipErrorInvalidConfiguration;
  if (c.D == 128) {
    hipLaunchKernelGGL((dense_decode_kernel<128>), dim3((unsigned)blocks), dim3(kAttendThreads),
                       (size_t)kAttendWaves * c.G * 128 * sizeof(float), c.stream, a);
  } else {
    hipLaunchKernelGGL((dense_decode_kernel<64>), dim3((unsigned)blocks), dim3(kAttendThreads),
                       (size_t)kAttendWaves * c.G * 64 * sizeof(float), c.stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = run_combine(c, a);
  return e;
}

hipError_t run_gather_kv(const LaunchCommon& c, const int32_t* idx, int M, const void* k_cache,
                         const void* v_cache, void* k_out, void* v_out) {
  const int rows_per_block = kGatherPasses * (kBlock / (c.D / 8));
  const long bpu = (M + rows_per_block - 1) / rows_per_block;
  const long blocks = bpu * c.units;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (c.D == 128)
    hipLaunchKernelGGL((gather_rows_kernel<128>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       c.stream, idx, M, c.Ncap, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, (uint16_t*)k_out, (uint16_t*)v_out, (int)bpu);
  else
    hipLaunchKernelGGL((gather_rows_kernel<64>), dim3((unsigned)blocks), dim3(kBlock), 0,
                       c.stream, idx, M, c.Ncap, (const uint16_t*)k_cache,
                       (const uint16_t*)v_cache, (uint16_t*)k_out, (uint16_t*)v_out, (int)bpu);
  return hipGetLastError();
}

hipError_t run_decode(const LaunchCommon& c, const DecodePlan& plan, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* idx, int M,
                      float scale, void* out, float* lse, void* workspace) {
  DecodeArgs a{};
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
  if (a.S > kMaxSplitsCombine) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (c.D == 128) launch_decode_d<128>(a, grid, plan.units, c.stream);
  else launch_decode_d<64>(a, grid, plan.units, c.stream);
  return hipGetLastError();
}

}  // namespace sa
