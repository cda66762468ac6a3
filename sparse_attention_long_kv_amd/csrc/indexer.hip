// Indexer scoring and exact top-M selection per (batch row, KV head) unit.
//
// JSSA article (rit.work blog, Joint Subspace Sparse Attention), "How JSSA
// preserves token order": the queries of one KV head's group are averaged and
// projected onto the head's basis, then every cached position is scored
// against the FP8 projected-key cache; each group keeps its own set.  The
// IndexCache article ("DeepSeek Sparse Attention") names the selection:
// keep the k (here M) most relevant positions.
//
// Scores.  qt = P[h]^T mean_g q[h*G+g] is formed in fp64 and rounded to fp32.
// A position's r FP8 codes are decoded exactly (gfx950 packed conversion) and
// dotted with qt in fp32: one 16-term fused multiply-add chain per 16 codes,
// the two chains of r = 32 added together.  One lane reads 16 bytes, so a
// wave reads 1 KB of contiguous cache per instruction.
//
// Selection is exact.  Scores map to order-preserving uint32 keys (0 = no
// position).  A workgroup holds up to 16384 keys in registers (64 per
// thread).  It finds the M-th largest key t by bisection over the key range,
// counting keys >= t with wave ballots, then emits every key > t plus the
// lowest-position keys == t, in ascending position order, with one ordered
// prefix scan.  The fused path ("index_topm") splits a unit's positions into
// chunks, selects the chunk-local top-M (exact for the union because the
// order (score desc, position asc) is total), and the last chunk workgroup of
// a unit to finish merges the candidates with the same machinery.  The
// unfused path ("topm") does the same from scores stored in HBM.
#include "device_common.hpp"
#include "kernels.h"

namespace sa {

// ------------------------------------------------------------------ query

// qt (R floats, LDS) for unit (b, h).  `part` is 256 doubles of LDS.
// Every thread of the block must call this (it synchronises).
template <int D, int R>
__device__ void indexer_query(const uint16_t* __restrict__ q, const float* __restrict__ P,
                              int b, int h, int G, int Hq, float* qt, double* part) {
  constexpr int kParts = kBlock / R;     // 8 (r=32) or 16 (r=16)
  constexpr int kPer = D / kParts;       // basis rows per part
  const int t = threadIdx.x;
  const int j = t % R, pi = t / R;
  const uint16_t* qb = q + ((size_t)b * Hq + (size_t)h * G) * D;
  const float* Ph = P + (size_t)h * D * R;
  double acc = 0.0;
  for (int k = 0; k < kPer; ++k) {
    const int i = pi * kPer + k;
    double qs = 0.0;
    for (int g = 0; g < G; ++g) qs += (double)__uint_as_float((uint32_t)qb[g * D + i] << 16);
    acc = fma(qs / (double)G, (double)Ph[i * R + j], acc);
  }
  part[t] = acc;
  __syncthreads();
  if (t < R) {
    double s = 0.0;
    for (int p = 0; p < kParts; ++p) s += part[p * R + t];
    qt[t] = (float)s;
  }
  __syncthreads();
}

// qt entries this lane multiplies: r=32 lanes pair up (even lane: codes
// 0..15, odd lane: 16..31); r=16 lanes own a whole position.
template <int R>
__device__ __forceinline__ void lane_query(const float* qt, float (&ql)[16]) {
  const int off = (R == 32) ? 16 * (lane_id() & 1) : 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) ql[k] = qt[off + k];
}

// One 16-code fused multiply-add chain.
__device__ __forceinline__ float score16(const float (&ql)[16], const uint4 c) {
  float f[16];
  fp8x4_to_f32(c.x, f);
  fp8x4_to_f32(c.y, f + 4);
  fp8x4_to_f32(c.z, f + 8);
  fp8x4_to_f32(c.w, f + 12);
  float acc = ql[0] * f[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) acc = __builtin_fmaf(ql[k], f[k], acc);
  return acc;
}

// Score of the position this lane serves; r=32 adds the partner lane's chain.
// Must be called with every lane of the wave active.
template <int R>
__device__ __forceinline__ float lane_score(const float (&ql)[16], const uint4 c) {
  float s = score16(ql, c);
  if (R == 32) s = s + dpp_f<kDppQuadSwap1>(s);
  return s;
}

__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ------------------------------------------------------------------ scores

constexpr int kScorePositionsPerBlock = 8192;

template <int D, int R>
__global__ __launch_bounds__(256) void index_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ P, const uint8_t* __restrict__ kp,
    const int32_t* __restrict__ seq_lens, int n_max, int Ncap, int Hq, int Hkv, int G,
    int blocks_per_unit, float* __restrict__ scores) {
  __shared__ float qt[32];
  __shared__ double part[kBlock];
  const int u = blockIdx.x / blocks_per_unit, blk = blockIdx.x % blocks_per_unit;
  const int b = u / Hkv, h = u % Hkv;
  indexer_query<D, R>(q, P, b, h, G, Hq, qt, part);
  float ql[16];
  lane_query<R>(qt, ql);
  const int len = seq_lens ? min(max(seq_lens[b], 0), n_max) : n_max;
  const int w = threadIdx.x / kWave, lane = lane_id();
  constexpr int kPPW = kWave * 16 / R;              // positions per wave instruction
  constexpr int kIters = kScorePositionsPerBlock / (4 * kPPW);
  const uint8_t* kpu = kp + (size_t)u * Ncap * R;
  float* su = scores + (size_t)u * n_max;
  const int pos_lane = (R == 32) ? (lane >> 1) : lane;
  for (int it = 0; it < kIters; ++it) {
    const int p0 = blk * kScorePositionsPerBlock + (it * 4 + w) * kPPW;
    if (p0 >= n_max) break;                         // uniform per wave
    const int p = p0 + pos_lane;
    uint4 c = make_uint4(0, 0, 0, 0);
    if (p < len) c = load16(kpu + (size_t)p0 * R + lane * 16);
    float s = lane_score<R>(ql, c);
    if (p >= len) s = -__builtin_inff();
    const bool writer = (R == 32) ? ((lane & 1) == 0) : true;
    if (writer && p < n_max) su[p] = s;
  }
}

hipError_t run_index_score(const LaunchCommon& c, const void* q, const float* P,
                           const uint8_t* kp, const int32_t* seq_lens, int n_max,
                           float* scores) {
  const int bpu = (n_max + kScorePositionsPerBlock - 1) / kScorePositionsPerBlock;
  const long blocks = (long)bpu * c.units;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kBlock);
  const uint16_t* qq = (const uint16_t*)q;
#define SA_LAUNCH_SCORE(DD, RR)                                                            \
  hipLaunchKernelGGL((index_score_kernel<DD, RR>), grid, block, 0, c.stream, qq, P, kp,    \
                     seq_lens, n_max, c.Ncap, c.Hq, c.Hkv, c.G, bpu, scores)
  if (c.D == 128 && c.R == 32) SA_LAUNCH_SCORE(128, 32);
  else if (c.D == 128 && c.R == 16) SA_LAUNCH_SCORE(128, 16);
  else if (c.D == 64 && c.R == 32) SA_LAUNCH_SCORE(64, 32);
  else SA_LAUNCH_SCORE(64, 16);
#undef SA_LAUNCH_SCORE
  return hipGetLastError();
}

// ------------------------------------------------------------------ select

struct SelectArgs {
  const uint16_t* q;
  const float* P;
  const uint8_t* kp;
  const float* scores;
  const int32_t* seq_lens;
  int n_max, Ncap, Hq, Hkv, G, M, S, chunk, mc;
  uint32_t* counters;
  int32_t* cand_cnt;
  uint32_t* cand_key;
  int32_t* cand_pos;
  int32_t* idx;
};

struct SelectShared {
  float qt[32];
  double part[kBlock];
  uint32_t red[8];
  uint32_t seg[kBlock];
  uint32_t wtot[4];
  uint32_t flag;
  int32_t cnt[kMaxSplits];
};

// Number of keys >= t over the block (every thread receives it).
template <int K>
__device__ __forceinline__ uint32_t count_ge(const uint32_t (&key)[K], uint32_t t,
                                             SelectShared& sh, int& ph) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < K; ++i) c += (uint32_t)popc64(ballot(key[i] >= t));
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) sh.red[ph * 4 + w] = c;
  __syncthreads();
  const uint32_t tot = sh.red[ph * 4] + sh.red[ph * 4 + 1] + sh.red[ph * 4 + 2] + sh.red[ph * 4 + 3];
  ph ^= 1;
  return tot;
}

// Block-wide min over nonzero keys and max over all keys.
__device__ __forceinline__ void block_key_range(uint32_t mn, uint32_t mx, SelectShared& sh,
                                                uint32_t& omn, uint32_t& omx) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, kWave));
  }
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) { sh.seg[w] = mn; sh.seg[4 + w] = mx; }
  __syncthreads();
  omn = min(min(sh.seg[0], sh.seg[1]), min(sh.seg[2], sh.seg[3]));
  omx = max(max(sh.seg[4], sh.seg[5]), max(sh.seg[6], sh.seg[7]));
  __syncthreads();
}

template <int K>
__device__ __forceinline__ void thread_key_range(const uint32_t (&key)[K], uint32_t& mn,
                                                 uint32_t& mx) {
#pragma unroll
  for (int i = 0; i < K; ++i) {
    mn = key[i] ? min(mn, key[i]) : mn;
    mx = max(mx, key[i]);
  }
}

// Largest t with count(key >= t) >= target, given count(key >= lo) >= target
// and hi = the largest key.  `cnt(t)` is a block-uniform count.
template <class CountFn>
__device__ __forceinline__ uint32_t find_threshold(CountFn cnt, uint32_t lo, uint32_t hi,
                                                   uint32_t target) {
  if (cnt(hi) >= target) return hi;
  while (hi - lo > 1) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (cnt(mid) >= target) lo = mid; else hi = mid;
  }
  return lo;
}

// Emit, in register order (i, wave, lane) -- which callers make equal to
// position order -- every key > t and the first `need` keys == t (counting
// from eq_base already emitted).  emit(i, slot) receives the output slot.
// Returns this tile's (gt, eq) totals packed as gt | eq << 16.
template <int K, class EmitFn>
__device__ __forceinline__ uint32_t emit_in_order(const uint32_t (&key)[K], uint32_t t,
                                                  uint32_t need, uint32_t gt_base,
                                                  uint32_t eq_base, SelectShared& sh,
                                                  EmitFn emit) {
  static_assert(K * 4 <= kBlock, "segments");
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const uint64_t mg = ballot(key[i] > t), me = ballot(key[i] == t);
    if (lane == 0) sh.seg[i * 4 + w] = (uint32_t)popc64(mg) | ((uint32_t)popc64(me) << 16);
  }
  __syncthreads();
  const uint32_t v = tid < K * 4 ? sh.seg[tid] : 0u;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) sh.wtot[w] = inc;
  __syncthreads();
  uint32_t wb = 0;
  for (int ww = 0; ww < w; ++ww) wb += sh.wtot[ww];
  const uint32_t total = sh.wtot[0] + sh.wtot[1] + sh.wtot[2] + sh.wtot[3];
  if (tid < K * 4) sh.seg[tid] = wb + inc - v;
  __syncthreads();
  const uint64_t lt = lanemask_lt();
  // An opaque copy of t keeps the compiler from carrying the first pass's
  // 2*K ballot masks (scalar register pairs) across the scan.
  uint32_t t2 = t;
  asm volatile("" : "+v"(t2));
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const uint64_t mg = ballot(key[i] > t2), me = ballot(key[i] == t2);
    const uint32_t pre = sh.seg[i * 4 + w];
    const uint32_t gtb = gt_base + (pre & 0xFFFFu) + (uint32_t)popc64(mg & lt);
    const uint32_t eqb = eq_base + (pre >> 16) + (uint32_t)popc64(me & lt);
    if (key[i] > t2) emit(i, gtb + min(eqb, need));
    else if (key[i] == t2 && eqb < need) emit(i, gtb + eqb);
  }
  __syncthreads();
  return total;
}

// Candidate key of flat slot f in a unit's [S][mc] candidate array (0 if empty).
__device__ __forceinline__ uint32_t cand_key_at(const uint32_t* ck, const SelectShared& sh,
                                                int f, int flat_n, int mc) {
  if (f >= flat_n) return 0u;
  const int s = f / mc, k = f - s * mc;
  return k < sh.cnt[s] ? ck[f] : 0u;
}

// Merge the chunk candidates of unit u into idx (last workgroup of the unit).
template <bool MULTI>
__device__ void merge_unit(const SelectArgs& a, int u, SelectShared& sh) {
  const int tid = threadIdx.x;
  const int S = a.S, mc = a.mc, M = a.M;
  const int flat_n = S * mc;
  uint32_t my = 0;
  for (int s = tid; s < S; s += kBlock) {
    const int c = a.cand_cnt[(size_t)u * S + s];
    sh.cnt[s] = c;
    my += (uint32_t)c;
  }
  const uint32_t total = wave_sum_u32(my);
  __syncthreads();
  if (lane_id() == 0) sh.red[tid / kWave] = total;
  __syncthreads();
  const uint32_t nvalid = sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3];
  __syncthreads();
  const uint32_t* ck = a.cand_key + (size_t)u * flat_n;
  const int32_t* cp = a.cand_pos + (size_t)u * flat_n;
  int32_t* idx_u = a.idx + (size_t)u * M;
  const uint32_t target = min(nvalid, (uint32_t)M);
  int ph = 0;
  constexpr int K = kMaxKeysPerThread;

  if (!MULTI) {
    uint32_t key[K];
#pragma unroll
    for (int i = 0; i < K; ++i) key[i] = cand_key_at(ck, sh, i * kBlock + tid, flat_n, mc);
    uint32_t t = 0, need = 0;
    if (nvalid > (uint32_t)M) {
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      thread_key_range(key, mn, mx);
      block_key_range(mn, mx, sh, mn, mx);
      t = find_threshold([&](uint32_t x) { return count_ge(key, x, sh, ph); }, mn, mx, target);
      const uint32_t gt = (t == 0xFFFFFFFFu) ? 0u : count_ge(key, t + 1, sh, ph);
      need = target - gt;
    }
    emit_in_order(key, t, need, 0, 0, sh, [&](int i, uint32_t slot) {
      idx_u[slot] = cp[i * kBlock + tid];
    });
  } else {
    const int ntiles = (flat_n + kMergeTile - 1) / kMergeTile;
    auto load_tile = [&](int tile, uint32_t (&key)[K]) {
#pragma unroll
      for (int i = 0; i < K; ++i)
        key[i] = cand_key_at(ck, sh, tile * kMergeTile + i * kBlock + tid, flat_n, mc);
    };
    uint32_t t = 0, need = 0;
    if (nvalid > (uint32_t)M) {
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      for (int tile = 0; tile < ntiles; ++tile) {
        uint32_t key[K];
        load_tile(tile, key);
        thread_key_range(key, mn, mx);
      }
      block_key_range(mn, mx, sh, mn, mx);
      auto cnt = [&](uint32_t x) {
        uint32_t c = 0;
        for (int tile = 0; tile < ntiles; ++tile) {
          uint32_t key[K];
          load_tile(tile, key);
          c += count_ge(key, x, sh, ph);
        }
        return c;
      };
      t = find_threshold(cnt, mn, mx, target);
      const uint32_t gt = (t == 0xFFFFFFFFu) ? 0u : cnt(t + 1);
      need = target - gt;
    }
    uint32_t gt_base = 0, eq_base = 0;
    for (int tile = 0; tile < ntiles; ++tile) {
      uint32_t key[K];
      load_tile(tile, key);
      const int fbase = tile * kMergeTile;
      const uint32_t tot = emit_in_order(key, t, need, gt_base, eq_base, sh,
                                         [&](int i, uint32_t slot) {
                                           idx_u[slot] = cp[fbase + i * kBlock + tid];
                                         });
      gt_base += tot & 0xFFFFu;
      eq_base += tot >> 16;
    }
  }
  for (int slot = (int)target + tid; slot < M; slot += kBlock) idx_u[slot] = -1;
}

// One chunk of one unit: keys, chunk-local top-M, candidates, then the
// last-arriving chunk workgroup of the unit merges.
template <int D, int R, int KPT, bool FUSED, bool MULTI>
__global__ __launch_bounds__(256) void select_kernel(const SelectArgs a) {
  __shared__ SelectShared sh;
  const int u = blockIdx.x / a.S, c = blockIdx.x % a.S;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int len = a.seq_lens ? min(max(a.seq_lens[b], 0), a.n_max) : a.n_max;
  const int base = c * a.chunk;
  const int nv = min(max(len - base, 0), a.chunk);
  int nsel = 0;

  if (nv > 0) {                                   // block-uniform
    uint32_t key[KPT];
    if (FUSED) {
      indexer_query<D, R>(a.q, a.P, b, h, a.G, a.Hq, sh.qt, sh.part);
      float ql[16];
      lane_query<R>(sh.qt, ql);
      const uint8_t* kpu = a.kp + (size_t)u * a.Ncap * R;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int p = base + i * kBlock + w * kWave + lane;
        if (R == 16) {
          uint4 cc = make_uint4(0, 0, 0, 0);
          if (p < len) cc = load16(kpu + (size_t)p * 16);
          const float s = lane_score<R>(ql, cc);
          key[i] = p < len ? score_key(s + 0.0f) : 0u;
        } else {
          const int p0 = base + i * kBlock + w * kWave;
          const int pa = p0 + (lane >> 1), pb = pa + 32;
          uint4 ca = make_uint4(0, 0, 0, 0), cb = make_uint4(0, 0, 0, 0);
          if (pa < len) ca = load16(kpu + (size_t)p0 * 32 + lane * 16);
          if (pb < len) cb = load16(kpu + (size_t)p0 * 32 + 1024 + lane * 16);
          const float sa = lane_score<R>(ql, ca);
          const float sb = lane_score<R>(ql, cb);
          // lane l takes position p0 + l: from lane 2l of the first half
          // (l < 32) or lane 2(l-32)+1 of the second
          const float x = (lane & 1) ? sb : sa;
          const int src = (lane < 32) ? 2 * lane : 2 * (lane - 32) + 1;
          const float s = __shfl(x, src, kWave);
          key[i] = p < len ? score_key(s + 0.0f) : 0u;
        }
      }
    } else {
      const float* su = a.scores + (size_t)u * a.n_max;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int p = base + i * kBlock + w * kWave + lane;
        key[i] = p < len ? score_key(su[p] + 0.0f) : 0u;
      }
    }

    uint32_t t = 0, need = 0;
    if (nv > a.M) {
      int ph = 0;
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      thread_key_range(key, mn, mx);
      block_key_range(mn, mx, sh, mn, mx);
      const uint32_t target = (uint32_t)a.M;
      t = find_threshold([&](uint32_t x) { return count_ge(key, x, sh, ph); }, mn, mx, target);
      const uint32_t gt = (t == 0xFFFFFFFFu) ? 0u : count_ge(key, t + 1, sh, ph);
      need = target - gt;
      nsel = a.M;
    } else {
      nsel = nv;
    }
    uint32_t* ck = a.cand_key + ((size_t)u * a.S + c) * a.mc;
    int32_t* cp = a.cand_pos + ((size_t)u * a.S + c) * a.mc;
    emit_in_order(key, t, need, 0, 0, sh, [&](int i, uint32_t slot) {
      ck[slot] = key[i];
      cp[slot] = base + i * kBlock + w * kWave + lane;
    });
  }
  if (tid == 0) a.cand_cnt[(size_t)u * a.S + c] = nsel;

  // last workgroup of the unit to arrive merges
  __threadfence();
  __syncthreads();
  if (tid == 0) sh.flag = (atomicAdd(&a.counters[u], 1u) == (uint32_t)(a.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (!sh.flag) return;
  __threadfence();
  if (tid == 0) atomicExch(&a.counters[u], 0u);
  merge_unit<MULTI>(a, u, sh);
}

template <int D, int R, bool FUSED, bool MULTI>
static void launch_select_kpt(const SelectArgs& a, int kpt, dim3 grid, hipStream_t st) {
  switch (kpt) {
#define SA_CASE(K)                                                                         \
  case K:                                                                                  \
    hipLaunchKernelGGL((select_kernel<D, R, K, FUSED, MULTI>), grid, dim3(kBlock), 0, st, a); \
    break;
    SA_CASE(1) SA_CASE(2) SA_CASE(4) SA_CASE(8) SA_CASE(16) SA_CASE(32) SA_CASE(64)
#undef SA_CASE
    default: break;
  }
}

template <bool FUSED, bool MULTI>
static void launch_select_shape(const LaunchCommon& c, const SelectArgs& a, int kpt, dim3 grid) {
  if (!FUSED) { launch_select_kpt<64, 16, false, MULTI>(a, kpt, grid, c.stream); return; }
  if (c.D == 128 && c.R == 32) launch_select_kpt<128, 32, true, MULTI>(a, kpt, grid, c.stream);
  else if (c.D == 128 && c.R == 16) launch_select_kpt<128, 16, true, MULTI>(a, kpt, grid, c.stream);
  else if (c.D == 64 && c.R == 32) launch_select_kpt<64, 32, true, MULTI>(a, kpt, grid, c.stream);
  else launch_select_kpt<64, 16, true, MULTI>(a, kpt, grid, c.stream);
}

hipError_t run_select(const LaunchCommon& c, const TopmPlan& plan, bool fused, const void* q,
                      const float* P, const uint8_t* kp, const float* scores,
                      const int32_t* seq_lens, int n_max, int M, int32_t* idx,
                      void* workspace) {
  SelectArgs a;
  a.q = (const uint16_t*)q;
  a.P = P;
  a.kp = kp;
  a.scores = scores;
  a.seq_lens = seq_lens;
  a.n_max = n_max;
  a.Ncap = c.Ncap;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.G = c.G;
  a.M = M;
  a.S = plan.splits;
  a.chunk = plan.chunk;
  a.mc = plan.mc;
  char* ws = (char*)workspace;
  a.counters = (uint32_t*)ws;
  a.cand_cnt = (int32_t*)(ws + plan.off_cnt);
  a.cand_key = (uint32_t*)(ws + plan.off_key);
  a.cand_pos = (int32_t*)(ws + plan.off_pos);
  a.idx = idx;
  const long blocks = (long)plan.units * plan.splits;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (fused) {
    if (plan.multi_tile) launch_select_shape<true, true>(c, a, plan.kpt, grid);
    else launch_select_shape<true, false>(c, a, plan.kpt, grid);
  } else {
    if (plan.multi_tile) launch_select_shape<false, true>(c, a, plan.kpt, grid);
    else launch_select_shape<false, false>(c, a, plan.kpt, grid);
  }
  return hipGetLastError();
}

}  // namespace sa
