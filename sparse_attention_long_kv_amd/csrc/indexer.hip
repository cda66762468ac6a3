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
// the two chains of r = 32 added together, in the same order in every kernel
// (so every kernel forms the same score bits).
//
// Selection is exact.  Scores map to order-preserving uint32 keys (0 = no
// position).  The M-th largest key t is found by a radix select (a 4096-bin
// LDS histogram of the first 12-bit digit, then the keys of the chosen bin
// ranked directly or by two more digits); every key > t and the
// lowest-position keys == t are emitted in ascending position order, by one
// ordered block scan over per-(row, wave) ballot counts when the keys sit in
// registers in position order, else through an LDS bitmap of positions.
// Two paths:
//  * the filter path (fused selection up to 2^19 positions, described before
//    filter_kernel below): a sampled bound, chunks that keep only the keys at
//    or above it, and one merge workgroup per unit;
//  * the chunk-exact path (scores from HBM, or shapes outside the filter
//    path): chunks hand over a superset of their top-M, merged per unit.
// Both give the same idx (the order (score desc, position asc) is total).
#include "append_common.hpp"
#include "attend_common.hpp"
#include "kernels.h"

namespace sa {

// ------------------------------------------------------------------ query

// qt (R floats, LDS) for unit (b, h).  `part` is max(8R, D) doubles of LDS
// (it first holds the group-mean query, then the partial sums).  The fp64 sums run
// in the same order whatever the workgroup size (mean over the group in head
// order; 8 parts of d/8 basis rows, then the parts in order), so every kernel
// forms the same qt bits.  Every thread of the block must call this (it
// synchronises).
template <int D, int R, int NT = kBlock>
__device__ void indexer_query(const uint16_t* __restrict__ q, const float* __restrict__ P,
                              int b, int h, int G, int Hq, float* qt, double* part) {
  constexpr int kParts = 8;              // basis-row groups, one partial sum each
  constexpr int kPer = D / kParts;       // basis rows per part
  static_assert(NT >= kParts * R && NT >= D, "workgroup too small for the query");
  static_assert(kParts * R <= NT && D <= NT, "part holds NT doubles");
  const int t = threadIdx.x;
  const int j = t % R, pi = t / R;
  const uint16_t* qb = q + ((size_t)b * Hq + (size_t)h * G) * D;
  const float* Ph = P + (size_t)h * D * R;
  // this thread's basis entries, loaded before the mean is formed
  float pv[kPer];
  if (t < kParts * R) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) pv[k] = Ph[(pi * kPer + k) * R + j];
  }
  double mean = 0.0;
  if (t < D) {
    for (int g = 0; g < G; ++g) mean += (double)__uint_as_float((uint32_t)qb[g * D + t] << 16);
    mean = mean / (double)G;
  }
  __syncthreads();                       // `part` may still be read by a previous call
  if (t < D) part[t] = mean;
  __syncthreads();
  double acc = 0.0;
  if (t < kParts * R) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc = fma(part[pi * kPer + k], (double)pv[k], acc);
  }
  __syncthreads();
  if (t < kParts * R) part[t] = acc;
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

// ------------------------------------------------------------------ select

struct SelectArgs {
  const uint16_t* q;
  const float* P;
  const uint8_t* kp;
  const float* scores;
  const int32_t* seq_lens;
  int n_max, Ncap, Hq, Hkv, G, M, S, chunk, ms;   // ms: candidate slots per chunk
  int32_t* cand_cnt;
  uint32_t* cand_key;
  int32_t* cand_pos;
  int32_t* idx;
};

// 16-byte loads each lane keeps in flight while scoring (tuning knob)
#ifndef SA_CHUNK_LOADS_IN_FLIGHT
#define SA_CHUNK_LOADS_IN_FLIGHT 8
#endif
// ... and in the filter's code stream (two groups of half of them alternate)
#ifndef SA_FILTER_LOADS_IN_FLIGHT
#define SA_FILTER_LOADS_IN_FLIGHT 4
#endif

// Radix digits of the 32-bit keys, most significant first: [20, 32) holds the
// sign, exponent and top 3 mantissa bits of the score; then [8, 20), [0, 8).
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;      // histogram bins per level
constexpr int kTopShift = 32 - kDigitBits;  // first-level digit = key >> 20
constexpr int kListCap = 6272;              // threshold-bin keys kept in LDS (chunks)
constexpr int kStageSlots = kListCap / 2 - kWave;   // candidates staged in the list region
constexpr int kMergeListCap = 1024;         // (merge: its LDS is nearly full)
constexpr int kRankMax = 256;               // lists up to this size are ranked directly
constexpr int kChunkThreads = kChunkBlock;  // chunk workgroups: 8 waves
constexpr int kMergeThreads = 1024;         // merge workgroups: 16 waves

template <int NT>
struct SelectShared {
  static constexpr int W = NT / kWave;
  float qt[32];
  double part[NT];
  uint32_t seg[NT];
  uint32_t wtot[W];
  uint32_t pick[4];
  uint32_t hist[kBins + kWave];   // + one private dummy bin per lane
  static constexpr int kCap = kListCap;
  alignas(16) uint32_t list[kCap];
};

// Inclusive prefix sum over the block in thread order; `total` gets the sum.
template <int NT, class Sh>
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, Sh& sh, uint32_t& total) {
  constexpr int W = NT / kWave;
  const int w = threadIdx.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane_id() == kWave - 1) sh.wtot[w] = inc;
  __syncthreads();
  uint32_t wb = 0, tot = 0;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) {
    wb += ww < w ? sh.wtot[ww] : 0u;
    tot += sh.wtot[ww];
  }
  total = tot;
  return wb + inc;
}

// With the current level's histogram in sh.hist (bins of keys on `path`),
// find the bin holding the key of 1-based rank target - above counted from the
// top; above += keys in higher bins; path gains the bin as its low digit.
// sh.pick[2] is left holding the chosen bin's count.
template <int NT, class Sh>
__device__ void pick_bin(Sh& sh, int width, uint32_t target, uint32_t& path, uint32_t& above) {
  constexpr int kPer = kBins / NT;
  const int tid = threadIdx.x;
  uint32_t c[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = sh.hist[tid * kPer + j];
    mine += c[j];
  }
  uint32_t total;
  const uint32_t incl = block_inclusive_scan<NT>(mine, sh, total);
  const uint32_t above_mine = total - incl;          // bins owned by higher threads
  const uint32_t rank = target - above;
  if (above_mine < rank && rank <= above_mine + mine) {
    uint32_t cum = above_mine;
#pragma unroll
    for (int j = kPer - 1; j >= 0; --j) {
      if (cum + c[j] >= rank) {
        sh.pick[0] = (uint32_t)(tid * kPer + j);
        sh.pick[1] = cum;
        sh.pick[2] = c[j];
        break;
      }
      cum += c[j];
    }
  }
  __syncthreads();
  const uint32_t b = sh.pick[0];
  above += sh.pick[1];
  __syncthreads();
  path = (path << width) | b;
}

// hist[bin] += 1 for every active lane.  Lanes whose bin is the first active
// lane's add together with one atomic: runs of equal keys (ties, or a digit
// all the keys share) would otherwise queue on one LDS address, 64 per wave.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin) {
  const uint32_t lead = __builtin_amdgcn_readfirstlane(bin);
  const bool same = bin == lead;
  const uint64_t m = ballot(same);
  if (same) {
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (below == 0u) atomicAdd(&hist[lead], (uint32_t)popc64(m));
  } else {
    atomicAdd(&hist[bin], 1u);
  }
}

// One radix level over keys produced by `visit(f)`, which calls f(key, valid)
// for each key this thread owns.  Keys off `path` (and invalid ones) count
// into the lane's private dummy bin so the atomics need no branch.
template <int NT, class Sh, class Visit>
__device__ __forceinline__ void radix_level(Sh& sh, int top, int lo, uint32_t target, uint32_t& path,
                            uint32_t& above, Visit visit) {
  const int width = top - lo;
  const uint32_t digit_mask = (1u << width) - 1u;
  for (int b = threadIdx.x; b < kBins + kWave; b += NT) sh.hist[b] = 0u;
  __syncthreads();
  const uint32_t dummy = (uint32_t)(kBins + lane_id());
  // an opaque copy stops the compiler from keeping per-key masks alive
  uint32_t pth = path;
  asm volatile("" : "+v"(pth));
  visit([&](uint32_t k, bool valid) {
    const bool on = valid && (top >= 32 || (k >> top) == pth);
    hist_add(sh.hist, on ? ((k >> lo) & digit_mask) : dummy);
  });
  __syncthreads();
  pick_bin<NT>(sh, width, target, path, above);
}

// Exact threshold among the n keys of the LDS list (n <= NT, list padded with
// zero keys to a multiple of 4): each thread ranks its own key against the
// whole list (broadcast LDS reads), and the thread holding the key of
// 1-based rank `rank` publishes it.  Returns t, gt = #list keys > t and
// eq = #list keys == t.
template <int NT, class Sh>
__device__ void rank_in_list(Sh& sh, uint32_t n, uint32_t rank, uint32_t& t, uint32_t& gt_out,
                             uint32_t& eq_out) {
  const int tid = threadIdx.x;
  if ((tid & ~(kWave - 1)) < (int)n) {             // waves holding no list key skip
    const uint32_t k = tid < (int)n ? sh.list[tid] : 0u;
    uint32_t gt = 0, ge = 0;
    const uint32_t n4 = (n + 3u) & ~3u;
    for (uint32_t j = 0; j < n4; j += 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(&sh.list[j]);
      gt += (x.x > k) + (x.y > k) + (x.z > k) + (x.w > k);
      ge += (x.x >= k) + (x.y >= k) + (x.z >= k) + (x.w >= k);
    }
    // threads holding equal keys write equal values
    if (tid < (int)n && gt < rank && rank <= ge) {
      sh.pick[0] = k;
      sh.pick[1] = gt;
      sh.pick[2] = ge - gt;
    }
  }
  __syncthreads();
  t = sh.pick[0];
  gt_out = sh.pick[1];
  eq_out = sh.pick[2];
  __syncthreads();
}

// Remaining levels of the exact threshold search, given the first-level bin
// `path` (digit key >> 20) and `above` = #keys in higher bins.  Keys of that
// bin (usually ~1% of the keys) are compacted into an LDS list -- counted per
// thread, offsets from one block scan, then written -- and the threshold is
// found there: by direct ranking when the list is short, else by two more
// radix levels; if the bin overflows the list, those levels run over `visit`.
// Returns t (the target-th largest key), need = target - #keys > t (how many
// keys equal to t are selected) and eq = #keys == t.
template <int NT, class Sh, class Visit>
__device__ __forceinline__ void resolve_bin(Sh& sh, uint32_t target, uint32_t path, uint32_t above,
                            uint32_t& t_out, uint32_t& need_out, uint32_t& eq_out, Visit visit) {
  const int tid = threadIdx.x;
  const uint32_t b1 = path;
  const uint32_t nbin = sh.pick[2];                  // the bin's count, from pick_bin
  if (nbin <= (uint32_t)kRankMax && nbin <= (uint32_t)NT && nbin + 4 <= (uint32_t)Sh::kCap) {
    // A short bin (the usual case): its keys take list slots in any order
    // (ranking does not need their order), one atomic slot each, and are
    // ranked directly -- no count pass and no block scan.
    if (tid == 0) sh.pick[3] = 0u;
    if (tid < 4) sh.list[nbin + tid] = 0u;           // pad for rank_in_list
    __syncthreads();
    visit([&](uint32_t k, bool valid) {
      if (valid && (k >> kTopShift) == b1) sh.list[atomicAdd(&sh.pick[3], 1u)] = k;
    });
    __syncthreads();
    uint32_t t, gt, eq;
    rank_in_list<NT>(sh, nbin, target - above, t, gt, eq);
    t_out = t;
    need_out = target - above - gt;
    eq_out = eq;
    return;
  }
  uint32_t cnt = 0;
  visit([&](uint32_t k, bool valid) { cnt += (valid && (k >> kTopShift) == b1) ? 1u : 0u; });
  uint32_t n;
  uint32_t off = block_inclusive_scan<NT>(cnt, sh, n) - cnt;
  if (n <= (uint32_t)Sh::kCap) {
    visit([&](uint32_t k, bool valid) {
      if (valid && (k >> kTopShift) == b1) sh.list[off++] = k;
    });
    if (tid < 4 && n + tid < (uint32_t)Sh::kCap) sh.list[n + tid] = 0u;   // pad for rank_in_list
  }
  __syncthreads();
  if (n <= (uint32_t)kRankMax && n <= (uint32_t)NT) {
    uint32_t t, gt, eq;
    rank_in_list<NT>(sh, n, target - above, t, gt, eq);
    t_out = t;
    need_out = target - above - gt;
    eq_out = eq;
    return;
  }
  if (n <= (uint32_t)Sh::kCap) {
    auto list_visit = [&](auto&& f) {
      for (uint32_t j = tid; j < n; j += NT) f(sh.list[j], true);
    };
    radix_level<NT>(sh, kTopShift, 8, target, path, above, list_visit);
    radix_level<NT>(sh, 8, 0, target, path, above, list_visit);
  } else {
    radix_level<NT>(sh, kTopShift, 8, target, path, above, visit);
    radix_level<NT>(sh, 8, 0, target, path, above, visit);
  }
  t_out = path;
  need_out = target - above;
  eq_out = sh.pick[2];
  __syncthreads();
}

// Exact threshold search from the first-level histogram in sh.hist.
template <int NT, class Sh, class Visit>
__device__ __forceinline__ void finish_threshold(Sh& sh, uint32_t target, uint32_t& t_out, uint32_t& need_out,
                                 uint32_t& eq_out, Visit visit) {
  uint32_t path = 0, above = 0;
  pick_bin<NT>(sh, kDigitBits, target, path, above);
  resolve_bin<NT>(sh, target, path, above, t_out, need_out, eq_out, visit);
}

// Emit, in register order (i, wave, lane) -- which callers make equal to
// position order -- the selected keys: every key > t and the first `need`
// keys == t.  emit(i, sel, slot) is called for every key (branch-free callers
// write unselected keys to a scratch slot); slot = number of selected keys
// before this one.  When every key == t is selected (need == eq, the usual
// case) selection is the single predicate key >= t, one ballot per row.
template <int NT, int K, class EmitFn>
__device__ __forceinline__ void emit_in_order(const uint32_t (&key)[K], uint32_t t, uint32_t need,
                                              uint32_t eq, SelectShared<NT>& sh, EmitFn emit) {
  constexpr int W = NT / kWave;
  static_assert(K * W <= NT, "segments");
  const int tid = threadIdx.x, w = tid / kWave;
  const bool single = need == eq;                 // block-uniform
  // pass 1: per (row, wave) counts, wave-major so pass 2 reads them at once
#pragma unroll
  for (int i = 0; i < K; ++i) {
    uint32_t v;
    if (single) {
      v = (uint32_t)popc64(ballot(key[i] >= t));
    } else {
      v = (uint32_t)popc64(ballot(key[i] > t)) | ((uint32_t)popc64(ballot(key[i] == t)) << 16);
    }
    sh.seg[w * K + i] = v;                        // same value from every lane
  }
  __syncthreads();
  // exclusive scan in (row, wave) order
  if constexpr (K <= 16) {
    // by one wave: lane l takes entries E l .. E l + E - 1 of that order
    // (all its reads before its writes); two barriers fewer than the
    // workgroup's scan
    if (w == 0) {
      constexpr int E = (K * W + kWave - 1) / kWave;
      const int lane = lane_id();
      uint32_t c[E], sum = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = E * lane + e, sr = f / W, sw = f % W;
        c[e] = f < K * W ? sh.seg[sw * K + sr] : 0u;
        sum += c[e];
      }
      uint32_t ex = wave_inclusive_scan(sum) - sum;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int f = E * lane + e, sr = f / W, sw = f % W;
        if (f < K * W) sh.seg[sw * K + sr] = ex;
        ex += c[e];
      }
    }
  } else {
    // (more keys per thread leave no registers for the one-wave form)
    const int sr = tid / W, sw = tid % W;
    const uint32_t v = tid < K * W ? sh.seg[sw * K + sr] : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(v, sh, total);
    __syncthreads();
    if (tid < K * W) sh.seg[sw * K + sr] = incl - v;
  }
  __syncthreads();
  uint32_t pre[K];
#pragma unroll
  for (int i = 0; i < K; ++i) pre[i] = sh.seg[w * K + i];
  // an opaque copy of t keeps the compiler from carrying pass 1's ballot
  // masks (scalar register pairs) into this pass
  uint32_t t2 = t;
  asm volatile("" : "+v"(t2));
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (single) {
      const bool sel = key[i] >= t2;
      const uint32_t slot = pre[i] + (uint32_t)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(ballot(sel) >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ballot(sel), 0u));
      emit(i, sel, slot);
    } else {
      const bool gt = key[i] > t2, eqk = key[i] == t2;
      const uint64_t mg = ballot(gt), me = ballot(eqk);
      const uint32_t gtb = (pre[i] & 0xFFFFu) +
          __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
      const uint32_t eqb = (pre[i] >> 16) +
          __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
      emit(i, gt || (eqk && eqb < need), gtb + min(eqb, need));
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ merge

// A unit's valid chunk candidates are compacted, in chunk order, into a dense
// LDS tile of up to kMergeTile (key, position) pairs -- 128 KB of gfx950's
// 160 KB -- so every pass below is a short loop over LDS.  Dense index order
// equals ascending position order.  Units with more valid candidates than one
// tile re-stage each tile per pass.
struct MergeLds {
  uint32_t key[kMergeTile];
  int32_t pos[kMergeTile];
  uint32_t hist[kBins + kWave];
  static constexpr int kCap = kMergeListCap;
  alignas(16) uint32_t list[kCap];
  int32_t off[kMaxSplits + 1];   // dense offset of each chunk's candidates
  uint32_t seg[kMergeThreads];
  uint32_t wtot[kMergeThreads / kWave];
  uint32_t pick[3];
};

// Copy dense candidates [d0, d0 + n) of unit u into the LDS tile.
__device__ void stage_tile(const SelectArgs& a, int u, MergeLds& sh, int d0, int n) {
  constexpr int NT = kMergeThreads;
  const uint32_t* ck = a.cand_key + (size_t)u * a.S * a.ms;
  const int32_t* cp = a.cand_pos + (size_t)u * a.S * a.ms;
  __syncthreads();
  int s = 0;
  {
    int lo = 0, hi = a.S;              // largest s with off[s] <= d0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sh.off[mid] <= d0) lo = mid; else hi = mid;
    }
    s = lo;
  }
  for (; s < a.S && sh.off[s] < d0 + n; ++s) {
    const int b0 = max(sh.off[s], d0), b1 = min(sh.off[s + 1], d0 + n);
    const int src = s * a.ms - sh.off[s];
#pragma unroll 4
    for (int d = b0 + threadIdx.x; d < b1; d += NT) {
      sh.key[d - d0] = ck[src + d];
      sh.pos[d - d0] = cp[src + d];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const SelectArgs a) {
  constexpr int NT = kMergeThreads;
  constexpr int W = NT / kWave;
  constexpr int kRows = kMergeTile / NT;
  __shared__ MergeLds sh;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave;
  const int S = a.S, M = a.M;

  for (int b = tid; b < kBins + kWave; b += NT) sh.hist[b] = 0u;

  // dense offsets of the chunks' candidate lists (exclusive scan of counts)
  const int spt = (S + NT - 1) / NT;    // chunks per thread, contiguous
  uint32_t my = 0;
  for (int j = 0; j < spt; ++j) {
    const int s = tid * spt + j;
    if (s < S) my += (uint32_t)a.cand_cnt[(size_t)u * S + s];
  }
  uint32_t nvalid;
  uint32_t run = block_inclusive_scan<NT>(my, sh, nvalid) - my;
  for (int j = 0; j < spt; ++j) {
    const int s = tid * spt + j;
    if (s < S) {
      sh.off[s] = (int)run;
      run += (uint32_t)a.cand_cnt[(size_t)u * S + s];
    }
  }
  if (tid == 0) sh.off[S] = (int)nvalid;
  __syncthreads();

  int32_t* idx_u = a.idx + (size_t)u * M;
  const uint32_t target = min(nvalid, (uint32_t)M);
  const int ntiles = ((int)nvalid + kMergeTile - 1) / kMergeTile;
  auto tile_n = [&](int tile) { return min((int)nvalid - tile * kMergeTile, kMergeTile); };
  const bool select = nvalid > (uint32_t)M;
  const uint32_t dummy = (uint32_t)(kBins + lane_id());

  // stage (single tile) and build the first-level histogram on the way
  if (ntiles == 1) {
    const int flat_n = S * a.ms;
    if (flat_n <= kMergeTile) {
      // one batch of loads over the whole [S][ms] array (all in flight), then
      // scatter the valid entries to their dense slots
      constexpr int K = kMergeTile / NT;
      const uint32_t* ck = a.cand_key + (size_t)u * flat_n;
      const int32_t* cp = a.cand_pos + (size_t)u * flat_n;
      uint32_t kv[K];
      int32_t pv[K];
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const int f = min(i * NT + tid, flat_n - 1);
        kv[i] = ck[f];
        pv[i] = cp[f];
      }
      const int ms = a.ms;
      const float inv_ms = 1.0f / (float)ms;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        // chunk of flat slot f: f / ms via a float reciprocal (f < 2^24, so
        // the estimate is off by at most one) and an exact correction
        const int f = i * NT + tid;
        int sc = (int)((float)f * inv_ms);
        sc -= (sc * ms > f) ? 1 : 0;
        sc += ((sc + 1) * ms <= f) ? 1 : 0;
        const int slot = f - sc * ms;
        const bool valid = f < flat_n && sc < S && slot < sh.off[sc + 1] - sh.off[sc];
        if (valid) {
          const int d = sh.off[sc] + slot;
          sh.key[d] = kv[i];
          sh.pos[d] = pv[i];
        }
        if (select) atomicAdd(&sh.hist[valid ? (kv[i] >> kTopShift) : dummy], 1u);
      }
      __syncthreads();
    } else {
      stage_tile(a, u, sh, 0, (int)nvalid);
      if (select) {
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
          const int j = i * NT + tid;
          atomicAdd(&sh.hist[j < (int)nvalid ? (sh.key[j] >> kTopShift) : dummy], 1u);
        }
        __syncthreads();
      }
    }
  } else if (select) {
    for (int tile = 0; tile < ntiles; ++tile) {
      stage_tile(a, u, sh, tile * kMergeTile, tile_n(tile));
      const int n = tile_n(tile);
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        const int j = i * NT + tid;
        atomicAdd(&sh.hist[j < n ? (sh.key[j] >> kTopShift) : dummy], 1u);
      }
    }
    __syncthreads();
  }

  // without selection every staged candidate (key >= 1) is emitted
  uint32_t t = 1, need = 0, eq = 0;
  if (select) {
    auto visit_all = [&](auto&& f) {
      for (int tile = 0; tile < ntiles; ++tile) {
        if (ntiles > 1) stage_tile(a, u, sh, tile * kMergeTile, tile_n(tile));
        const int n = tile_n(tile);
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
          const int j = i * NT + tid;
          f(sh.key[min(j, n - 1)], j < n);
        }
      }
    };
    finish_threshold<NT>(sh, target, t, need, eq, visit_all);
  }

  // Ordered emission: row i of thread (w, lane) is dense index i*NT + 64w + lane,
  // so (row, wave, lane) order is ascending position order.  Output slots are
  // staged in LDS (the histogram region is free now; unselected entries go to
  // a per-lane scratch slot past the real ones) when they fit, then written
  // with contiguous stores.
  const bool single = need == eq;                 // selection is key >= t
  const bool staged = target <= (uint32_t)kBins;
  int32_t* out = staged ? reinterpret_cast<int32_t*>(sh.hist) : idx_u;
  const int lane = lane_id();
  __syncthreads();
  uint32_t gt_base = 0, eq_base = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    if (ntiles > 1) stage_tile(a, u, sh, tile * kMergeTile, tile_n(tile));
    const int n = tile_n(tile);
    const int rows = (n + NT - 1) / NT;             // <= kRows
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int j = i * NT + tid;
      const uint32_t k = sh.key[min(j, n - 1)];
      uint32_t v;
      if (single) {
        v = (uint32_t)popc64(ballot(j < n && k >= t));
      } else {
        v = (uint32_t)popc64(ballot(j < n && k > t)) |
            ((uint32_t)popc64(ballot(j < n && k == t)) << 16);
      }
      if (i < rows) sh.seg[w * kRows + i] = v;      // same value from every lane
    }
    __syncthreads();
    const int sr = tid / W, sw = tid % W;
    const uint32_t v = tid < rows * W ? sh.seg[sw * kRows + sr] : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(v, sh, total);
    __syncthreads();
    if (tid < rows * W) sh.seg[sw * kRows + sr] = incl - v;
    __syncthreads();
    uint32_t pre[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) pre[i] = sh.seg[w * kRows + i];
    uint32_t t2 = t;
    asm volatile("" : "+v"(t2));
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (i >= rows) break;                         // block-uniform
      const int j = i * NT + tid;
      const uint32_t k = sh.key[min(j, n - 1)];
      const int32_t p = sh.pos[min(j, n - 1)];
      bool sel;
      uint32_t slot;
      if (single) {
        sel = j < n && k >= t2;
        const uint64_t m = ballot(sel);
        slot = gt_base + pre[i] +
               __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      } else {
        const bool gt = j < n && k > t2, eqk = j < n && k == t2;
        const uint64_t mg = ballot(gt), me = ballot(eqk);
        const uint32_t gtb = gt_base + (pre[i] & 0xFFFFu) +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, 0u));
        const uint32_t eqb = eq_base + (pre[i] >> 16) +
            __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
        sel = gt || (eqk && eqb < need);
        slot = gtb + min(eqb, need);
      }
      if (staged) out[sel ? slot : (uint32_t)(kBins + lane)] = p;
      else if (sel) out[slot] = p;
    }
    if (single) {
      gt_base += total;
    } else {
      gt_base += total & 0xFFFFu;
      eq_base += total >> 16;
    }
    __syncthreads();
  }
  if (staged)
    for (int slot = tid; slot < (int)target; slot += NT) idx_u[slot] = out[slot];
  for (int slot = (int)target + tid; slot < M; slot += NT) idx_u[slot] = -1;
}

// Register-resident merge, used when a unit's candidate slots fit KPT rows of
// the 1024-thread workgroup (S * ms <= 1024 * KPT, ms a multiple of 1024).
// Slot f of the flat [S][ms] candidate array is key register f / 1024 of
// thread f % 1024, so register order (i, wave, lane) is ascending position
// order (chunks are in position order and so is each chunk's list); slots
// past a chunk's count hold key 0 ("no position").  Selection then runs
// exactly as in a chunk: first-level histogram, threshold, ordered emission.
template <int KPT>
__global__ __launch_bounds__(kMergeThreads) void merge_regs_kernel(const SelectArgs a) {
  constexpr int NT = kMergeThreads;
  __shared__ SelectShared<NT> sh;
  __shared__ int32_t cnt_s[kMaxMergeKeysPerThread];
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id();
  const int S = a.S, M = a.M;
  const int rows_per_chunk = a.ms / NT;
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  if (tid < S) cnt_s[tid] = a.cand_cnt[(size_t)u * S + tid];
  __syncthreads();
  uint32_t nvalid = 0;
  for (int c = 0; c < S; ++c) nvalid += (uint32_t)cnt_s[c];
  const uint32_t* ck = a.cand_key + (size_t)u * S * a.ms;
  const int32_t* cp = a.cand_pos + (size_t)u * S * a.ms;
  uint32_t key[KPT];
  int32_t pos[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = i / rows_per_chunk;
    const int slot = (i - c * rows_per_chunk) * NT + tid;
    const bool valid = c < S && slot < cnt_s[min(c, S - 1)];
    const size_t f = (size_t)i * NT + tid;
    key[i] = valid ? ck[f] : 0u;
    pos[i] = valid ? cp[f] : -1;
  }
  const bool select = nvalid > (uint32_t)M;
  const uint32_t target = min(nvalid, (uint32_t)M);
  if (select) {
    const uint32_t dummy = (uint32_t)(kBins + lane);
#pragma unroll
    for (int i = 0; i < KPT; ++i) atomicAdd(&sh.hist[key[i] ? (key[i] >> kTopShift) : dummy], 1u);
    __syncthreads();
  }
  // without selection every candidate (key >= 1) is emitted
  uint32_t t = 1, need = 0, eq = 0;
  if (select) {
    finish_threshold<NT>(sh, target, t, need, eq, [&](auto&& f) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) f(key[i], key[i] != 0u);
    });
  }
  int32_t* idx_u = a.idx + (size_t)u * M;
  const bool staged = target <= (uint32_t)(kListCap - kWave);
  int32_t* out = reinterpret_cast<int32_t*>(sh.list);
  emit_in_order(key, t, need, eq, sh, [&](int i, bool sel, uint32_t slot) {
    if (staged) out[sel ? slot : (uint32_t)(kListCap - kWave + lane)] = pos[i];
    else if (sel) idx_u[slot] = pos[i];
  });
  if (staged)
    for (int j = tid; j < (int)target; j += NT) idx_u[j] = out[j];
  for (int j = (int)target + tid; j < M; j += NT) idx_u[j] = -1;
}

// ------------------------------------------------------------------ chunks

// One chunk of one unit: keys, chunk-local exact top-M, candidates out.
// Key register i of thread (wave w, lane l) is position base + i*NT + 64w + l.
// The first-level radix histogram is built while the keys are produced, so
// it hides under the memory stream.
template <int D, int R, int KPT, bool FUSED>
__global__ __launch_bounds__(kChunkThreads, 4) void chunk_select_kernel(const SelectArgs a) {
  constexpr int NT = kChunkThreads;
  __shared__ SelectShared<NT> sh;
  const int u = blockIdx.x / a.S, c = blockIdx.x % a.S;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int len = a.seq_lens ? min(max(a.seq_lens[b], 0), a.n_max) : a.n_max;
  const int base = c * a.chunk;
  const int nv = min(max(len - base, 0), a.chunk);
  const bool select = nv > a.M;
  const uint32_t dummy = (uint32_t)(kBins + lane);
  int nsel = 0;

  if (nv > 0) {                                   // block-uniform
    for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
    uint32_t key[KPT];
    if (FUSED) {
      // this chunk's rows only: loads past the valid positions return zero
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(a.kp + ((size_t)u * a.Ncap + base) * R, (uint32_t)nv * R);
      // lane byte offset within one wave's 64 positions; r=32 lanes pair up
      // on a position (first half of the wave's rows: +0, second: +1024)
      const uint32_t voff = (uint32_t)(w * kWave * R + lane * 16);
      constexpr int kLoadsPerIter = R / 16;
      constexpr int kPerBatch = SA_CHUNK_LOADS_IN_FLIGHT / kLoadsPerIter;
      constexpr int kBatch = (KPT < kPerBatch) ? KPT : kPerBatch;
      uint4 ca[kBatch], cb[kBatch];
      auto load_batch = [&](int i0) {
#pragma unroll
        for (int x = 0; x < kBatch; ++x) {
          // the whole offset is in the lane offset: the hardware range check
          // covers the vector and immediate offsets, not the scalar one
          const uint32_t off = voff + (uint32_t)((i0 + x) * NT * R);
          ca[x] = buffer_load16(rs, off, 0);
          if (R == 32) cb[x] = buffer_load16(rs, off + 1024, 0);
        }
      };
      // the first batch is in flight while the indexer query is formed (its
      // barriers also order the histogram clearing above)
      load_batch(0);
      indexer_query<D, R, NT>(a.q, a.P, b, h, a.G, a.Hq, sh.qt, sh.part);
      float ql[16];
      lane_query<R>(sh.qt, ql);
#pragma unroll
      for (int i0 = 0; i0 < KPT; i0 += kBatch) {
        if (i0 > 0) load_batch(i0);
#pragma unroll
        for (int x = 0; x < kBatch; ++x) {
          const int i = i0 + x;
          const int p = base + i * NT + w * kWave + lane;
          float s;
          if (R == 16) {
            s = lane_score<R>(ql, ca[x]);
          } else {
            const float sa = lane_score<R>(ql, ca[x]);
            const float sb = lane_score<R>(ql, cb[x]);
            // lane l takes position p0 + l: from lane 2l of the first half
            // (l < 32) or lane 2(l-32)+1 of the second
            const float xv = (lane & 1) ? sb : sa;
            const int src = (lane < 32) ? 2 * lane : 2 * (lane - 32) + 1;
            s = __shfl(xv, src, kWave);
          }
          key[i] = p < len ? score_key(s + 0.0f) : 0u;
          if (select) atomicAdd(&sh.hist[p < len ? (key[i] >> kTopShift) : dummy], 1u);
        }
      }
    } else {
      const float* su = a.scores + (size_t)u * a.n_max + base;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(su, (uint32_t)nv * 4u);
      __syncthreads();                            // histogram cleared
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int p = base + i * NT + w * kWave + lane;
        const float sv = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, (i * NT + w * kWave + lane) * 4, 0, 0));
        key[i] = p < len ? score_key(sv + 0.0f) : 0u;
        if (select) atomicAdd(&sh.hist[p < len ? (key[i] >> kTopShift) : dummy], 1u);
      }
    }

    // without selection every valid key (key >= 1) is emitted
    uint32_t t = 1, need = 0, eq = 0;
    if (select) {
      __syncthreads();
      uint32_t path = 0, above = 0;
      pick_bin<NT>(sh, kDigitBits, (uint32_t)a.M, path, above);
      const uint32_t in_bin = sh.pick[2];
      if (above + in_bin <= (uint32_t)a.ms) {
        // Superset: every key of the first-level bin holding the M-th largest
        // key, and every higher key.  It contains the chunk's exact top-M; the
        // merge selects exactly over the union.
        t = max(path << kTopShift, 1u);           // key 0 marks no position
        nsel = (int)(above + in_bin);
      } else {
        resolve_bin<NT>(sh, (uint32_t)a.M, path, above, t, need, eq, [&](auto&& f) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) f(key[i], key[i] != 0u);
        });
        nsel = a.M;
      }
    } else {
      nsel = nv;
    }
    uint32_t* ck = a.cand_key + ((size_t)u * a.S + c) * a.ms;
    int32_t* cp = a.cand_pos + ((size_t)u * a.S + c) * a.ms;
    if (nsel <= kStageSlots) {
      // compact in LDS (the list region is free now; unselected keys go to a
      // per-lane scratch slot past the real ones), then write out with
      // whole-wave contiguous stores
      uint32_t* lk = sh.list;
      uint32_t* lp = sh.list + kListCap / 2;
      emit_in_order(key, t, need, eq, sh, [&](int i, bool sel, uint32_t slot) {
        const uint32_t d = sel ? slot : (uint32_t)(kStageSlots + lane);
        lk[d] = key[i];
        lp[d] = (uint32_t)(base + i * NT + w * kWave + lane);
      });
      for (int j = tid; j < nsel; j += NT) {
        ck[j] = lk[j];
        cp[j] = (int32_t)lp[j];
      }
    } else {
      emit_in_order(key, t, need, eq, sh, [&](int i, bool sel, uint32_t slot) {
        if (sel) {
          ck[slot] = key[i];
          cp[slot] = base + i * NT + w * kWave + lane;
        }
      });
    }
  }
  if (tid == 0) a.cand_cnt[(size_t)u * a.S + c] = nsel;
}

// ------------------------------------------------------------------ filter path
//
// The fused selection's main path for contexts up to 2^19 positions:
//  1. bound (sample_kernel, or append_bound_kernel in the decode step): per
//     unit, score 128 evenly spread blocks of 8 positions and take the k-th
//     largest sample key, k ~ 3 M (sample size) / len, as a bound thr that
//     about 3M keys of the unit reach (the whole unit when it has at most
//     1024 positions: then k = M and thr is the exact M-th key).
//  2. filter_kernel: chunks of the unit stream their FP8 rows (or the given
//     scores), score every position and append each score >= thr, with its
//     position, to an LDS list of the wave that scored it (ballot + bit
//     count, no key held in registers); a list that fills up goes to the
//     unit's spill pool (clustered high scores); once every wave has
//     finished reading, the 8 lists go out back to back as the chunk's
//     candidates, packed (key, position) pairs in no particular order.
//  3. merge (filter_merge_kernel, or select_attend_kernel in the decode
//     step): if the kept keys fit the merge (chunk lists plus spill pool) and
//     at least M of them reached thr, then thr <= the M-th largest key of the
//     unit, so the candidates hold every selected position; they are loaded
//     into registers, the exact M-th key is found among them and idx is
//     emitted through a bitmap of positions.  Otherwise the workgroup selects
//     exactly by streaming the unit's rows again and marking the selection in
//     the bitmap (slow but rare).
// Keys are bit-identical to the chunk-exact path's, so both give the same idx.

// Inclusive prefix sum over the block in thread order (wtot: NT/64 words of LDS).
template <int NT>
__device__ __forceinline__ uint32_t block_scan_small(uint32_t v, uint32_t* wtot, uint32_t& total) {
  constexpr int W = NT / kWave;
  const int w = threadIdx.x / kWave;
  const uint32_t inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane_id() == kWave - 1) wtot[w] = inc;
  __syncthreads();
  uint32_t wb = 0, tot = 0;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) {
    wb += ww < w ? wtot[ww] : 0u;
    tot += wtot[ww];
  }
  total = tot;
  return wb + inc;
}

// A position's score comes from its FP8 code row (R = 16 or 32 codes,
// scored against the unit's indexer query) or, for a selection over scores
// the caller already holds (sparse_attn_topm), from one fp32 value per
// position: R = kScoreInput.
constexpr int kScoreInput = 1;

struct FilterArgs {
  const uint16_t* q;
  const float* P;
  const uint8_t* kp;
  const float* scores;   // [units][n_max] when R == kScoreInput
  const int32_t* seq_lens;
  int n_max, Ncap, Hq, Hkv, G, M, S, chunk, cap, cslots, spill_cap;
  int units;         // B * Hkv
  int64_t ustride;   // pairs per unit in cand: S * cslots, then spill_cap
  uint32_t* thr;     // [units]
  float* qt;         // [units][32] indexer queries (written by the bound stage)
  int32_t* path;     // [units] how the merge selected: 0 from the kept keys, 1 by the
                     // exact streaming pass (a diagnostic, read by sparse_attn_selection_fallbacks)
  int32_t* cnt;      // [units][S + 1] kept positions per chunk (-1 when a wave list
                     // overflowed), then the pairs reserved in the spill pool (zeroed by
                     // the bound stage)
  uint2* cand;       // per unit: [S][cslots] (key, position) of the kept positions (any
                     // order), then the spill pool [spill_cap] of lists that filled up
  float* sc;         // the score-all plan: [units][sstride] scores, position order
  int64_t sstride;
  int32_t* idx;
};

constexpr int kSampleThreads = kMergeThreads;
constexpr int kSampleKeys = kSampleBlocks * kSampleBlock / kSampleThreads;
constexpr int kBitmapWords = kFilterMaxN / 32;
constexpr int kFilterMergeKeys = kFilterSlots / kMergeThreads;   // 16 per thread
static_assert(kFilterMaxCap * kFilterWaves <= kFilterSlots, "a chunk's slots fit the merge");
constexpr int kFilterMaxSplits = kFilterSlots / (kFilterWaves * kFilterMinCap);   // 16
static_assert(kFilterMaxSplits <= kWave && (kFilterMaxSplits & (kFilterMaxSplits - 1)) == 0,
              "one wave scans the chunk counts; chunks are found by bisection");
// bisection table of the merge: the chunks' starts, then the spill pool's
constexpr int kMergeStarts = 2 * kFilterMaxSplits;
static_assert(kMergeStarts <= kWave, "one wave writes the table");

__device__ __forceinline__ int unit_len(const int32_t* seq_lens, int b, int n_max) {
  return seq_lens ? min(max(seq_lens[b], 0), n_max) : n_max;
}

// Score of one whole position by one thread: the same 16-code chains, added
// in the same order, as the paired-lane scoring of the chunk-exact kernel,
// hence the same bits.
template <int R>
__device__ __forceinline__ float position_score(const float (&qlo)[16], const float (&qhi)[16],
                                                const uint8_t* row) {
  const uint4 c0 = load16(row);
  float s = score16(qlo, c0);
  if (R == 32) s = s + score16(qhi, load16(row + 16));
  return s;
}

template <int R>
__device__ __forceinline__ void query_halves(const float* qt, float (&qlo)[16], float (&qhi)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    qlo[k] = qt[k];
    qhi[k] = R == 32 ? qt[16 + k] : 0.0f;
  }
}

// ------------------------------------------------------------------ scores

// sparse_attn_index_score: the filter stage's stream without the filter.
// Each 512-thread workgroup forms the unit's query (indexer_query: the same
// bits in every kernel) and scores a chunk of 2048 positions, lane l of wave
// w position base + i*512 + 64w + l on its own (both 16-byte halves of an
// r = 32 row; the chains of position_score), two rows of loads in flight;
// every position n < n_max gets one coalesced 4-byte store (-inf from len_b
// on).  Small chunks, many workgroups: the stores of one spread out over the
// reads of the others (measured at 128K: 2048 positions 222 us, 8192 236,
// 32768 253, 1024 232; pairs of lanes per position over 8192, 243).
constexpr int kScoreThreads = 512;
constexpr int kScorePositionsPerBlock = 2048;

template <int D, int R>
__global__ __launch_bounds__(kScoreThreads) void index_score_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ P, const uint8_t* __restrict__ kp,
    const int32_t* __restrict__ seq_lens, int n_max, int Ncap, int Hq, int Hkv, int G,
    int blocks_per_unit, float* __restrict__ scores) {
  constexpr int NT = kScoreThreads;
  __shared__ float qt[32];
  __shared__ double part[NT];
  const int u = blockIdx.x / blocks_per_unit, blk = blockIdx.x % blocks_per_unit;
  const int b = u / Hkv, h = u % Hkv;
  const int tid = threadIdx.x;
  const int len = seq_lens ? min(max(seq_lens[b], 0), n_max) : n_max;
  const int base = blk * kScorePositionsPerBlock;
  const int nw = min(n_max - base, kScorePositionsPerBlock);     // positions written
  const int nv = min(max(len - base, 0), nw);                      // ... of which valid
  // this chunk's valid rows only: loads past them return zero
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(kp + ((size_t)u * Ncap + base) * R, (uint32_t)nv * R);
  const uint32_t voff = (uint32_t)(tid * R);
  const int rows = (nw + NT - 1) / NT;
  uint4 a0 = make_uint4(0u, 0u, 0u, 0u), b0 = a0, a1 = a0, b1 = a0;
  a0 = buffer_load16(rs, voff, 0);
  if (R == 32) b0 = buffer_load16(rs, voff + 16, 0);
  if (rows > 1) {
    a1 = buffer_load16(rs, voff + NT * R, 0);
    if (R == 32) b1 = buffer_load16(rs, voff + NT * R + 16, 0);
  }
  indexer_query<D, R, NT>(q, P, b, h, G, Hq, qt, part);
  float qlo[16], qhi[16];
  query_halves<R>(qt, qlo, qhi);
  float* su = scores + (size_t)u * n_max + base;
  auto put = [&](const uint4& ca, const uint4& cb, int i) {
    const int p = i * NT + tid;                       // within the chunk
    float s = score16(qlo, ca);
    if (R == 32) s = s + score16(qhi, cb);
    if (p < nw) su[p] = base + p < len ? s : -__builtin_inff();
  };
  for (int i = 0; i < rows; i += 2) {                 // block-uniform
    put(a0, b0, i);
    if (i + 2 < rows) {
      a0 = buffer_load16(rs, voff + (uint32_t)((i + 2) * NT * R), 0);
      if (R == 32) b0 = buffer_load16(rs, voff + (uint32_t)((i + 2) * NT * R) + 16, 0);
    }
    if (i + 1 < rows) {
      put(a1, b1, i + 1);
      if (i + 3 < rows) {
        a1 = buffer_load16(rs, voff + (uint32_t)((i + 3) * NT * R), 0);
        if (R == 32) b1 = buffer_load16(rs, voff + (uint32_t)((i + 3) * NT * R) + 16, 0);
      }
    }
  }
}

hipError_t run_index_score(const LaunchCommon& c, const void* q, const float* P,
                           const uint8_t* kp, const int32_t* seq_lens, int n_max,
                           float* scores) {
  const int bpu = (n_max + kScorePositionsPerBlock - 1) / kScorePositionsPerBlock;
  const long blocks = (long)bpu * c.units;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kScoreThreads);
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

// The bound stage for unit u (the whole workgroup; it synchronises).
// prologue() runs while the sampled rows are in flight (every thread calls
// it) and leaves the unit's indexer query in sh.qt.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// after_sample() runs once the sample has been scored (every global load of
// the bound has returned), before its selection (LDS work only).
template <int D, int R, class Prologue, class AfterSample = NoHook>
__device__ __forceinline__ uint32_t sample_bound(const FilterArgs& a,
                                                 SelectShared<kSampleThreads>& sh, int u,
                                                 Prologue prologue,
                                                 AfterSample after_sample = AfterSample()) {
  constexpr int NT = kSampleThreads;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x;
  const int len = unit_len(a.seq_lens, b, a.n_max);
  if (tid == 0) a.cnt[(size_t)u * (a.S + 1) + a.S] = 0;   // the filter reserves spill from 0
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  // blocks of 8 consecutive positions, evenly spread over [0, len); the row
  // loads go out first
  constexpr int kTotal = kSampleBlocks * kSampleBlock;
  const bool all = len <= kTotal;
  uint32_t key[kSampleKeys];
  uint4 c0[kSampleKeys], c1[kSampleKeys];
  float sv[kSampleKeys];
  bool ok[kSampleKeys];
#pragma unroll
  for (int i = 0; i < kSampleKeys; ++i) {
    const int slot = i * NT + tid;
    const int blk = slot / kSampleBlock, off = slot % kSampleBlock;
    const int p = all ? slot
                      : (int)(((int64_t)blk * (len - kSampleBlock)) / (kSampleBlocks - 1)) + off;
    ok[i] = p < len && len > a.M;
    if constexpr (R == kScoreInput) {
      sv[i] = a.scores[(size_t)u * a.n_max + (ok[i] ? p : 0)];
    } else {
      const uint8_t* row = a.kp + ((size_t)u * a.Ncap + (ok[i] ? p : 0)) * R;
      c0[i] = load16(row);
      if (R == 32) c1[i] = load16(row + 16);
    }
  }
  prologue();
  if constexpr (R != kScoreInput) {
    if (tid < R) a.qt[(size_t)u * 32 + tid] = sh.qt[tid];
  }
  if (len <= a.M) {                                   // every valid position is selected
    if (tid == 0) a.thr[u] = 1u;
    return 1u;
  }
  if constexpr (R == kScoreInput) {
#pragma unroll
    for (int i = 0; i < kSampleKeys; ++i) key[i] = ok[i] ? score_key(sv[i] + 0.0f) : 0u;
  } else {
    float qlo[16], qhi[16];
    query_halves<R>(sh.qt, qlo, qhi);
#pragma unroll
    for (int i = 0; i < kSampleKeys; ++i) {
      float s = score16(qlo, c0[i]);
      if (R == 32) s = s + score16(qhi, c1[i]);
      key[i] = ok[i] ? score_key(s + 0.0f) : 0u;
    }
  }
  // the k-th largest sample key, k ~ keep * (sample size) / len, so that
  // about keep = min(kSampleSafety M, kFilterKeepTarget) keys of the unit
  // reach it: enough above M for the sample's noise, and well inside the
  // merge's kFilterSlots (a sample of the whole unit gives the exact M-th key)
  const int ns = all ? len : kTotal;
  const int64_t keep = min((int64_t)kSampleSafety * a.M, (int64_t)kFilterKeepTarget);
  if (!all && keep >= len) {                          // keep every position (len < 12288):
    const uint32_t low = score_key(-__builtin_inff());   // the key of -inf, below all
    if (tid == 0) a.thr[u] = low;
    return low;
  }
  uint32_t k = all ? (uint32_t)a.M
                   : (uint32_t)min((int64_t)ns, (keep * ns + len - 1) / len);
  k = max(k, 1u);
  after_sample();
  const uint32_t dummy = (uint32_t)(kBins + lane_id());
#pragma unroll
  for (int i = 0; i < kSampleKeys; ++i)
    atomicAdd(&sh.hist[key[i] ? (key[i] >> kTopShift) : dummy], 1u);
  __syncthreads();
  uint32_t t, need, eq;
  finish_threshold<NT>(sh, k, t, need, eq, [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < kSampleKeys; ++i) f(key[i], key[i] != 0u);
  });
  if (tid == 0) a.thr[u] = t;
  return t;
}

template <int D, int R>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(const FilterArgs a) {
  __shared__ SelectShared<kSampleThreads> sh;
  const int u = blockIdx.x;
  sample_bound<D, R>(a, sh, u, [&] {
    if constexpr (R != kScoreInput)
      indexer_query<D, R, kSampleThreads>(a.q, a.P, u / a.Hkv, u % a.Hkv, a.G, a.Hq, sh.qt,
                                          sh.part);
  });
}

// Decode-step prologue: append the unit's new rows, then the bound stage, in
// one workgroup (the bound is an estimate: whether its sample sees the new
// rows does not matter; the filter and merge that follow do see them).
struct AppendArgs {
  const int32_t* pos;
  int T;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
};

// The unit's new rows t0 .. t1 - 1 (all of them by default) are appended
// (append_row's arithmetic), the first while the indexer query is formed
// (indexer_query's arithmetic); both projections share one load of the
// basis, and every global load of both goes out before the first barrier.
// Further rows follow one at a time.  Leaves the query in qt; part holds
// NT >= 512 + d doubles of LDS.
template <int D, int R, int NT>
__device__ __forceinline__ void append_rows_and_query(const FilterArgs& a, const AppendArgs& ap,
                                                      int u, float* qt, double* part,
                                                      int t0 = 0, int t1 = -1) {
  if (t1 < 0) t1 = ap.T;
  constexpr int kPer = D / kProjParts;
  constexpr int kMeanT = 512;                       // threads [512, 512 + d) form the mean
  static_assert(kProjParts * 32 <= 256 && kMeanT + D <= NT, "thread roles");
  double* part_a = part;                            // [8r] partial sums of the new row's code
  double* part_m = part + 256;                      // [d]  group-mean query
  double* part_q = part + kMeanT;                   // [8r] partial sums of the query
  const int t = threadIdx.x;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int pi = t / R, j = t % R;
  const bool proj = t < kProjParts * R;
  const float* Ph = a.P + (size_t)h * D * R;
  float pv[kPer];
  if (proj) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) pv[k] = Ph[(pi * kPer + k) * R + j];
  }
  if (t >= kMeanT && t < kMeanT + D) {
    const int i = t - kMeanT;
    const uint16_t* qb = a.q + ((size_t)b * a.Hq + (size_t)h * a.G) * D;
    double mean = 0.0;
    for (int g = 0; g < a.G; ++g) mean += (double)__uint_as_float((uint32_t)qb[g * D + i] << 16);
    part_m[i] = mean / (double)a.G;
  }
  const int p0 = ap.pos[b];
  auto row_of = [&](int tok, size_t& row) {
    const long n = (long)p0 + tok;
    row = (size_t)u * a.Ncap + (size_t)n;
    return n >= 0 && n < a.Ncap;                    // block-uniform
  };
  size_t row0 = 0;
  const bool ok0 = t1 > t0 && row_of(t0, row0);
  if (ok0) {
    const uint16_t* kr = ap.k_new + ((size_t)u * ap.T + t0) * D;
    const uint16_t* vr = ap.v_new + ((size_t)u * ap.T + t0) * D;
    if (t < D / 8) {
      const size_t off = row0 * D + t * 8;
      *reinterpret_cast<uint4*>(ap.k_cache + off) = *reinterpret_cast<const uint4*>(kr + t * 8);
      *reinterpret_cast<uint4*>(ap.v_cache + off) = *reinterpret_cast<const uint4*>(vr + t * 8);
    }
    if (proj) {
      float kv[kPer];
#pragma unroll
      for (int k = 0; k < kPer; k += 8)
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(kr + pi * kPer + k), kv + k);
      double acc = 0.0;
#pragma unroll
      for (int k = 0; k < kPer; ++k) acc = fma((double)kv[k], (double)pv[k], acc);
      part_a[t] = acc;
    }
  }
  __syncthreads();
  if (ok0 && t < R) {
    double sum = 0.0;
#pragma unroll
    for (int q = 0; q < kProjParts; ++q) sum += part_a[q * R + t];
    const_cast<uint8_t*>(a.kp)[row0 * R + t] = (uint8_t)f64_to_e4m3(sum);
  }
  if (proj) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc = fma(part_m[pi * kPer + k], (double)pv[k], acc);
    part_q[t] = acc;
  }
  __syncthreads();
  if (t < R) {
    double sum = 0.0;
    for (int q = 0; q < kProjParts; ++q) sum += part_q[q * R + t];
    qt[t] = (float)sum;
  }
  for (int tok = t0 + 1; tok < t1; ++tok) {
    size_t row;
    if (!row_of(tok, row)) continue;
    append_row<D, R>(ap.k_new + ((size_t)u * ap.T + tok) * D,
                     ap.v_new + ((size_t)u * ap.T + tok) * D, Ph, row, ap.k_cache, ap.v_cache,
                     const_cast<uint8_t*>(a.kp) + row * R, part_a);
    __syncthreads();                                // part_a is reused
  }
  __syncthreads();
}

template <int D, int R>
__global__ __launch_bounds__(kSampleThreads) void append_bound_kernel(const FilterArgs a,
                                                                       const AppendArgs ap) {
  __shared__ SelectShared<kSampleThreads> sh;
  const int u = blockIdx.x;
  sample_bound<D, R>(a, sh, u, [&] {
    append_rows_and_query<D, R, kSampleThreads>(a, ap, u, sh.qt, sh.part);
  });
}

// The FP8 code stream is read once: non-temporal loads (measured on a plain
// streaming read: 6.1 TB/s with the default policy, 6.6-7.1 TB/s
// non-temporal, but only when each wave's load covers 1 KB of contiguous
// bytes -- two 16-byte halves of 32-byte rows loaded lane by lane, each load
// spanning 2 KB, lose the gain).
constexpr int kStreamPolicy = 2;   // nt

__device__ __forceinline__ uint4 stream_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const sa_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Scores of the nv code rows (R bytes each) at the start of `rs`, read as
// contiguous 16-byte lanes: in round k the workgroup reads bytes
// [16 NT k, 16 NT (k + 1)), thread t the 16 bytes at 16 NT k + 16 t, that is
// position PR k + 16 t / R (PR = 16 NT / R positions per round) -- for
// r = 32 one half (t & 1) of the row.  The two lanes of an r = 32 row each
// form their half's 16-code chain and add the other's with one DPP step
// (lo + hi and hi + lo are the same sum), and the even lane owns the
// position.  keep(s, p, owner) is called by every lane (a wave-uniform call)
// with p relative to the start; rows past nv read as zero.  L loads per lane
// are in flight: two groups of L / 2 rounds alternate, one scored while the
// other loads.  qt: the unit's 32-float indexer query.
template <int R, int NT, int L>
struct CodeStream {
  static_assert(R == 16 || R == 32, "rank");
  static constexpr int PR = NT * 16 / R;              // positions per round
  static constexpr int H = L / 2 > 0 ? L / 2 : 1;     // rounds per load group
  __amdgpu_buffer_rsrc_t rs;
  int rounds;
  bool issued;
  uint4 ga[H], gb[H];

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t r, int nv) {
    rs = r;
    rounds = (nv + PR - 1) / PR;
    issued = false;
  }
  __device__ __forceinline__ void load(uint4 (&g)[H], int k0) {
#pragma unroll
    for (int x = 0; x < H; ++x)
      g[x] = stream_load16(rs, (uint32_t)((k0 + x) * NT * 16 + threadIdx.x * 16));
  }
  // the first two groups of loads (may be issued early, before the query and
  // the bound are known)
  __device__ __forceinline__ void issue_first() {
    load(ga, 0);
    if (H < rounds) load(gb, H);
    issued = true;
  }
  template <class Keep>
  __device__ __forceinline__ void run(const float* qt, Keep keep) {
    const int t = threadIdx.x;
    const int lane_pos = t * 16 / R;
    const bool owner = R == 16 || (t & 1) == 0;
    float ql[16];
    const int qoff = R == 32 ? 16 * (t & 1) : 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) ql[k] = qt[qoff + k];
    auto score = [&](const uint4 (&g)[H], int k0) {
#pragma unroll
      for (int x = 0; x < H; ++x) {
        float s = score16(ql, g[x]);
        if (R == 32) s = s + dpp_f<kDppQuadSwap1>(s);
        keep(s, (k0 + x) * PR + lane_pos, owner);
      }
    };
    if (!issued) issue_first();
    for (int k0 = 0; k0 < rounds; k0 += 2 * H) {      // block-uniform trip counts
      score(ga, k0);
      if (k0 + 2 * H < rounds) load(ga, k0 + 2 * H);
      if (k0 + H < rounds) {
        score(gb, k0 + H);
        if (k0 + 3 * H < rounds) load(gb, k0 + 3 * H);
      }
    }
  }
};

// CodeStream over the nv rows of `rs` in one call: init, then run.
template <int R, int NT, int L, class Keep>
__device__ __forceinline__ void stream_code_scores(__amdgpu_buffer_rsrc_t rs, int nv,
                                                   const float* qt, Keep keep) {
  CodeStream<R, NT, L> cs;
  cs.init(rs, nv);
  cs.run(qt, keep);
}

// The unit kernel's code stream: CodeStream's loads and scores, handed out
// to the S streaming waves in chunks on demand.  A chunk is H consecutive 1 KB
// wave loads (H KB of contiguous codes, H PW positions); wave w starts on
// chunks w and S + w and takes each further chunk from an LDS counter that
// starts at 2 S.  With a fixed split the waves of one SIMD do not keep pace
// (instruction issue favours the older wave): measured at 131072 positions,
// the later four of eight waves finished 5.8 us after the first four, whose
// memory-level parallelism the tail then lacked.  On demand, the waves end
// within a chunk of each other.  Loads past nv read as zero; keep(s, p, owner)
// as for CodeStream.
template <int R, int L>
struct WaveStream {
  static_assert(R == 16 || R == 32, "rank");
  static constexpr int H = L / 2 > 0 ? L / 2 : 1;    // loads per chunk
  static constexpr int PW = kWave * 16 / R;          // positions per wave load
  __amdgpu_buffer_rsrc_t rs;
  int nch, ca, cb;                                   // chunks; the two claimed (ca older)
  bool issued;
  uint4 ga[H], gb[H];

  // positions covered by the chunks the S waves start on
  static constexpr int first_span(int S) { return 2 * S * H * PW; }

  __device__ __forceinline__ void init(__amdgpu_buffer_rsrc_t r, int nv, int w, int S) {
    rs = r;
    nch = (nv + H * PW - 1) / (H * PW);
    ca = w;
    cb = w + S;
    issued = false;
  }
  __device__ __forceinline__ void load(uint4 (&g)[H], int c) {
#pragma unroll
    for (int x = 0; x < H; ++x)
      g[x] = stream_load16(rs, (uint32_t)((c * H + x) * kWave * 16 + lane_id() * 16));
  }
  // the starting chunks' loads (may be issued early, before the query and the
  // bound are known)
  __device__ __forceinline__ void issue_first() {
    if (ca < nch) load(ga, ca);
    if (cb < nch) load(gb, cb);
    issued = true;
  }
  template <class Keep>
  __device__ __forceinline__ void run(const float* qt, uint32_t* next, Keep keep) {
    const int lane = lane_id();
    const int lane_pos = lane * 16 / R;
    const bool owner = R == 16 || (lane & 1) == 0;
    float ql[16];
    const int qoff = R == 32 ? 16 * (lane & 1) : 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) ql[k] = qt[qoff + k];
    auto score = [&](const uint4 (&g)[H], int c) {
#pragma unroll
      for (int x = 0; x < H; ++x) {
        float s = score16(ql, g[x]);
        if (R == 32) s = s + dpp_f<kDppQuadSwap1>(s);
        keep(s, (c * H + x) * PW + lane_pos, owner);
      }
    };
    auto claim = [&]() {
      uint32_t c = 0u;
      if (lane == 0) c = atomicAdd(next, 1u);
      return (int)__builtin_amdgcn_readlane(c, 0);
    };
    if (!issued) issue_first();
    // Claims only grow, so when the older claim is past the end the younger
    // one is too, and no load is left in flight at the exit.
    for (;;) {                                        // wave-uniform trip count
      if (ca >= nch) break;
      score(ga, ca);
      ca = claim();
      if (ca < nch) load(ga, ca);
      if (cb >= nch) break;
      score(gb, cb);
      cb = claim();
      if (cb < nch) load(gb, cb);
    }
  }
};

template <int D, int R>
__global__ __launch_bounds__(kChunkThreads) void filter_kernel(const FilterArgs a) {
  constexpr int NT = kChunkThreads;
  // Each wave lists the positions it keeps in LDS; at the end the 8 lists go
  // out back to back as the chunk's candidates, (key, position) pairs in no
  // particular order (the merge emits through a bitmap of positions).
  __shared__ uint32_t sk[kFilterWaves][kFilterMaxCap];
  __shared__ int32_t sp[kFilterWaves][kFilterMaxCap];
  __shared__ uint32_t wn[kFilterWaves];
  const int u = blockIdx.x / a.S, c = blockIdx.x % a.S;
  const int b = u / a.Hkv;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int len = unit_len(a.seq_lens, b, a.n_max);
  const int base = c * a.chunk;
  const int nv = min(max(len - base, 0), a.chunk);
  const int pend = base + nv;                         // this chunk's valid positions end here
  int32_t* cnt = a.cnt + (size_t)u * (a.S + 1) + c;
  uint32_t* spill_cnt = reinterpret_cast<uint32_t*>(a.cnt + (size_t)u * (a.S + 1) + a.S);
  if (len <= a.M || nv == 0) {                        // block-uniform
    if (threadIdx.x == 0) *cnt = 0;
    return;
  }
  // key >= thr  <=>  score >= thrf for every score that is not NaN (the
  // chains produce none; -0 and +0 share the key of +0, and -0 >= +0 holds)
  const float thrf = key_score(a.thr[u]);
  uint2* lc = a.cand + (size_t)u * a.ustride + (size_t)c * a.cslots;
  uint32_t wc = 0;                                    // positions in this wave's list
  // A full list goes to the unit's spill pool (clustered high scores): one
  // lane reserves its slots with an atomic, the wave copies it out, and the
  // list starts again.  A pool too small for it is left counting past its
  // capacity, which sends the merge to the exact fallback.
  uint2* spill_u = a.cand + (size_t)u * a.ustride + (size_t)a.S * a.cslots;
  auto spill_list = [&]() {
    uint32_t at = 0u;
    if (lane == 0) at = atomicAdd(spill_cnt, wc);
    at = (uint32_t)__shfl((int)at, 0, kWave);
    if (at + wc <= (uint32_t)a.spill_cap) {
      for (int j = lane; j < (int)wc; j += kWave)
        spill_u[at + j] =
            make_uint2(score_key(__uint_as_float(sk[w][j]) + 0.0f), (uint32_t)sp[w][j]);
    }
    wc = 0;
  };
  // One position per lane (the call is wave-uniform): keep it if it is in the
  // chunk and its score reaches the bound.
  auto keep = [&](float s, int p, bool owner) {
    const bool ge = s >= thrf, in = owner && p < pend;
    const bool sel = ge && in;
    const uint64_t m = ballot(ge) & ballot(in);       // (two compares, no select)
    const uint32_t n = (uint32_t)popc64(m);
    if (wc + n > (uint32_t)a.cap) spill_list();       // wave-uniform, rare
    const uint32_t slot = wc + __builtin_amdgcn_mbcnt_hi(
                                   (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (sel && slot < (uint32_t)a.cap) {
      sk[w][slot] = __float_as_uint(s);               // keyed when written out
      sp[w][slot] = p;
    }
    wc += n;
  };
  // Loads cover this chunk's rows only: past its valid positions they return
  // zero, and those positions (at or past pend) are never kept.  Two
  // register sets: while one batch is scored the next one is in flight
  // (software pipelining keeps the memory queue full).  Every trip count is
  // block-uniform.
  if constexpr (R == kScoreInput) {
    // Lane l of wave w holds positions base + 4(i NT + 64w + l) + e, e < 4:
    // one 16-byte load of four scores.
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.scores + (size_t)u * a.n_max + base, (uint32_t)nv * 4u);
    const uint32_t voff = (uint32_t)((w * kWave + lane) * 16);
    constexpr int kBatch = SA_FILTER_LOADS_IN_FLIGHT;
    struct Batch {
      uint4 v[kBatch];
    };
    auto load_batch = [&](Batch& bt, int i0) {
#pragma unroll
      for (int x = 0; x < kBatch; ++x) bt.v[x] = stream_load16(rs, voff + (uint32_t)((i0 + x) * NT * 16));
    };
    auto score_batch = [&](const Batch& bt, int i0) {
#pragma unroll
      for (int x = 0; x < kBatch; ++x) {
        const int p = base + 4 * ((i0 + x) * NT + w * kWave + lane);
        keep(__uint_as_float(bt.v[x].x), p, true);
        keep(__uint_as_float(bt.v[x].y), p + 1, true);
        keep(__uint_as_float(bt.v[x].z), p + 2, true);
        keep(__uint_as_float(bt.v[x].w), p + 3, true);
      }
    };
    const int rows = (nv + 4 * NT - 1) / (4 * NT);
    Batch b0, b1;
    load_batch(b0, 0);
    if (kBatch < rows) load_batch(b1, kBatch);
    for (int i0 = 0; i0 < rows; i0 += 2 * kBatch) {
      score_batch(b0, i0);
      if (i0 + 2 * kBatch < rows) load_batch(b0, i0 + 2 * kBatch);
      if (i0 + kBatch < rows) {
        score_batch(b1, i0 + kBatch);
        if (i0 + 3 * kBatch < rows) load_batch(b1, i0 + 3 * kBatch);
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.kp + ((size_t)u * a.Ncap + base) * R, (uint32_t)nv * R);
    stream_code_scores<R, NT, SA_FILTER_LOADS_IN_FLIGHT>(
        rs, nv, a.qt + (size_t)u * 32,
        [&](float sc, int p, bool owner) { keep(sc, base + p, owner); });
  }
  // The lists go out only once every wave has finished reading: stores mixed
  // into the read stream cost far more (measured), and one 8-byte store per
  // candidate costs less than two 4-byte ones.  (Full lists went to the
  // spill pool, so no list holds more than cap; a count past cap would mark
  // the chunk -1 and send the merge to the exact fallback.)
  if (lane == 0) wn[w] = wc;
  __syncthreads();
  uint32_t off = 0, total = 0;
  bool over = false;
#pragma unroll
  for (int ww = 0; ww < kFilterWaves; ++ww) {
    const uint32_t x = wn[ww];
    over |= x > (uint32_t)a.cap;
    off += ww < w ? x : 0u;
    total += x;
  }
  if (!over) {
    for (int j = lane; j < (int)wc; j += kWave)
      lc[off + j] = make_uint2(score_key(__uint_as_float(sk[w][j]) + 0.0f), (uint32_t)sp[w][j]);
  }
  if (threadIdx.x == 0) *cnt = over ? -1 : (int)total;
}

// Mark the selected positions of a unit in `bm` (bit p = position p) and
// write them to idx in ascending order (idx_u may be null when M <= the list
// capacity: the -1-padded selection is then left in sh.list).  visit(f) calls f(key, pos, valid)
// for every key of the unit that may be selected (every key >= t at least).
// Selection: every key > t and, of the keys == t, the `need` lowest positions
// (found as the top `need` of the keys ~pos).  Fills idx[0, M) completely.
template <int NT, class Visit>
__device__ __forceinline__ void emit_bitmap(SelectShared<NT>& sh, uint32_t* bm, int len, uint32_t t,
                            uint32_t need, uint32_t eq, int M, int32_t* idx_u, Visit visit) {
  const int tid = threadIdx.x, lane = lane_id();
  const int words = (len + 31) >> 5;
  for (int j = tid; j < words; j += NT) bm[j] = 0u;
  __syncthreads();
  const bool single = need == eq;
  visit([&](uint32_t k, int p, bool valid) {
    if (valid && (k > t || (single && k == t))) atomicOr(&bm[p >> 5], 1u << (p & 31));
  });
  if (!single) {
    // ties straddle the cut: rank the tied positions, lowest first
    for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
    __syncthreads();
    const uint32_t dummy = (uint32_t)(kBins + lane);
    visit([&](uint32_t k, int p, bool valid) {
      const bool e = valid && k == t;
      hist_add(sh.hist, e ? (~(uint32_t)p >> kTopShift) : dummy);
    });
    __syncthreads();
    uint32_t tp, np, ep;
    finish_threshold<NT>(sh, need, tp, np, ep, [&](auto&& f) {
      visit([&](uint32_t k, int p, bool valid) { f(~(uint32_t)p, valid && k == t); });
    });
    const int last = (int)~tp;                        // highest tied position selected
    visit([&](uint32_t k, int p, bool valid) {
      if (valid && k == t && p <= last) atomicOr(&bm[p >> 5], 1u << (p & 31));
    });
  }
  __syncthreads();
  // ascending positions: thread j owns a contiguous run of words
  const int wpt = (words + NT - 1) / NT;
  const int w0 = min(tid * wpt, words), w1 = min(w0 + wpt, words);
  uint32_t mine = 0;
  for (int j = w0; j < w1; ++j) mine += (uint32_t)__builtin_popcount(bm[j]);
  uint32_t total;
  uint32_t off = block_inclusive_scan<NT>(mine, sh, total) - mine;
  int32_t* out = reinterpret_cast<int32_t*>(sh.list);   // free now; holds >= kFilterMaxM
  const bool staged = M <= kListCap;
  for (int j = w0; j < w1; ++j) {
    uint32_t x = bm[j];
    while (x) {
      const int bit = __builtin_ctz(x);
      x &= x - 1u;
      const int32_t pos = j * 32 + bit;
      if (off < (uint32_t)M) {
        if (staged) out[off] = pos;
        else idx_u[off] = pos;
      }
      ++off;
    }
  }
  __syncthreads();
  if (staged) {
    for (int j = tid; j < M; j += NT) {
      const int32_t v = j < (int)total ? out[j] : -1;
      if (j >= (int)total) out[j] = -1;
      if (idx_u) idx_u[j] = v;
    }
  } else {
    for (int j = (int)total + tid; j < M; j += NT) idx_u[j] = -1;
  }
}

// Emit, in ascending order, the selected positions of a unit whose
// candidates sit in registers in no particular order (key[i], pos[i] for
// i < nk; key 0 = none): every key > t and, of the keys == t, the `need`
// lowest positions.  The selection is marked in an LDS bitmap of positions;
// a selected position's output slot is the number of marked positions below
// it (one block scan over per-thread groups of words gives a count before
// each word, then a bit count inside the word).  Leaves the M positions, -1 padded, in sh.list (as int32) and
// copies them to idx_u when it is not null.
template <int NT, int K>
__device__ __forceinline__ void emit_selected(SelectShared<NT>& sh, uint32_t* bm, int len,
                                              uint32_t t, uint32_t need, uint32_t eq, int M,
                                              int nk, const uint32_t (&key)[K],
                                              const int32_t (&pos)[K], int32_t* idx_u) {
  const int tid = threadIdx.x, lane = lane_id();
  const int words = (len + 31) >> 5;
  const int wpt = (words + NT - 1) / NT;              // words per thread group
  for (int j = tid; j < words; j += NT) bm[j] = 0u;
  int last = 0x7FFFFFFF;                              // highest tied position taken
  if (need != eq) {                                   // block-uniform: ties straddle the cut
    // the need lowest tied positions = the need largest of ~position
    for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
    __syncthreads();
    const uint32_t dummy = (uint32_t)(kBins + lane);
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (i < nk) atomicAdd(&sh.hist[key[i] == t ? (~(uint32_t)pos[i] >> kTopShift) : dummy], 1u);
    __syncthreads();
    uint32_t tp, np, ep;
    finish_threshold<NT>(sh, need, tp, np, ep, [&](auto&& f) {
#pragma unroll
      for (int i = 0; i < K; ++i)
        if (i < nk) f(~(uint32_t)pos[i], key[i] == t);
    });
    last = (int)~tp;
  }
  __syncthreads();                                    // bm is clear
  auto taken = [&](int i) { return key[i] > t || (key[i] == t && pos[i] <= last); };
#pragma unroll
  for (int i = 0; i < K; ++i)
    if (i < nk && taken(i)) atomicOr(&bm[pos[i] >> 5], 1u << (pos[i] & 31));
  __syncthreads();
  const int w0 = min(tid * wpt, words), w1 = min(w0 + wpt, words);
  uint32_t mine = 0;
  for (int j = w0; j < w1; ++j) mine += (uint32_t)__builtin_popcount(bm[j]);
  uint32_t total;
  const uint32_t incl = block_inclusive_scan<NT>(mine, sh, total);
  // marked positions before each word: a table in the (free) histogram when
  // the bitmap is short enough, else per thread group
  const bool table = words <= kBins + kWave;          // block-uniform
  if (table) {
    uint32_t run = incl - mine;
    for (int j = w0; j < w1; ++j) {
      sh.hist[j] = run;
      run += (uint32_t)__builtin_popcount(bm[j]);
    }
  } else {
    sh.seg[tid] = incl - mine;
  }
  __syncthreads();
  int32_t* out = reinterpret_cast<int32_t*>(sh.list);
#pragma unroll
  for (int i = 0; i < K; ++i) {
    if (i < nk && taken(i)) {
      const int p = pos[i], wj = p >> 5;
      uint32_t slot;
      if (table) {
        slot = sh.hist[wj];
      } else {
        const int grp = wj / wpt;
        slot = sh.seg[grp];
        for (int j = grp * wpt; j < wj; ++j) slot += (uint32_t)__builtin_popcount(bm[j]);
      }
      slot += (uint32_t)__builtin_popcount(bm[wj] & ((1u << (p & 31)) - 1u));
      if (slot < (uint32_t)M) out[slot] = p;
    }
  }
  for (int j = (int)total + tid; j < M; j += NT) out[j] = -1;
  __syncthreads();
  if (idx_u)
    for (int j = tid; j < M; j += NT) idx_u[j] = out[j];
}

// Exact selection of one unit by streaming its rows (or scores) again: the
// filter's bound was above the M-th key, or the unit kept more keys than the
// merge holds.
template <int D, int R>
__device__ __forceinline__ void select_unit_streaming(const FilterArgs& a, SelectShared<kMergeThreads>& sh,
                                                   uint32_t* bm, int u, int b, int h, int len,
                                                   int32_t* idx_u) {
  constexpr int NT = kMergeThreads;
  const int tid = threadIdx.x;
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  if (R != kScoreInput && tid < R) sh.qt[tid] = a.qt[(size_t)u * 32 + tid];
  __syncthreads();
  float qlo[16], qhi[16];
  if constexpr (R != kScoreInput) query_halves<R>(sh.qt, qlo, qhi);
  // Every pass visits the thread's positions p0 + tid in order, the loads of
  // kAhead of them going out before any is scored (the chains and their
  // order are position_score's).
  constexpr int kAhead = 2;
  auto visit3 = [&](auto&& f) {
    for (int p0 = 0; p0 < len; p0 += NT * kAhead) {   // block-uniform
      uint4 ca[kAhead], cb[kAhead];
      float sv[kAhead];
#pragma unroll
      for (int k = 0; k < kAhead; ++k) {
        const int p = p0 + k * NT + tid;
        const int pc = p < len ? p : 0;
        if constexpr (R == kScoreInput) {
          sv[k] = a.scores[(size_t)u * a.n_max + pc];
        } else {
          const uint8_t* row = a.kp + ((size_t)u * a.Ncap + pc) * R;
          ca[k] = load16(row);
          if (R == 32) cb[k] = load16(row + 16);
        }
      }
#pragma unroll
      for (int k = 0; k < kAhead; ++k) {
        const int p = p0 + k * NT + tid;
        const bool ok = p < len;
        float s;
        if constexpr (R == kScoreInput) {
          s = sv[k];
        } else {
          s = score16(qlo, ca[k]);
          if (R == 32) s = s + score16(qhi, cb[k]);
        }
        f(ok ? score_key(s + 0.0f) : 0u, p, ok);
      }
    }
  };
  const uint32_t dummy = (uint32_t)(kBins + lane_id());
  visit3([&](uint32_t k, int, bool ok) { hist_add(sh.hist, ok ? (k >> kTopShift) : dummy); });
  __syncthreads();
  uint32_t t, need, eq;
  finish_threshold<NT>(sh, (uint32_t)a.M, t, need, eq, [&](auto&& f) {
    visit3([&](uint32_t k, int, bool ok) { f(k, ok); });
  });
  emit_bitmap<NT>(sh, bm, len, t, need, eq, a.M, idx_u, visit3);
}

// LDS of the merge workgroup.
struct MergeShared {
  SelectShared<kMergeThreads> sh;
  uint32_t bm[kBitmapWords];        // used by the streaming fallback only
  uint32_t start_s[kMergeStarts];
  uint32_t red[kMergeThreads / kWave];
};

// The merge of unit u by the whole workgroup (it synchronises).  Leaves the
// unit's M selected positions, ascending and -1 padded, in sh.list (as int32)
// and, when write_idx, also in idx (and the unit's path flag).
// gather(key, pos, nk, total) puts the unit's kept candidates (key, position)
// into the threads' registers in any order (key 0 = empty slot; rows >= nk,
// block-uniform, are all empty) and sets total to their number, or to 0 when
// a list overflowed or they do not fit the registers (the unit then takes the
// exact fallback); it synchronises.  bm: the bitmap of kBitmapWords words
// (also the fallback's); red: kMergeThreads / kWave words.
template <int D, int R, class Gather>
__device__ __forceinline__ void merge_unit_core(const FilterArgs& a, SelectShared<kMergeThreads>& sh,
                                                uint32_t* bm, uint32_t* red, int u,
                                                bool write_idx, Gather gather) {
  constexpr int NT = kMergeThreads;
  constexpr int KPT = kFilterMergeKeys;
  static_assert(kFilterMaxM <= kListCap - kWave, "the selection is staged in LDS");
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int len = unit_len(a.seq_lens, b, a.n_max);
  const int M = a.M;
  int32_t* idx_u = write_idx ? a.idx + (size_t)u * M : nullptr;
  int32_t* out = reinterpret_cast<int32_t*>(sh.list);
  if (len <= M) {                                     // every valid position, in order
    for (int j = tid; j < M; j += NT) {
      out[j] = j < len ? j : -1;
      if (idx_u) idx_u[j] = out[j];
    }
    if (write_idx && tid == 0) a.path[u] = 0;
    __syncthreads();
    return;
  }
  uint32_t key[KPT];
  int32_t pos[KPT];
  int nk;
  uint32_t total;
  gather(key, pos, nk, total);
  if (write_idx && tid == 0) a.path[u] = total < (uint32_t)M ? 1 : 0;
  if (total < (uint32_t)M) {                          // block-uniform (0 after an overflow)
    select_unit_streaming<D, R>(a, sh, bm, u, b, h, len, idx_u);
    __syncthreads();
    return;
  }
  const uint32_t thr = a.thr[u];
  uint32_t kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) kmax = max(kmax, key[i]);
  // Every candidate is >= thr >= 1.  Spread the candidates' range over the
  // first radix digit: k' = ((key - thr) << lsh) + 1 (order-preserving, 0 is
  // left for "no key", bit 31 of k' - 1 stays clear so k' cannot overflow).
  kmax = wave_max_u32(kmax);
  if (lane == 0) red[w] = kmax;
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  __syncthreads();                                    // (sources are no longer read)
  kmax = 0u;
#pragma unroll
  for (int ww = 0; ww < NT / kWave; ++ww) kmax = max(kmax, red[ww]);
  const uint32_t span = kmax - thr;
  const int lsh = span ? max(__clz((int)span) - 1, 0) : 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = key[i] ? ((key[i] - thr) << lsh) + 1u : 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (i < nk && key[i] != 0u) atomicAdd(&sh.hist[key[i] >> kTopShift], 1u);
  __syncthreads();
  uint32_t t, need, eq;
  finish_threshold<NT>(sh, (uint32_t)M, t, need, eq, [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (i < nk) f(key[i], key[i] != 0u);
  });
  // the candidates are in no particular order: emit through a bitmap of the
  // unit's positions
  emit_selected<NT>(sh, bm, len, t, need, eq, M, nk, key, pos, idx_u);
}

// The merge over the filter kernel's chunk lists and the unit's spill pool
// (in the workspace): the unit's candidates are numbered g = 0 .. total-1
// chunk after chunk, the pool last (one wave forms the exclusive prefix of
// the counts), and candidate g sits in register g / NT of thread g % NT,
// found by bisection of the prefix.  A chunk whose lists overflowed (-1), a
// pool that ran out, or more candidates than the registers hold give total 0.
template <int D, int R>
__device__ __forceinline__ void filter_merge_unit(const FilterArgs& a, MergeShared& ms, int u,
                                                  bool write_idx) {
  constexpr int NT = kMergeThreads;
  constexpr int KPT = kFilterMergeKeys;
  const int S = a.S;
  const uint2* cu = a.cand + (size_t)u * a.ustride;
  uint32_t* start_s = ms.start_s;
  uint32_t* red = ms.red;
  merge_unit_core<D, R>(
      a, ms.sh, ms.bm, red, u, write_idx,
      [&](uint32_t (&key)[KPT], int32_t (&pos)[KPT], int& nk, uint32_t& total) {
        const int tid = threadIdx.x, lane = lane_id();
        if (tid < kWave) {
          const int c = lane <= S ? a.cnt[(size_t)u * (S + 1) + lane] : 0;
          const bool over = ballot(c < 0 || (lane == S && c > a.spill_cap)) != 0;
          const uint32_t v = (uint32_t)max(c, 0);
          const uint32_t incl = wave_inclusive_scan(v);
          if (lane < kMergeStarts) start_s[lane] = lane <= S ? incl - v : 0xFFFFFFFFu;
          if (lane == kWave - 1) red[0] = (over || incl > (uint32_t)(NT * KPT)) ? 0u : incl;
        }
        __syncthreads();
        total = red[0];
        nk = (int)((total + NT - 1) / NT);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          key[i] = 0u;
          pos[i] = 0;
          const uint32_t g = (uint32_t)(i * NT + tid);
          if (i < nk && g < total) {
            uint32_t c = 0;                           // last chunk with start_c <= g
#pragma unroll
            for (int step = kMergeStarts / 2; step >= 1; step >>= 1)
              if (start_s[c + step] <= g) c += step;
            const uint2 kv = cu[(size_t)c * a.cslots + (g - start_s[c])];
            key[i] = kv.x;
            pos[i] = (int32_t)kv.y;
          }
        }
        __syncthreads();                              // red is reused
      });
}

template <int D, int R>
__global__ __launch_bounds__(kMergeThreads) void filter_merge_kernel(const FilterArgs a) {
  __shared__ MergeShared ms;
  filter_merge_unit<D, R>(a, ms, blockIdx.x, true);
}

// The merge followed, in the same workgroup, by the attention of split
// `split` of the unit over the selection it just left in LDS (no reload of
// idx, no second launch; every split's workgroup merges, split 0 writes idx).
// The waves' output tiles reuse the fallback's bitmap: 16 G d floats fit its
// 64 KB when G d <= 1024.
template <int D, int R>
__global__ __launch_bounds__(kMergeThreads) void select_attend_kernel(const FilterArgs a,
                                                                      const DecodeArgs d) {
  static_assert(kAttendThreads == kMergeThreads, "one workgroup shape for both");
  __shared__ MergeShared ms;
  __shared__ float sm[kAttendWaves][kMaxHeads], sl[kAttendWaves][kMaxHeads];
  const int u = blockIdx.x / d.S, split = blockIdx.x % d.S;
  filter_merge_unit<D, R>(a, ms, u, split == 0);
  AttendWave<D, kAttendWaves> aw;
  aw.init(d, u);
  const int r0 = split * d.rps;
  const int r1 = min(d.M, r0 + d.rps);
  aw.rows(d, reinterpret_cast<const int32_t*>(ms.sh.list) + r0, r1 - r0);
  aw.finish(d, u, split, sm, sl, reinterpret_cast<float*>(ms.bm));
}


// ------------------------------------------------------------------ every position scored
//
// Short units, few of them (at most kScoresMaxN positions, too few units for
// one workgroup each): a first launch scores every position -- each
// workgroup one chunk of a unit -- and the merge selects exactly over all of
// a unit's scores, 16 per thread in registers.  No bound, no filter, no
// fallback; the candidates the filter plan would keep are a third of such a
// unit anyway.  Each scoring workgroup forms the unit's indexer query (the
// bits every kernel forms) and appends the unit's new rows that fall in its
// chunk (the last chunk also those past it); a chunk with no new row has all
// of its code loads in flight before the query is formed.  The scores are
// CodeStream's chains (the filter's bits).
//
// Layout: position p = 1024 r + t (t < 1024, r < 16) goes to float
// 4096 (r / 4) + 4 t + r % 4 of the unit's array, so that merge thread t
// loads its 16 scores (key register r = position 1024 r + t) as four 16-byte
// loads.  Both launches keep a unit's workgroups on one XCD (workgroups are
// handed to the 8 XCDs in turn), so the merges of its splits find its scores
// in one L2.
constexpr int kScoreAllThreads = kSampleThreads;   // the prologue's thread roles need 1024
constexpr int kScoreAllLoads = 4;                  // 4 x 16 KB: a 2048-position chunk at once
constexpr int kXcds = 8;

__device__ __forceinline__ int scores_slot(int p) {
  static_assert(kMergeThreads == 1024, "the layout follows the merge's 1024 threads");
  const int r = p >> 10, t = p & 1023;
  return ((r >> 2) << 12) | (t << 2) | (r & 3);
}

// Workgroup g of a units x per grid -> (unit, part) with a unit's parts on
// one XCD when units divide evenly among them, else unit-major.
__device__ __forceinline__ void xcd_unit_part(int g, int units, int per, int& u, int& part) {
  if (units % kXcds == 0) {
    const int x = g % kXcds, j = g / kXcds;
    part = j % per;
    u = x + kXcds * (j / per);
  } else {
    u = g / per;
    part = g % per;
  }
}

template <int D, int R>
__global__ __launch_bounds__(kScoreAllThreads) void score_all_kernel(const FilterArgs a,
                                                                     const AppendArgs ap) {
  constexpr int NT = kScoreAllThreads;
  __shared__ float qt[32];
  __shared__ double part[NT];
  int u, c;
  xcd_unit_part(blockIdx.x, a.units, a.S, u, c);
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int len = unit_len(a.seq_lens, b, a.n_max);
  const int base = c * a.chunk;
  const int nv = min(max(len - base, 0), a.chunk);
  // the new rows this workgroup appends: those in [base, base + chunk), and
  // for the last chunk every row past it too
  int t0 = 0, t1 = 0;
  if (ap.T > 0) {
    const long p0 = ap.pos[b];
    t0 = (int)min(max((long)base - p0, 0L), (long)ap.T);
    t1 = c == a.S - 1 ? ap.T : (int)min(max((long)base + a.chunk - p0, 0L), (long)ap.T);
  }
  const bool fresh = t1 > t0;                         // block-uniform
  CodeStream<R, NT, kScoreAllLoads> cs;
  cs.init(make_rsrc(a.kp + ((size_t)u * a.Ncap + base) * R, (uint32_t)nv * R), nv);
  if (!fresh && nv > 0) cs.issue_first();
  if (fresh)
    append_rows_and_query<D, R, NT>(a, ap, u, qt, part, t0, t1);
  else
    indexer_query<D, R, NT>(a.q, a.P, b, h, a.G, a.Hq, qt, part);
  // a chunk with new rows reads its codes only once their stores completed
  if (fresh) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (c == 0 && threadIdx.x < R) a.qt[(size_t)u * 32 + threadIdx.x] = qt[threadIdx.x];
  float* su = a.sc + (size_t)u * a.sstride;
  if (nv > 0)
    cs.run(qt, [&](float sc, int p, bool owner) {
      if (owner && p < nv) su[scores_slot(base + p)] = sc;
    });
}

// Exact threshold over keys whose scores all lie in [key_score(klo),
// key_score(khi)] (finite, the first below the second; key 0: none): the
// first level bins the scores by value, 4096 equal-width bins (monotone in
// the key, so every key of a higher bin is larger, and equal keys share a
// bin), which leaves few keys in the bin of the target-th largest where the
// scores crowd; that bin's keys are then ranked directly (or, when it is
// large, selected by radix levels over their keys).  Each key's bin is formed
// once.  Returns t, need and eq as finish_threshold does.
template <int NT, int K>
__device__ __forceinline__ void threshold_by_value(SelectShared<NT>& sh, const uint32_t (&key)[K],
                                                   uint32_t klo, uint32_t khi, uint32_t target,
                                                   uint32_t& t_out, uint32_t& need_out,
                                                   uint32_t& eq_out) {
  const int tid = threadIdx.x;
  const float smin = key_score(klo), smax = key_score(khi);
  const float scale = (float)kBins / (smax - smin);
  // a key's bin, or a lane's private dummy bin (>= kBins) for no key
  const uint32_t dummy = (uint32_t)(kBins + lane_id());
  uint32_t bn[K];
#pragma unroll
  for (int i = 0; i < K; ++i) {
    const float x = (key_score(key[i]) - smin) * scale;
    bn[i] = key[i] ? min((uint32_t)x, (uint32_t)kBins - 1u) : dummy;
  }
  // (value bins rarely repeat within a wave: one plain atomic per key)
#pragma unroll
  for (int i = 0; i < K; ++i) atomicAdd(&sh.hist[bn[i]], 1u);
  __syncthreads();
  uint32_t path = 0, above = 0;
  pick_bin<NT>(sh, kDigitBits, target, path, above);
  const uint32_t bstar = path, nbin = sh.pick[2];
  const uint32_t rank = target - above;
  if (nbin <= (uint32_t)kRankMax && nbin <= (uint32_t)NT && nbin + 4 <= (uint32_t)SelectShared<NT>::kCap) {
    if (tid == 0) sh.pick[3] = 0u;
    if (tid < 4) sh.list[nbin + tid] = 0u;           // pad for rank_in_list
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (bn[i] == bstar) sh.list[atomicAdd(&sh.pick[3], 1u)] = key[i];
    __syncthreads();
    uint32_t t, gt, eq;
    rank_in_list<NT>(sh, nbin, rank, t, gt, eq);
    t_out = t;
    need_out = rank - gt;
    eq_out = eq;
    return;
  }
  // a crowded bin: the exact search over its keys alone
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < K; ++i) hist_add(sh.hist, bn[i] == bstar ? (key[i] >> kTopShift) : dummy);
  __syncthreads();
  finish_threshold<NT>(sh, rank, t_out, need_out, eq_out, [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < K; ++i) f(key[i], bn[i] == bstar);
  });
}

// The merge of unit u over its scores (the whole workgroup; it synchronises):
// position 1024 i + t sits in key register i of thread t, so register order
// (i, wave, lane) is position order.  The M-th largest key is found exactly
// (threshold_by_value, or finish_threshold over the keys when the scores
// span no finite range) and the selection is emitted in register order
// (emit_in_order: every key above it and, of the keys equal to it, the
// lowest positions).  Leaves the M positions, ascending, in sh.list and, when
// write_idx, in idx (with the unit's path flag 0).  interleaved: the scores
// in score_all_kernel's layout, else in position order (a caller's).  red:
// 2 NT / kWave words.
__device__ __forceinline__ void scores_merge_unit(const FilterArgs& a,
                                                  SelectShared<kMergeThreads>& sh,
                                                  uint32_t* red, int u, bool write_idx,
                                                  bool interleaved) {
  constexpr int NT = kMergeThreads, K = kFilterMergeKeys, W = NT / kWave;
  static_assert(NT * K >= kScoresMaxN && K % 4 == 0, "a unit's scores fit the registers");
  static_assert(kFilterMaxM <= kListCap - kWave, "the selection is staged in LDS");
  const int b = u / a.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int len = unit_len(a.seq_lens, b, a.n_max);
  const int M = a.M;
  int32_t* idx_u = write_idx ? a.idx + (size_t)u * M : nullptr;
  int32_t* out = reinterpret_cast<int32_t*>(sh.list);
  if (write_idx && tid == 0) a.path[u] = 0;
  if (len <= M) {                                     // every valid position, in order
    for (int j = tid; j < M; j += NT) {
      out[j] = j < len ? j : -1;
      if (idx_u) idx_u[j] = out[j];
    }
    __syncthreads();
    return;
  }
  const float* su = a.sc + (size_t)u * a.sstride;
  uint32_t key[K];
  if (interleaved) {                                  // block-uniform
#pragma unroll
    for (int i4 = 0; i4 < K / 4; ++i4) {
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (4 * i4 * NT < len) v = *reinterpret_cast<const float4*>(su + (i4 << 12) + (tid << 2));
      const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = (4 * i4 + e) * NT + tid;
        key[4 * i4 + e] = p < len ? score_key(x[e] + 0.0f) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int p = i * NT + tid;
      key[i] = p < len ? score_key(su[p] + 0.0f) : 0u;
    }
  }
  // the keys' range (key 0: none)
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    kmax = max(kmax, key[i]);
    kmin = min(kmin, key[i] ? key[i] : 0xFFFFFFFFu);
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  if (lane == 0) {
    red[w] = kmax;
    red[W + w] = kmin;
  }
  for (int bb = tid; bb < kBins + kWave; bb += NT) sh.hist[bb] = 0u;
  __syncthreads();
  kmax = 0u;
  kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int ww = 0; ww < W; ++ww) {
    kmax = max(kmax, red[ww]);
    kmin = min(kmin, red[W + ww]);
  }
  uint32_t t, need, eq;
  // by value when every score is finite (keys outside [key(-inf), key(+inf)]
  // are NaN scores) and the range and its bin width are finite
  const uint32_t kneg = score_key(-__builtin_inff()), kpos = score_key(__builtin_inff());
  const float smin = key_score(kmin), smax = key_score(kmax);
  const bool by_value = kmin < kmax && kmin >= kneg && kmax <= kpos &&
                        smin > -__builtin_inff() && smax < __builtin_inff() &&
                        smax - smin < __builtin_inff() &&
                        (float)kBins / (smax - smin) < __builtin_inff();   // block-uniform
  if (by_value) {
    threshold_by_value<NT>(sh, key, kmin, kmax, (uint32_t)M, t, need, eq);
  } else {
    const uint32_t dummy = (uint32_t)(kBins + lane);
#pragma unroll
    for (int i = 0; i < K; ++i) hist_add(sh.hist, key[i] ? (key[i] >> kTopShift) : dummy);
    __syncthreads();
    finish_threshold<NT>(sh, (uint32_t)M, t, need, eq, [&](auto&& f) {
#pragma unroll
      for (int i = 0; i < K; ++i) f(key[i], key[i] != 0u);
    });
  }
  emit_in_order(key, t, need, eq, sh, [&](int i, bool sel, uint32_t slot) {
    out[sel ? slot : (uint32_t)(kListCap - kWave + lane)] = i * NT + tid;
  });
  if (idx_u)
    for (int j = tid; j < M; j += NT) idx_u[j] = out[j];
}

template <bool INTERLEAVED>
__global__ __launch_bounds__(kMergeThreads) void scores_merge_kernel(const FilterArgs a) {
  __shared__ SelectShared<kMergeThreads> sh;
  __shared__ uint32_t red[2 * kMergeThreads / kWave];
  scores_merge_unit(a, sh, red, blockIdx.x, true, INTERLEAVED);
}

// Merge and attention in one launch, as select_attend_kernel: each of the
// unit's d.S workgroups merges (split 0 writes idx) and attends over its
// split of the selection it leaves in LDS.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void scores_select_attend_kernel(const FilterArgs a,
                                                                             const DecodeArgs d) {
  static_assert(kAttendThreads == kMergeThreads, "one workgroup shape for both");
  __shared__ SelectShared<kMergeThreads> sh;
  __shared__ uint32_t red[2 * kMergeThreads / kWave];
  __shared__ float sm[kAttendWaves][kMaxHeads], sl[kAttendWaves][kMaxHeads];
  __shared__ float so[kFusedAttendMaxGD * kAttendWaves];   // the waves' output tiles
  int u, split;
  xcd_unit_part(blockIdx.x, a.units, d.S, u, split);
  scores_merge_unit(a, sh, red, u, split == 0, true);
  AttendWave<D, kAttendWaves> aw;
  aw.init(d, u);
  const int r0 = split * d.rps;
  const int r1 = min(d.M, r0 + d.rps);
  aw.rows(d, reinterpret_cast<const int32_t*>(sh.list) + r0, r1 - r0);
  aw.finish(d, u, split, sm, sl, so);
}

// ------------------------------------------------------------------ one workgroup per unit
//
// When the units fill the chip, one 1024-thread workgroup per unit runs the
// whole step in one launch: it appends the new rows and forms the query and
// the sampled bound (append_bound_kernel's arithmetic), streams the unit's
// codes (WaveStream: chunks handed to the waves on demand), keeps every score
// >= the bound in the LDS list of the wave that scored it (a full list goes
// to the unit's spill pool, as in the filter kernel), merges exactly over the
// lists and the pool (merge_unit_core: the candidates never travel through
// HBM) and, with ATTEND, attends over the selection it leaves in LDS
// (AttendWave, the attention kernels' arithmetic, one split).

// Loads in flight per lane and the waves that stream (any others wait at the
// merge's first barrier; the lists' LDS is shared out among the streaming
// waves).  Measured at 128K with the chunks handed out on demand: all 16
// waves with 4 loads 209.9-210.2 us per step, 8 with 8 211.2-212.7, 8 with 6
// 210.0-210.7, 16 with 2 212.4-213.7, 8 with 4 239.
#ifndef SA_UNIT_LOADS_IN_FLIGHT
#define SA_UNIT_LOADS_IN_FLIGHT 4
#endif
#ifndef SA_UNIT_STREAM_WAVES
#define SA_UNIT_STREAM_WAVES 16
#endif
constexpr int kUnitStreamWaves = SA_UNIT_STREAM_WAVES;
constexpr int kUnitListCap = kUnitWaves * kUnitCap / kUnitStreamWaves;   // slots per list
static_assert(kUnitStreamWaves >= 1 && kUnitStreamWaves <= kUnitWaves &&
                  kUnitWaves % kUnitStreamWaves == 0, "streaming waves");
// merge registers per thread: a list's share, then the spill pool's
constexpr int kUnitListRows = kUnitCap / kWave;                          // 12
constexpr int kUnitSpillRows = kFilterMergeKeys - kUnitListRows;         // 4
static_assert(kUnitListRows * kWave * kUnitWaves / kUnitStreamWaves >= kUnitListCap,
              "a list fits its waves' registers");

struct UnitShared {
  union {
    struct {
      float s[kUnitStreamWaves][kUnitListCap];     // kept scores (keyed when merged)
      int32_t p[kUnitStreamWaves][kUnitListCap];   // and their positions
    } lists;
    uint32_t bm[kBitmapWords];              // the merge's bitmap; then the output tiles
  } u;
  SelectShared<kMergeThreads> sh;
  uint32_t red[kMergeThreads / kWave];
  uint32_t wn[kUnitWaves];
  uint32_t spill_n;
  uint32_t next;                            // the code stream's next free chunk
  float sm[kAttendWaves][kMaxHeads], sl[kAttendWaves][kMaxHeads];
};
static_assert(kUnitWaves == kMergeThreads / kWave, "one list per wave");

template <int D, int R, bool ATTEND>
__global__ __launch_bounds__(kMergeThreads) void unit_kernel(const FilterArgs a,
                                                             const AppendArgs ap,
                                                             const DecodeArgs d) {
  static_assert(kAttendThreads == kMergeThreads && kSampleThreads == kMergeThreads,
                "one workgroup shape for every phase");
  __shared__ UnitShared us;
  const int u = blockIdx.x;
  const int b = u / a.Hkv;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int len = unit_len(a.seq_lens, b, a.n_max);
  if (tid == 0) {
    us.spill_n = 0u;
    us.next = (uint32_t)(2 * kUnitStreamWaves);     // the chunks after the starting ones
  }
  const bool streams = len > a.M && w < kUnitStreamWaves;       // wave-uniform
  WaveStream<R, SA_UNIT_LOADS_IN_FLIGHT> cs;
  cs.init(make_rsrc(a.kp + (size_t)u * a.Ncap * R, (uint32_t)len * R), len, w, kUnitStreamWaves);
  // The first rounds of the stream may be loaded while the bound is being
  // selected, when they lie wholly below the first new row (so they cannot
  // read a code the append is writing).
  const long first_new = ap.T > 0 ? (long)ap.pos[b] : (long)len;
  const bool early = streams && first_new >= (long)decltype(cs)::first_span(kUnitStreamWaves);
  // The decode step's prologue (the new rows appended, the indexer query
  // formed) and the sampled bound, as append_bound_kernel forms them (the
  // same arithmetic, so the same bits), with the query left in us.sh.qt and
  // the bound returned to every thread.
  const uint32_t thr = sample_bound<D, R>(
      a, us.sh, u,
      [&] {
        if (ap.T > 0)
          append_rows_and_query<D, R, kMergeThreads>(a, ap, u, us.sh.qt, us.sh.part);
        else
          indexer_query<D, R, kMergeThreads>(a.q, a.P, b, u % a.Hkv, a.G, a.Hq, us.sh.qt,
                                              us.sh.part);
      },
      [&] {
        if (early) {
          // the new rows' stores complete first (the bound's loads have all
          // returned by now, so this waits for nothing else)
          __builtin_amdgcn_s_waitcnt(0);
          cs.issue_first();
        }
      });
  // every store of the new rows has completed before any wave streams the
  // codes or, later, reads the rows (done above when the first loads went
  // out early; long since, in practice: the bound's selection ran between)
  if (!cs.issued) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t wc = 0;                                    // positions in this wave's list
  if (streams) {                                      // (else all are taken)
    // key >= thr  <=>  score >= thrf (see filter_kernel)
    const float thrf = key_score(thr);
    uint2* spill_u = a.cand + (size_t)u * a.ustride;
    auto spill_list = [&]() {                         // wave-uniform, rare
      uint32_t at = 0u;
      if (lane == 0) at = atomicAdd(&us.spill_n, wc);
      at = (uint32_t)__shfl((int)at, 0, kWave);
      if (at + wc <= (uint32_t)a.spill_cap) {
        for (int j = lane; j < (int)wc; j += kWave)
          spill_u[at + j] = make_uint2(score_key(us.u.lists.s[w][j] + 0.0f),
                                       (uint32_t)us.u.lists.p[w][j]);
      }
      wc = 0;
    };
    auto keep = [&](float sc, int p, bool owner) {
      const bool ge = sc >= thrf, in = owner && p < len;
      const bool sel = ge && in;
      const uint64_t m = ballot(ge) & ballot(in);
      const uint32_t n = (uint32_t)popc64(m);
      if (wc + n > (uint32_t)kUnitListCap) spill_list();
      const uint32_t slot = wc + __builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (sel && slot < (uint32_t)kUnitListCap) {
        us.u.lists.s[w][slot] = sc;
        us.u.lists.p[w][slot] = p;
      }
      wc += n;
    };
    cs.run(us.sh.qt, &us.next, keep);
  }
  if (lane == 0 && w < kUnitStreamWaves) us.wn[w] = wc;
  __syncthreads();                                    // lists, counts and spill writes done
  // The merge reads each wave list straight into registers: list c is read
  // by waves c WPL .. c WPL + WPL - 1, each lane taking every (64 WPL)-th
  // entry (at most kUnitListRows per thread), and the spill pool fills the
  // remaining rows (at most kUnitSpillRows per thread: a larger pool sends the
  // unit to the exact fallback, as an overflowing list does).
  merge_unit_core<D, R>(
      a, us.sh, us.u.bm, us.red, u, true,
      [&](uint32_t (&key)[kFilterMergeKeys], int32_t (&pos)[kFilterMergeKeys], int& nk,
          uint32_t& total) {
        constexpr int WPL = kUnitWaves / kUnitStreamWaves;   // merge waves per list
        const int c = w / WPL;
        const int j0 = (w % WPL) * kWave + lane;
        const uint32_t nlist = us.wn[c];
        const uint32_t nspill = us.spill_n;
#pragma unroll
        for (int i = 0; i < kUnitListRows; ++i) {
          const int j = j0 + i * WPL * kWave;
          key[i] = 0u;
          pos[i] = 0;
          if (j < (int)nlist) {
            key[i] = score_key(us.u.lists.s[c][j] + 0.0f);
            pos[i] = us.u.lists.p[c][j];
          }
        }
        const bool spill_fits = nspill <= (uint32_t)(kUnitSpillRows * kMergeThreads);
#pragma unroll
        for (int i = kUnitListRows; i < kFilterMergeKeys; ++i) {
          const uint32_t g = (uint32_t)((i - kUnitListRows) * kMergeThreads + tid);
          key[i] = 0u;
          pos[i] = 0;
          if (spill_fits && g < nspill) {
            const uint2 kv = a.cand[(size_t)u * a.ustride + g];
            key[i] = kv.x;
            pos[i] = (int32_t)kv.y;
          }
        }
        nk = nspill > 0 ? kFilterMergeKeys : kUnitListRows;
        uint32_t n = nspill;
#pragma unroll
        for (int cc = 0; cc < kUnitStreamWaves; ++cc) n += us.wn[cc];
        total = spill_fits ? n : 0u;
        __syncthreads();                              // the lists are read (bm aliases them)
      });
  if constexpr (ATTEND) {
    AttendWave<D, kAttendWaves> aw;
    aw.init(d, u);
    aw.rows(d, reinterpret_cast<const int32_t*>(us.sh.list), d.M);
    aw.finish(d, u, 0, us.sm, us.sl, reinterpret_cast<float*>(us.u.bm));
  }
}

// Units of the last filter-path selection that took the exact streaming
// pass (path flag 1); -1 when the shape has no filter path (path == null).
__global__ __launch_bounds__(256) void count_fallbacks_kernel(const int32_t* __restrict__ path,
                                                              int units, int32_t* count) {
  __shared__ uint32_t part[256 / kWave];
  uint32_t n = 0;
  if (path)
    for (int u = threadIdx.x; u < units; u += 256) n += path[u] == 1 ? 1u : 0u;
  n = wave_sum_u32(n);
  if (lane_id() == 0) part[threadIdx.x / kWave] = n;
  __syncthreads();
  if (threadIdx.x == 0)
    *count = path ? (int32_t)(part[0] + part[1] + part[2] + part[3]) : -1;
}

hipError_t run_count_fallbacks(const LaunchCommon& c, const FilterPlan& plan,
                               const void* workspace, int32_t* count) {
  const int32_t* path =
      plan.enabled ? (const int32_t*)((const char*)workspace + plan.off_path) : nullptr;
  hipLaunchKernelGGL(count_fallbacks_kernel, dim3(1), dim3(256), 0, c.stream, path, c.units,
                     count);
  return hipGetLastError();
}

template <int D, int R>
static void launch_filter_dr(const FilterArgs& a, const AppendArgs* ap, const DecodeArgs* da,
                             int stages, int units, bool unit_wg, bool all_scores,
                             hipStream_t st) {
  if (all_scores) {
    // the bound stage scores every position (and appends), the merge stage
    // selects over the scores (and attends); the candidates stage has
    // nothing of its own
    AppendArgs none{};
    none.T = 0;
    if (stages & kSelectBound)
      hipLaunchKernelGGL((score_all_kernel<D, R>), dim3((unsigned)(units * a.S)),
                         dim3(kScoreAllThreads), 0, st, a, ap ? *ap : none);
    if ((stages & kSelectMerge) && da)
      hipLaunchKernelGGL((scores_select_attend_kernel<D>), dim3((unsigned)(units * da->S)),
                         dim3(kMergeThreads), 0, st, a, *da);
    else if (stages & kSelectMerge)
      hipLaunchKernelGGL(scores_merge_kernel<true>, dim3(units), dim3(kMergeThreads), 0, st, a);
    return;
  }
  if (unit_wg) {
    // one launch for the whole selection (and the append and attention when
    // given), made by the candidates stage; the bound and merge stages have
    // nothing of their own
    AppendArgs none{};
    none.T = 0;
    if ((stages & kSelectChunks) && da)
      hipLaunchKernelGGL((unit_kernel<D, R, true>), dim3(units), dim3(kMergeThreads), 0, st, a,
                         ap ? *ap : none, *da);
    else if (stages & kSelectChunks)
      hipLaunchKernelGGL((unit_kernel<D, R, false>), dim3(units), dim3(kMergeThreads), 0, st, a,
                         ap ? *ap : none, DecodeArgs{});
    return;
  }
  if ((stages & kSelectBound) && ap)
    hipLaunchKernelGGL((append_bound_kernel<D, R>), dim3(units), dim3(kSampleThreads), 0, st, a,
                       *ap);
  else if (stages & kSelectBound)
    hipLaunchKernelGGL((sample_kernel<D, R>), dim3(units), dim3(kSampleThreads), 0, st, a);
  if (stages & kSelectChunks)
    hipLaunchKernelGGL((filter_kernel<D, R>), dim3((unsigned)(units * a.S)), dim3(kChunkThreads),
                       0, st, a);
  if ((stages & kSelectMerge) && da)
    hipLaunchKernelGGL((select_attend_kernel<D, R>), dim3((unsigned)(units * da->S)),
                       dim3(kMergeThreads), 0, st, a, *da);
  else if (stages & kSelectMerge)
    hipLaunchKernelGGL((filter_merge_kernel<D, R>), dim3(units), dim3(kMergeThreads), 0, st, a);
}

// The three stages over scores the caller holds (sparse_attn_topm).
static void launch_filter_scores(const FilterArgs& a, int stages, int units, hipStream_t st) {
  constexpr int D = 128, R = kScoreInput;           // D plays no part in selection
  if (stages & kSelectBound)
    hipLaunchKernelGGL((sample_kernel<D, R>), dim3(units), dim3(kSampleThreads), 0, st, a);
  if (stages & kSelectChunks)
    hipLaunchKernelGGL((filter_kernel<D, R>), dim3((unsigned)(units * a.S)), dim3(kChunkThreads),
                       0, st, a);
  if (stages & kSelectMerge)
    hipLaunchKernelGGL((filter_merge_kernel<D, R>), dim3(units), dim3(kMergeThreads), 0, st, a);
}

hipError_t run_filter_select(const LaunchCommon& c, const FilterPlan& plan, int stages,
                             const void* q, const float* P, const uint8_t* kp,
                             const int32_t* seq_lens, int n_max, int M, int32_t* idx,
                             void* workspace, const AppendRows* rows, const AttendFused* att,
                             const float* scores) {
  FilterArgs a;
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
  a.cap = plan.cap;
  a.cslots = plan.cslots;
  a.units = plan.units;

  char* ws = (char*)workspace;
  a.thr = (uint32_t*)(ws + plan.off_thr);
  a.qt = (float*)(ws + plan.off_qt);
  a.path = (int32_t*)(ws + plan.off_path);
  a.cnt = (int32_t*)(ws + plan.off_cnt);
  a.cand = (uint2*)(ws + plan.off_cand);
  a.spill_cap = plan.spill_cap;
  a.ustride = plan.ustride;
  a.sc = plan.all_scores ? (float*)(ws + plan.off_cand) : nullptr;
  a.sstride = plan.sstride;
  a.idx = idx;
  if ((long)plan.units * plan.splits > INT32_MAX) return hipErrorInvalidConfiguration;
  AppendArgs ap;
  if (rows) {
    ap.pos = rows->pos;
    ap.T = rows->T;
    ap.k_new = (const uint16_t*)rows->k_new;
    ap.v_new = (const uint16_t*)rows->v_new;
    ap.k_cache = (uint16_t*)rows->k_cache;
    ap.v_cache = (uint16_t*)rows->v_cache;
  }
  const AppendArgs* app = rows ? &ap : nullptr;
  DecodeArgs da{};
  if (att) {
    const DecodePlan& dp = *att->plan;
    if (c.G < 1 || c.G > kMaxHeads || (long)c.G * c.D > kBitmapWords / kAttendWaves ||
        (long)plan.units * dp.splits > INT32_MAX)
      return hipErrorInvalidConfiguration;
    da.q = (const uint16_t*)q;
    da.k = (const uint16_t*)att->k_cache;
    da.v = (const uint16_t*)att->v_cache;
    da.idx = idx;
    da.M = M;
    da.Ncap = c.Ncap;
    da.Hq = c.Hq;
    da.Hkv = c.Hkv;
    da.G = c.G;
    da.S = dp.splits;
    da.rps = dp.rows_per_split;
    da.qscale = att->scale * 1.4426950408889634f;
    da.out = (uint16_t*)att->out;
    da.lse = att->lse;
    char* pw = (char*)att->partials;
    da.pm = (float*)(pw + dp.off_m);
    da.pl = (float*)(pw + dp.off_l);
    da.po = (float*)(pw + dp.off_o);
  }
  const DecodeArgs* dap = att ? &da : nullptr;
  if (scores) {
    if (rows || att || plan.unit_wg) return hipErrorInvalidValue;
    if (plan.all_scores) {                            // the caller's scores are the merge's
      a.sc = const_cast<float*>(scores);
      a.sstride = n_max;
      if (stages & kSelectMerge)
        hipLaunchKernelGGL(scores_merge_kernel<false>, dim3(plan.units), dim3(kMergeThreads), 0,
                           c.stream, a);
    } else {
      launch_filter_scores(a, stages, plan.units, c.stream);
    }
    return hipGetLastError();
  }
  const bool uw = plan.unit_wg, as = plan.all_scores;
  if (uw && att && da.S != 1) return hipErrorInvalidConfiguration;
  if (c.D == 128 && c.R == 32) launch_filter_dr<128, 32>(a, app, dap, stages, plan.units, uw, as, c.stream);
  else if (c.D == 128 && c.R == 16) launch_filter_dr<128, 16>(a, app, dap, stages, plan.units, uw, as, c.stream);
  else if (c.D == 64 && c.R == 32) launch_filter_dr<64, 32>(a, app, dap, stages, plan.units, uw, as, c.stream);
  else launch_filter_dr<64, 16>(a, app, dap, stages, plan.units, uw, as, c.stream);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && att && !uw && (stages & kSelectMerge)) e = run_combine(c, da);
  return e;
}

template <int D, int R, bool FUSED>
static void launch_chunks_kpt(const SelectArgs& a, int kpt, dim3 grid, hipStream_t st) {
  switch (kpt) {
#define SA_CASE(K)                                                                         \
  case K:                                                                                  \
    hipLaunchKernelGGL((chunk_select_kernel<D, R, K, FUSED>), grid, dim3(kChunkThreads), 0, \
                       st, a);                                                             \
    break;
    SA_CASE(1) SA_CASE(2) SA_CASE(4) SA_CASE(8) SA_CASE(16) SA_CASE(32)
#undef SA_CASE
    default: break;
  }
}

template <bool FUSED>
static void launch_chunks(const LaunchCommon& c, const SelectArgs& a, int kpt, dim3 grid) {
  if (!FUSED) { launch_chunks_kpt<64, 16, false>(a, kpt, grid, c.stream); return; }
  if (c.D == 128 && c.R == 32) launch_chunks_kpt<128, 32, true>(a, kpt, grid, c.stream);
  else if (c.D == 128 && c.R == 16) launch_chunks_kpt<128, 16, true>(a, kpt, grid, c.stream);
  else if (c.D == 64 && c.R == 32) launch_chunks_kpt<64, 32, true>(a, kpt, grid, c.stream);
  else launch_chunks_kpt<64, 16, true>(a, kpt, grid, c.stream);
}

hipError_t run_select(const LaunchCommon& c, const TopmPlan& plan, int stages, bool fused,
                      const void* q, const float* P, const uint8_t* kp, const float* scores,
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
  a.ms = plan.ms;
  char* ws = (char*)workspace;
  a.cand_cnt = (int32_t*)(ws + plan.off_cnt);
  a.cand_key = (uint32_t*)(ws + plan.off_key);
  a.cand_pos = (int32_t*)(ws + plan.off_pos);
  a.idx = idx;
  const long blocks = (long)plan.units * plan.splits;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (stages & kSelectChunks) {
    if (fused) launch_chunks<true>(c, a, plan.kpt, dim3((unsigned)blocks));
    else launch_chunks<false>(c, a, plan.kpt, dim3((unsigned)blocks));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kSelectMerge) {
    // the kernel boundary orders the candidate writes before the merge's reads
    const dim3 grid(plan.units), block(kMergeThreads);
    switch (plan.merge_kpt) {
      case 4: hipLaunchKernelGGL(merge_regs_kernel<4>, grid, block, 0, c.stream, a); break;
      case 8: hipLaunchKernelGGL(merge_regs_kernel<8>, grid, block, 0, c.stream, a); break;
      case 12: hipLaunchKernelGGL(merge_regs_kernel<12>, grid, block, 0, c.stream, a); break;
      case 16: hipLaunchKernelGGL(merge_regs_kernel<16>, grid, block, 0, c.stream, a); break;
      case 20: hipLaunchKernelGGL(merge_regs_kernel<20>, grid, block, 0, c.stream, a); break;
      case 24: hipLaunchKernelGGL(merge_regs_kernel<24>, grid, block, 0, c.stream, a); break;
      default: hipLaunchKernelGGL(merge_kernel, grid, block, 0, c.stream, a); break;
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace sa
