// Host-side argument checks, launch planning and status strings (plain C++).
#include "host_plan.h"

#include <algorithm>

namespace sa {

int check_shape(const sa_shape* s) {
  if (!s) return SA_ERR_INVALID;
  if (s->batch < 1 || s->num_kv_heads < 1 || s->num_q_heads < 1 || s->capacity < 1)
    return SA_ERR_INVALID;
  if (s->num_q_heads % s->num_kv_heads != 0) return SA_ERR_INVALID;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G > 16) return SA_ERR_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (s->rank != 16 && s->rank != 32) return SA_ERR_UNSUPPORTED;
  // every per-unit row index and in-unit byte offset must fit in int32
  if ((int64_t)s->capacity * s->head_dim * 2 > INT32_MAX) return SA_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->num_kv_heads > (1 << 24)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

bool ptr_ok(const void* p, size_t align) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) % align) == 0;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int plan_topm(const sa_shape& s, int n_max, int M, TopmPlan* p) {
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  int chunk = kMaxChunk;
  // shrink chunks until the grid fills the chip, but never below one block
  // nor into more than kMaxSplits chunks per unit
  while (chunk > kMinChunk && units * ceil_div(n_max, chunk) < kTargetBlocks &&
         ceil_div(n_max, chunk / 2) <= kMaxSplits)
    chunk >>= 1;
  const int64_t splits = ceil_div(n_max, chunk);
  if (splits > kMaxSplits) return SA_ERR_UNSUPPORTED;
  p->units = (int)units;
  p->chunk = chunk;
  p->kpt = chunk / kChunkBlock;
  p->splits = (int)splits;
  p->mc = std::min(M, chunk);
  // Slots beyond mc let a chunk hand over a superset (every key of the radix
  // bin holding its M-th largest key, and all higher ones) instead of its
  // exact top-M; multiples of the merge width map slots to whole merge rows.
  p->ms = (int)align_up((size_t)std::min(chunk, p->mc + kSupersetSlack), kMergeThreadsHost);
  const int64_t rows = splits * (p->ms / kMergeThreadsHost);
  p->merge_kpt = rows <= kMaxMergeKeysPerThread ? (int)align_up((size_t)rows, 4) : 0;
  if (p->merge_kpt > kMaxMergeKeysPerThread) p->merge_kpt = 0;
  size_t off = 0;
  p->off_cnt = off;
  off = align_up(off + (size_t)units * splits * sizeof(int32_t), kAlign);
  p->off_key = off;
  off = align_up(off + (size_t)units * splits * p->ms * sizeof(uint32_t), kAlign);
  p->off_pos = off;
  off = align_up(off + (size_t)units * splits * p->ms * sizeof(int32_t), kAlign);
  p->end = off;
  return SA_OK;
}

int plan_decode(const sa_shape& s, int M, DecodePlan* p) {
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  const int G = s.num_q_heads / s.num_kv_heads;
  int64_t splits = std::max<int64_t>(1, ceil_div(kDecodeTargetBlocks, units));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, ceil_div(M, kMinRowsPerSplit)));
  const int64_t rps = ceil_div(M, splits);
  splits = ceil_div(M, rps);          // no empty workgroups
  p->units = (int)units;
  p->splits = (int)splits;
  p->rows_per_split = (int)rps;
  size_t off = 0;
  const size_t parts = (size_t)units * splits * G;
  p->off_m = off;
  off = align_up(off + parts * sizeof(float), kAlign);
  p->off_l = off;
  off = align_up(off + parts * sizeof(float), kAlign);
  p->off_o = off;
  off = align_up(off + parts * s.head_dim * sizeof(float), kAlign);
  p->end = off;
  return SA_OK;
}

static void plan_partials(const sa_shape& s, DecodePlan* p) {
  const int G = s.num_q_heads / s.num_kv_heads;
  size_t off = 0;
  const size_t parts = (size_t)p->units * p->splits * G;
  p->off_m = off;
  off = align_up(off + parts * sizeof(float), kAlign);
  p->off_l = off;
  off = align_up(off + parts * sizeof(float), kAlign);
  p->off_o = off;
  off = align_up(off + parts * s.head_dim * sizeof(float), kAlign);
  p->end = off;
}

int plan_dense(const sa_shape& s, int n_max, DecodePlan* p) {
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  int64_t splits = std::max<int64_t>(1, ceil_div(kDecodeTargetBlocks, units));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, ceil_div(n_max, kDenseSplitRows)));
  const int64_t rps = (int64_t)align_up((size_t)ceil_div(n_max, splits), kDenseSplitRows);
  splits = ceil_div(n_max, rps);
  p->units = (int)units;
  p->splits = (int)splits;
  p->rows_per_split = (int)rps;
  plan_partials(s, p);
  return SA_OK;
}

size_t dense_workspace_bytes(const sa_shape& s, int n_max) {
  if (check_shape(&s) != SA_OK) return 0;
  if (n_max < 1 || n_max > s.capacity) return 0;
  DecodePlan dp;
  if (plan_dense(s, n_max, &dp) != SA_OK) return 0;
  return std::max<size_t>(dp.end, kAlign);
}

int plan_filter(const sa_shape& s, int n_max, int M, FilterPlan* p, int cu_count,
                bool all_scores) {
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  *p = FilterPlan{};
  p->units = (int)units;
  if (n_max > kFilterMaxN || M > kFilterMaxM || M >= n_max) return SA_OK;
  const int64_t keep_target = std::min<int64_t>((int64_t)kSampleSafety * M, kFilterKeepTarget);
  // One workgroup per unit when the units fill whole rounds of the CUs (at
  // least kUnitMinFill of them), the attention needs no split (units >=
  // kDecodeTargetBlocks) and fits the merge's LDS (G d <= kFusedAttendMaxGD),
  // and the wave lists hold twice the kept keys they expect.
  if (cu_count > 0 && units >= kDecodeTargetBlocks &&
      (s.num_q_heads / s.num_kv_heads) * s.head_dim <= kFusedAttendMaxGD &&
      2 * keep_target <= (int64_t)kUnitWaves * kUnitCap) {
    const int64_t rounds = (units + cu_count - 1) / cu_count;
    if ((double)units >= kUnitMinFill * (double)(rounds * cu_count)) {
      p->enabled = true;
      p->unit_wg = true;
      p->chunk = (int)align_up((size_t)n_max, kChunkBlock);
      p->splits = 1;
      p->cap = kUnitCap;
      p->cslots = 0;
      p->spill_cap = kFilterSlots / 2;
      p->ustride = p->spill_cap;
      size_t off = 0;
      p->off_thr = off;
      off = align_up(off + (size_t)units * sizeof(uint32_t), kAlign);
      p->off_qt = off;
      off = align_up(off + (size_t)units * 32 * sizeof(float), kAlign);
      p->off_path = off;
      off = align_up(off + (size_t)units * sizeof(int32_t), kAlign);
      p->off_cnt = off;
      off = align_up(off + (size_t)units * 2 * sizeof(int32_t), kAlign);
      p->off_cand = off;                       // the spill pool, (key, position) pairs
      off = align_up(off + (size_t)units * p->ustride * 2 * sizeof(uint32_t), kAlign);
      p->end = off;
      return SA_OK;
    }
  }
  if (all_scores && n_max <= kScoresMaxN) {
    // scoring workgroups of kScoreChunkMin positions or more, about one per
    // CU (a 1024-thread workgroup fills one)
    int64_t chunk = kScoreChunkMin;
    while (chunk < n_max && units * ceil_div(n_max, chunk) > kDecodeTargetBlocks) chunk *= 2;
    p->enabled = true;
    p->all_scores = true;
    p->chunk = (int)chunk;
    p->splits = (int)ceil_div(n_max, chunk);
    p->sstride = (int64_t)align_up((size_t)n_max, 4096);   // whole 4096-float rows of the layout
    size_t off = 0;
    p->off_thr = off;
    off = align_up(off + (size_t)units * sizeof(uint32_t), kAlign);
    p->off_qt = off;
    off = align_up(off + (size_t)units * 32 * sizeof(float), kAlign);
    p->off_path = off;
    off = align_up(off + (size_t)units * sizeof(int32_t), kAlign);
    p->off_cnt = off;                          // (no counts)
    p->off_cand = off;                         // the scores, [units][sstride] floats
    off = align_up(off + (size_t)units * p->sstride * sizeof(float), kAlign);
    p->end = off;
    return SA_OK;
  }
  // Chunks as large as 32768 positions (fewer, longer workgroups stream
  // better: about two rounds of the chip's slots), smaller while the grid is
  // short of 1024 workgroups, but never more than 16 per unit (lists keep
  // >= 128 slots).
  int64_t chunk = kFilterMaxChunk;
  while (chunk > 2048 && units * ceil_div(n_max, chunk) < 1024) chunk >>= 1;
  int64_t splits = ceil_div(n_max, chunk);
  const int64_t max_splits = kFilterSlots / (kFilterWaves * kFilterMinCap);
  if (splits > max_splits) {
    chunk = align_up((size_t)ceil_div(n_max, max_splits), kChunkBlock);
    splits = ceil_div(n_max, chunk);
  }
  // Wave lists of twice the kept keys a list expects (the bound keeps about
  // min(kSampleSafety M, kFilterKeepTarget) keys per unit, spread evenly over
  // the lists), so that only clustered high scores spill.
  const int64_t lists = splits * kFilterWaves;
  int64_t cap = kFilterMinCap;
  while (cap < kFilterMaxCap && cap * lists < 2 * keep_target) cap *= 2;
  p->enabled = true;
  p->chunk = (int)chunk;
  p->splits = (int)splits;
  p->cap = (int)cap;
  p->cslots = (int)(cap * kFilterWaves);
  size_t off = 0;
  p->off_thr = off;
  off = align_up(off + (size_t)units * sizeof(uint32_t), kAlign);
  p->off_qt = off;
  off = align_up(off + (size_t)units * 32 * sizeof(float), kAlign);
  p->off_path = off;
  off = align_up(off + (size_t)units * sizeof(int32_t), kAlign);
  // A wave list that fills up goes to the unit's spill pool (one atomic
  // reservation per full list), which follows the unit's chunk slots; its
  // count follows the unit's chunk counts.  Half of the merge's capacity:
  // with the ~3M kept keys of a unit that leaves room for clusters of several
  // thousand high-scoring positions.
  p->spill_cap = kFilterSlots / 2;
  p->ustride = splits * p->cslots + p->spill_cap;
  p->off_cnt = off;
  off = align_up(off + (size_t)units * (splits + 1) * sizeof(int32_t), kAlign);
  p->off_cand = off;                       // (key, position) pairs
  off = align_up(off + (size_t)units * p->ustride * 2 * sizeof(uint32_t), kAlign);
  p->end = off;
  return SA_OK;
}

size_t workspace_bytes(const sa_shape& s, int n_max, int M) {
  if (check_shape(&s) != SA_OK) return 0;
  if (n_max < 1 || n_max > s.capacity || M < 1) return 0;
  DecodePlan dp;
  if (plan_decode(s, M, &dp) != SA_OK) return 0;
  size_t need = dp.end;
  if (M <= n_max) {
    TopmPlan tp;
    if (plan_topm(s, n_max, M, &tp) != SA_OK) return 0;
    need = std::max(need, tp.end);
    for (bool all_scores : {false, true}) {
      FilterPlan fp;
      if (plan_filter(s, n_max, M, &fp, 0, all_scores) != SA_OK) return 0;
      if (fp.enabled) need = std::max(need, fp.end);
      if (fused_attend_ok(s, fp)) need = std::max(need, fused_partials_offset(fp) + dp.end);
    }
  }
  return need;
}

}  // namespace sa

extern "C" size_t sparse_attn_workspace_size(const sa_shape* shape, int32_t n_max,
                                             int32_t M) {
  if (!shape) return 0;
  return sa::workspace_bytes(*shape, n_max, M);
}

extern "C" size_t sparse_attn_dense_workspace_size(const sa_shape* shape, int32_t n_max) {
  if (!shape) return 0;
  return sa::dense_workspace_bytes(*shape, n_max);
}

extern "C" const char* sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported shape or size";
    case SA_ERR_WORKSPACE: return "workspace missing or too small";
    case SA_ERR_HIP: return "HIP runtime or launch error";
    case SA_ERR_TOO_LARGE:
      return "shape needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}
