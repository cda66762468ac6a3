// Host-side argument checks and launch planning.  No HIP types: this part is
// plain C++ so that its logic can be exercised without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// Fixed launch geometry shared with the kernels.
constexpr int kBlock = 256;              // threads per workgroup (4 waves of 64)
constexpr int kChunkBlock = 512;         // chunk-select workgroups (8 waves)
constexpr int kMaxKeysPerThread = 64;    // register-resident merge keys
constexpr int kMaxChunkKeysPerThread = 32;
constexpr int kMaxChunk = kChunkBlock * kMaxChunkKeysPerThread;   // 16384 positions
constexpr int kMinChunk = kChunkBlock;                            // 512 positions
constexpr int kMergeTile = kBlock * kMaxKeysPerThread;  // keys per merge tile
constexpr int kMaxSplits = 1024;         // chunks per (b, KV head) unit
constexpr int kTargetBlocks = 2048;      // enough workgroups for 256 CUs
constexpr int kMinRowsPerSplit = 64;     // attention rows per workgroup (min)
constexpr int kDecodeTargetBlocks = 256; // attention workgroups (16 waves) per launch: one per CU
constexpr int kDenseSplitRows = 256;     // dense baseline: rows per split, a multiple of this
constexpr int kSupersetSlack = 1024;     // extra candidate slots per chunk (see plan_topm)
constexpr int kMergeThreadsHost = 1024;  // merge workgroup size
constexpr int kMaxMergeKeysPerThread = 24;   // register-resident merge (else LDS tiles)
constexpr size_t kAlign = 256;

struct TopmPlan {
  int units;        // B * Hkv
  int chunk;        // positions per chunk workgroup (multiple of 512)
  int kpt;          // keys per thread = chunk / 512
  int splits;       // chunks per unit
  int mc;           // exact candidates per chunk at most = min(M, chunk)
  int ms;           // candidate slots per chunk (multiple of 1024, >= mc)
  int merge_kpt;    // merge keys per thread when registers hold them all, else 0
  size_t off_cnt, off_key, off_pos, end;   // byte offsets in the workspace
};

// Filter path of the fused selection: a sampled per-unit lower bound on the
// M-th score, chunks that keep only the keys at or above it (per-wave lists,
// no per-chunk selection), and a merge that selects exactly over the lists
// and falls back to an exact pass over the unit when the bound was too high
// or a list overflowed.
constexpr int kFilterMaxN = 1 << 19;     // merge marks selected positions in an LDS bitmap
constexpr int kFilterMaxM = 6144;        // selected positions staged in LDS by the merge
constexpr int kFilterSlots = 16384;      // kept keys the merge holds per unit (16 per thread)
constexpr int kFilterMinCap = 128;       // slots per wave list, at least
constexpr int kFilterMaxCap = 512;       // slots per wave list, at most (staged in LDS)
constexpr int kFilterMaxChunk = 32768;   // positions per filter workgroup, at most
constexpr int kFilterWaves = 8;          // lists per chunk (one per wave of 512 threads)
constexpr int kSampleBlocks = 128;       // sampled position blocks per unit
constexpr int kSampleBlock = 8;          // positions per sampled block (256 B of FP8 rows)
constexpr int kSampleSafety = 3;         // the bound aims at ~3 M keys per unit...
constexpr int kFilterKeepTarget = kFilterSlots / 4 * 3;   // ...but at most 12288 (3/4 of
                                         // the merge's slots: >= 2 M up to kFilterMaxM)

// The filter path's merge workgroup can go on to attend over its selection
// when the 16 waves' G x d output tiles fit the merge's 64 KB bitmap.
constexpr int kFusedAttendMaxGD = (kFilterMaxN / 8) / (16 * 4);   // G d <= 1024

// One workgroup per unit (the units fill the chip): a 1024-thread workgroup
// streams the whole unit, keeps its candidates in 16 LDS wave lists, merges
// them and attends, in one launch.
constexpr int kUnitWaves = 16;
constexpr int kUnitCap = 768;            // slots per wave list
constexpr double kUnitMinFill = 0.9;     // units / (CUs x rounds of workgroups), at least

// Short units, few of them: every position is scored (one launch, chunks of
// the unit in parallel, a 4-byte score per position) and the merge selects
// exactly over all of a unit's scores, held 16 per thread in position order
// (no bound, no filter, no fallback).
constexpr int kScoresMaxN = kFilterSlots;   // 16384 positions per unit, at most
constexpr int kScoreChunkMin = 2048;        // positions per scoring workgroup, at least

struct FilterPlan {
  bool enabled;
  bool unit_wg;     // one workgroup per unit (splits = 1, lists in LDS, spill pool only)
  bool all_scores;  // every position scored, merge over the scores (chunk, splits: the
                    // scoring workgroups; off_cand: the scores, sstride floats per unit)
  int64_t sstride;
  int units;
  int chunk;        // positions per filter workgroup (multiple of 512)
  int splits;       // chunks per unit
  int cap;          // slots per wave list (power of two)
  int cslots;       // candidate slots per chunk = 8 * cap (one list per wave)
  int spill_cap;    // slots of the unit's spill pool (lists that filled up mid-chunk)
  int64_t ustride;  // pairs per unit: splits * cslots chunk slots, then the spill pool
  size_t off_thr, off_qt, off_path, off_cnt, off_cand, end;   // off_path: per unit, how the
                                         // last merge selected (0 kept keys, 1 exact pass)
};

struct DecodePlan {
  int units;
  int splits;           // workgroups per unit
  int rows_per_split;   // selected rows per workgroup
  size_t off_m, off_l, off_o, end;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape checks shared by every entry point (SA_OK or a negative status).
int check_shape(const sa_shape* s);
// Non-null and aligned to `align` bytes.
bool ptr_ok(const void* p, size_t align);

int plan_topm(const sa_shape& s, int n_max, int M, TopmPlan* out);
int plan_decode(const sa_shape& s, int M, DecodePlan* out);
// Dense attention baseline over n_max rows, split like the sparse attention
// (splits of a multiple of kDenseSplitRows rows).
int plan_dense(const sa_shape& s, int n_max, DecodePlan* out);
size_t dense_workspace_bytes(const sa_shape& s, int n_max);
// Fills `out`; out->enabled is false when the shape needs the chunk-exact path.
// cu_count > 0 (the device's compute units) allows the one-workgroup-per-unit
// plan where it applies (its workspace never exceeds the chunked plan's);
// all_scores allows the plan that scores every position, for units of at most
// kScoresMaxN positions that the unit plan does not take.  workspace_bytes
// covers every plan.
int plan_filter(const sa_shape& s, int n_max, int M, FilterPlan* out, int cu_count = 0,
                bool all_scores = false);
// Where the fused merge + attention keeps its split states: past the filter
// path's workspace.
inline size_t fused_partials_offset(const FilterPlan& fp) { return align_up(fp.end, kAlign); }
inline bool fused_attend_ok(const sa_shape& s, const FilterPlan& fp) {
  return fp.enabled && (s.num_q_heads / s.num_kv_heads) * s.head_dim <= kFusedAttendMaxGD;
}
size_t workspace_bytes(const sa_shape& s, int n_max, int M);

}  // namespace sa
