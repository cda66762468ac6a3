// Launch entry points of the kernel translation units (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_plan.h"

namespace sa {

struct LaunchCommon {
  int B, Hq, Hkv, G, D, R, Ncap, units;
  hipStream_t stream;
};

hipError_t run_append_kv(const LaunchCommon& c, const int32_t* pos, int T, const void* k_new,
                         const void* v_new, const float* P, void* k_cache, void* v_cache,
                         uint8_t* kp);
hipError_t run_project_keys(const LaunchCommon& c, const void* k_cache, const float* P,
                            int n_begin, int n_count, uint8_t* kp);
hipError_t run_index_score(const LaunchCommon& c, const void* q, const float* P,
                           const uint8_t* kp, const int32_t* seq_lens, int n_max,
                           float* scores);
// Selection runs as two launches: per-chunk candidates (kSelectChunks; fused
// == true computes the scores from (q, P, kp), otherwise reads `scores`), then
// the per-unit merge into idx (kSelectMerge).  `stages` picks either or both.
constexpr int kSelectChunks = 1, kSelectMerge = 2, kSelectBound = 4;
hipError_t run_select(const LaunchCommon& c, const TopmPlan& plan, int stages, bool fused,
                      const void* q, const float* P, const uint8_t* kp, const float* scores,
                      const int32_t* seq_lens, int n_max, int M, int32_t* idx,
                      void* workspace);
// New rows appended by the decode-step prologue (see run_filter_select).
struct AppendRows {
  const int32_t* pos;
  int T;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
};

// Attention run by the merge launch of the filter path, with run_decode's
// plan and arguments; the split states (plan->splits > 1) go to `partials`,
// which must not overlap the selection's workspace.
struct AttendFused {
  const DecodePlan* plan;
  const void* k_cache;
  const void* v_cache;
  float scale;
  void* out;
  float* lse;
  void* partials;
};

// Filter path of the fused selection (plan.enabled): stages kSelectBound
// (sampled bound; with `rows`, the same launch first appends those rows),
// kSelectChunks (filtering chunks), kSelectMerge (with `att`, each merge
// workgroup then attends over the selection, followed by the split merge
// when there are several splits; needs G d <= 1024).  With `scores`
// ([B][Hkv][n_max] fp32), the stages select over those scores instead of
// scoring the FP8 cache (q, P, kp unused; no rows, no att).
hipError_t run_filter_select(const LaunchCommon& c, const FilterPlan& plan, int stages,
                             const void* q, const float* P, const uint8_t* kp,
                             const int32_t* seq_lens, int n_max, int M, int32_t* idx,
                             void* workspace, const AppendRows* rows = nullptr,
                             const AttendFused* att = nullptr, const float* scores = nullptr);
// Diagnostic: units of the last filter-path selection in `workspace` that
// took the exact streaming pass, written to *count (-1 without a filter path).
hipError_t run_count_fallbacks(const LaunchCommon& c, const FilterPlan& plan,
                               const void* workspace, int32_t* count);
hipError_t run_decode(const LaunchCommon& c, const DecodePlan& plan, const void* q,
                      const void* k_cache, const void* v_cache, const int32_t* idx, int M,
                      float scale, void* out, float* lse, void* workspace);
// Comparison baselines: dense attention over every valid row (plan from
// plan_dense), and the copy of the selected rows into contiguous buffers.
hipError_t run_dense_decode(const LaunchCommon& c, const DecodePlan& plan, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                            int n_max, float scale, void* out, float* lse, void* workspace);
hipError_t run_gather_kv(const LaunchCommon& c, const int32_t* idx, int M, const void* k_cache,
                         const void* v_cache, void* k_out, void* v_out);
struct DecodeArgs;
// Merge of the split states when DecodeArgs::S > 1 (no launch otherwise).
// Streaming read of `bytes` (a positive multiple of 4 MiB) at buf.
hipError_t run_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
// Reads of the selected K and V rows alone (mode 0: into registers, 1: into LDS).
hipError_t run_row_read(const LaunchCommon& c, const int32_t* idx, int M, const void* k_cache,
                        const void* v_cache, int mode, uint32_t* sink);

hipError_t run_combine(const LaunchCommon& c, const DecodeArgs& a);
hipError_t run_linear_gate(const LaunchCommon& c, const void* q, const void* k_new,
                           const void* v_new, float* S, float* z, const float* w_gate,
                           const void* o_sparse, void* out, int update_state);

}  // namespace sa
