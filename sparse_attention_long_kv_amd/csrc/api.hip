// C-ABI entry points: host-side checks, planning, launches.
#include <cmath>
#include <cstdlib>
#include <mutex>

#include "host_plan.h"
#include "kernels.h"
#include "sparse_attn.h"

namespace {

using namespace sa;

bool sync_mode() {
  static const bool on = [] {
    const char* e = std::getenv("SPARSE_ATTN_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

int finish(hipError_t launch, hipStream_t stream) {
  if (launch != hipSuccess) return SA_ERR_HIP;
  if (sync_mode()) {
    if (hipStreamSynchronize(stream) != hipSuccess) return SA_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return SA_ERR_HIP;
  }
  return SA_OK;
}

// Compute units of the current device (0 if unknown), for the plan that runs
// one workgroup per unit when the units fill the chip.  SPARSE_ATTN_UNIT_WG=0
// in the environment keeps the chunked filter plan instead (both give the
// same bits; a testing aid).
int unit_cu_count() {
  const char* e = std::getenv("SPARSE_ATTN_UNIT_WG");
  if (e && e[0] == '0') return 0;
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static int cache[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// The plan that scores every position (short units, too few for one
// workgroup each) where it applies.  SPARSE_ATTN_SCORES_PLAN=0 in the
// environment keeps the filter plan instead (both give the same bits; a
// testing aid).
bool scores_plan_on() {
  const char* e = std::getenv("SPARSE_ATTN_SCORES_PLAN");
  return !(e && e[0] == '0');
}

LaunchCommon common(const sa_shape& s, void* stream) {
  LaunchCommon c;
  c.B = s.batch;
  c.Hq = s.num_q_heads;
  c.Hkv = s.num_kv_heads;
  c.G = s.num_q_heads / s.num_kv_heads;
  c.D = s.head_dim;
  c.R = s.rank;
  c.Ncap = s.capacity;
  c.units = s.batch * s.num_kv_heads;
  c.stream = (hipStream_t)stream;
  return c;
}

constexpr size_t A16 = 16, A4 = 4;

int check_topm_common(const sa_shape* shape, const int32_t* seq_lens, int32_t n_max,
                      int32_t M, const int32_t* idx, const void* ws, size_t ws_bytes,
                      TopmPlan* plan, bool need_idx = true) {
  if (seq_lens && !ptr_ok(seq_lens, A4)) return SA_ERR_INVALID;
  if (need_idx && !ptr_ok(idx, A4)) return SA_ERR_INVALID;
  if (n_max < 1 || n_max > shape->capacity) return SA_ERR_INVALID;
  if (M < 1 || M > n_max) return SA_ERR_INVALID;
  const int st = plan_topm(*shape, n_max, M, plan);
  if (st != SA_OK) return st;
  if (!ptr_ok(ws, kAlign) || ws_bytes < workspace_bytes(*shape, n_max, M)) return SA_ERR_WORKSPACE;
  return SA_OK;
}

}  // namespace

extern "C" int sparse_attn_append_kv(const sa_shape* shape, const int32_t* pos, int32_t T,
                                     const void* k_new, const void* v_new, const float* P,
                                     void* k_cache, void* v_cache, uint8_t* kp_cache,
                                     void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (T < 0 || T > shape->capacity) return SA_ERR_INVALID;
  if (!ptr_ok(pos, A4) || !ptr_ok(k_new, A16) || !ptr_ok(v_new, A16) || !ptr_ok(P, A4) ||
      !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) || !ptr_ok(kp_cache, A16))
    return SA_ERR_INVALID;
  if (T == 0) return SA_OK;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_append_kv(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp_cache), c.stream);
}

extern "C" int sparse_attn_project_keys(const sa_shape* shape, const void* k_cache,
                                        const float* P, int32_t n_begin, int32_t n_count,
                                        uint8_t* kp_cache, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (n_begin < 0 || n_count < 0 || (int64_t)n_begin + n_count > shape->capacity)
    return SA_ERR_INVALID;
  if (!ptr_ok(k_cache, A16) || !ptr_ok(P, A4) || !ptr_ok(kp_cache, A16)) return SA_ERR_INVALID;
  if (n_count == 0) return SA_OK;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_project_keys(c, k_cache, P, n_begin, n_count, kp_cache), c.stream);
}

extern "C" int sparse_attn_index_score(const sa_shape* shape, const void* q, const float* P,
                                       const uint8_t* kp_cache, const int32_t* seq_lens,
                                       int32_t n_max, float* scores, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(q, A16) || !ptr_ok(P, A4) || !ptr_ok(kp_cache, A16) || !ptr_ok(scores, A4))
    return SA_ERR_INVALID;
  if (seq_lens && !ptr_ok(seq_lens, A4)) return SA_ERR_INVALID;
  if (n_max < 1 || n_max > shape->capacity) return SA_ERR_INVALID;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_index_score(c, q, P, kp_cache, seq_lens, n_max, scores), c.stream);
}

extern "C" int sparse_attn_topm(const sa_shape* shape, const float* scores,
                                const int32_t* seq_lens, int32_t n_max, int32_t M, int32_t* idx,
                                void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(scores, A4)) return SA_ERR_INVALID;
  TopmPlan plan;
  st = check_topm_common(shape, seq_lens, n_max, M, idx, workspace, ws_bytes, &plan);
  if (st != SA_OK) return st;
  const LaunchCommon c = common(*shape, stream);
  // the filter path over the given scores where it applies (sampled bound,
  // filter, merge: the same idx as the chunk-exact path, in fewer bytes)
  FilterPlan fplan;
  st = plan_filter(*shape, n_max, M, &fplan, 0, scores_plan_on());
  if (st != SA_OK) return st;
  if (fplan.enabled)
    return finish(run_filter_select(c, fplan, kSelectBound | kSelectChunks | kSelectMerge,
                                    nullptr, nullptr, nullptr, seq_lens, n_max, M, idx,
                                    workspace, nullptr, nullptr, scores),
                  c.stream);
  return finish(run_select(c, plan, kSelectChunks | kSelectMerge, false, nullptr, nullptr, nullptr,
                           scores, seq_lens, n_max, M, idx, workspace),
                c.stream);
}

namespace {

// Launches stage mask `stages` of the fused selection (all of it for
// sparse_attn_index_topm).
int index_topm_stages(const sa_shape* shape, int stages, const void* q, const float* P,
                      const uint8_t* kp_cache, const int32_t* seq_lens, int32_t n_max, int32_t M,
                      int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(q, A16) || !ptr_ok(P, A4) || !ptr_ok(kp_cache, A16)) return SA_ERR_INVALID;
  TopmPlan plan;
  st = check_topm_common(shape, seq_lens, n_max, M, idx, workspace, ws_bytes, &plan,
                         /*need_idx=*/(stages & kSelectMerge) != 0);
  if (st != SA_OK) return st;
  FilterPlan fplan;
  st = plan_filter(*shape, n_max, M, &fplan, unit_cu_count(), scores_plan_on());
  if (st != SA_OK) return st;
  const LaunchCommon c = common(*shape, stream);
  if (fplan.enabled)
    return finish(run_filter_select(c, fplan, stages, q, P, kp_cache, seq_lens, n_max, M, idx,
                                    workspace),
                  c.stream);
  if ((stages & (kSelectChunks | kSelectMerge)) == 0) return SA_OK;
  return finish(run_select(c, plan, stages & (kSelectChunks | kSelectMerge), true, q, P, kp_cache,
                           nullptr, seq_lens, n_max, M, idx, workspace),
                c.stream);
}

}  // namespace

extern "C" int sparse_attn_index_topm(const sa_shape* shape, const void* q, const float* P,
                                      const uint8_t* kp_cache, const int32_t* seq_lens,
                                      int32_t n_max, int32_t M, int32_t* idx, void* workspace,
                                      size_t ws_bytes, void* stream) {
  return index_topm_stages(shape, kSelectBound | kSelectChunks | kSelectMerge, q, P, kp_cache,
                           seq_lens, n_max, M, idx, workspace, ws_bytes, stream);
}

extern "C" int sparse_attn_index_topm_stage(const sa_shape* shape, int32_t stage, const void* q,
                                            const float* P, const uint8_t* kp_cache,
                                            const int32_t* seq_lens, int32_t n_max, int32_t M,
                                            int32_t* idx, void* workspace, size_t ws_bytes,
                                            void* stream) {
  int mask;
  switch (stage) {
    case SA_STAGE_BOUND: mask = kSelectBound; break;
    case SA_STAGE_CANDIDATES: mask = kSelectChunks; break;
    case SA_STAGE_MERGE: mask = kSelectMerge; break;
    default: return SA_ERR_INVALID;
  }
  return index_topm_stages(shape, mask, q, P, kp_cache, seq_lens, n_max, M, idx, workspace,
                           ws_bytes, stream);
}

namespace {

constexpr int kStepAppend = 1, kStepCandidates = 2, kStepMerge = 4, kStepAttend = 8;

int decode_step_stages(const sa_shape* shape, int stages, const int32_t* pos, int32_t T,
                       const void* k_new, const void* v_new, const void* q, const float* P,
                       void* k_cache, void* v_cache, uint8_t* kp_cache, const int32_t* seq_lens,
                       int32_t n_max, int32_t M, float softmax_scale, int32_t* idx, void* out,
                       float* lse, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (T < 0 || T > shape->capacity) return SA_ERR_INVALID;
  if (!ptr_ok(pos, A4) || !ptr_ok(k_new, A16) || !ptr_ok(v_new, A16) || !ptr_ok(q, A16) ||
      !ptr_ok(P, A4) || !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) ||
      !ptr_ok(kp_cache, A16) || !ptr_ok(out, A16))
    return SA_ERR_INVALID;
  if (lse && !ptr_ok(lse, A4)) return SA_ERR_INVALID;
  if (!std::isfinite(softmax_scale)) return SA_ERR_INVALID;
  TopmPlan tplan;
  st = check_topm_common(shape, seq_lens, n_max, M, idx, workspace, ws_bytes, &tplan);
  if (st != SA_OK) return st;
  FilterPlan fplan;
  st = plan_filter(*shape, n_max, M, &fplan, unit_cu_count(), scores_plan_on());
  if (st != SA_OK) return st;
  DecodePlan dplan;
  st = plan_decode(*shape, M, &dplan);
  if (st != SA_OK) return st;
  const LaunchCommon c = common(*shape, stream);
  hipError_t e = hipSuccess;
  if (fplan.unit_wg) {
    // One workgroup per unit: the whole step is one launch (append, bound,
    // filter, merge and attention), made by the first stage; the later
    // stages have nothing left to do.
    const AttendFused att{&dplan, k_cache, v_cache, softmax_scale, out, lse, workspace};
    if (stages & kStepAppend) {
      const AppendRows rows{pos, T, k_new, v_new, k_cache, v_cache};
      e = run_filter_select(c, fplan, kSelectChunks, q, P, kp_cache, seq_lens, n_max, M, idx,
                            workspace, &rows, &att);
    }
    return finish(e, c.stream);
  }
  if (stages & kStepAppend) {
    if (fplan.enabled) {
      const AppendRows rows{pos, T, k_new, v_new, k_cache, v_cache};
      e = run_filter_select(c, fplan, kSelectBound, q, P, kp_cache, seq_lens, n_max, M, idx,
                            workspace, &rows);
    } else if (T > 0) {
      e = run_append_kv(c, pos, T, k_new, v_new, P, k_cache, v_cache, kp_cache);
    }
    if (e != hipSuccess) return finish(e, c.stream);
  }
  // merge and attention in one launch where the filter path allows it
  const bool fuse = (stages & kStepMerge) && (stages & kStepAttend) && fused_attend_ok(*shape, fplan);
  if (fuse) stages &= ~kStepAttend;
  const AttendFused att{&dplan, k_cache, v_cache, softmax_scale, out, lse,
                        (char*)workspace + fused_partials_offset(fplan)};
  for (int sel : {kStepCandidates, kStepMerge}) {
    if (!(stages & sel)) continue;
    const int mask = sel == kStepCandidates ? kSelectChunks : kSelectMerge;
    e = fplan.enabled ? run_filter_select(c, fplan, mask, q, P, kp_cache, seq_lens, n_max, M,
                                          idx, workspace, nullptr,
                                          fuse && sel == kStepMerge ? &att : nullptr)
                      : run_select(c, tplan, mask, true, q, P, kp_cache, nullptr, seq_lens, n_max,
                                   M, idx, workspace);
    if (e != hipSuccess) return finish(e, c.stream);
  }
  if (stages & kStepAttend)
    e = run_decode(c, dplan, q, k_cache, v_cache, idx, M, softmax_scale, out, lse, workspace);
  return finish(e, c.stream);
}

}  // namespace

extern "C" int sparse_attn_decode_step(const sa_shape* shape, const int32_t* pos, int32_t T,
                                       const void* k_new, const void* v_new, const void* q,
                                       const float* P, void* k_cache, void* v_cache,
                                       uint8_t* kp_cache, const int32_t* seq_lens, int32_t n_max,
                                       int32_t M, float softmax_scale, int32_t* idx, void* out,
                                       float* lse, void* workspace, size_t ws_bytes,
                                       void* stream) {
  return decode_step_stages(shape, kStepAppend | kStepCandidates | kStepMerge | kStepAttend, pos,
                            T, k_new, v_new, q, P, k_cache, v_cache, kp_cache, seq_lens, n_max,
                            M, softmax_scale, idx, out, lse, workspace, ws_bytes, stream);
}

extern "C" int sparse_attn_decode_step_stage(const sa_shape* shape, int32_t stage,
                                             const int32_t* pos, int32_t T, const void* k_new,
                                             const void* v_new, const void* q, const float* P,
                                             void* k_cache, void* v_cache, uint8_t* kp_cache,
                                             const int32_t* seq_lens, int32_t n_max, int32_t M,
                                             float softmax_scale, int32_t* idx, void* out,
                                             float* lse, void* workspace, size_t ws_bytes,
                                             void* stream) {
  int mask;
  switch (stage) {
    case SA_STEP_APPEND_BOUND: mask = kStepAppend; break;
    case SA_STEP_CANDIDATES: mask = kStepCandidates; break;
    case SA_STEP_MERGE: mask = kStepMerge; break;
    case SA_STEP_ATTEND: mask = kStepAttend; break;
    case SA_STEP_SELECT_ATTEND: mask = kStepMerge | kStepAttend; break;
    default: return SA_ERR_INVALID;
  }
  return decode_step_stages(shape, mask, pos, T, k_new, v_new, q, P, k_cache, v_cache, kp_cache,
                            seq_lens, n_max, M, softmax_scale, idx, out, lse, workspace, ws_bytes,
                            stream);
}

extern "C" int sparse_attn_decode(const sa_shape* shape, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* idx, int32_t M,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(q, A16) || !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) || !ptr_ok(idx, A4) ||
      !ptr_ok(out, A16))
    return SA_ERR_INVALID;
  if (lse && !ptr_ok(lse, A4)) return SA_ERR_INVALID;
  if (M < 1 || !std::isfinite(softmax_scale)) return SA_ERR_INVALID;
  DecodePlan plan;
  st = plan_decode(*shape, M, &plan);
  if (st != SA_OK) return st;
  if (!ptr_ok(workspace, kAlign) || ws_bytes < plan.end) return SA_ERR_WORKSPACE;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_decode(c, plan, q, k_cache, v_cache, idx, M, softmax_scale, out, lse,
                           workspace),
                c.stream);
}

extern "C" int sparse_attn_dense_decode(const sa_shape* shape, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const int32_t* seq_lens, int32_t n_max,
                                        float softmax_scale, void* out, float* lse,
                                        void* workspace, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(q, A16) || !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) || !ptr_ok(out, A16))
    return SA_ERR_INVALID;
  if ((lse && !ptr_ok(lse, A4)) || (seq_lens && !ptr_ok(seq_lens, A4))) return SA_ERR_INVALID;
  if (n_max < 1 || n_max > shape->capacity || !std::isfinite(softmax_scale))
    return SA_ERR_INVALID;
  DecodePlan plan;
  st = plan_dense(*shape, n_max, &plan);
  if (st != SA_OK) return st;
  if (!ptr_ok(workspace, kAlign) || ws_bytes < dense_workspace_bytes(*shape, n_max))
    return SA_ERR_WORKSPACE;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_dense_decode(c, plan, q, k_cache, v_cache, seq_lens, n_max, softmax_scale,
                                 out, lse, workspace),
                c.stream);
}

extern "C" int sparse_attn_gather_kv(const sa_shape* shape, const int32_t* idx, int32_t M,
                                     const void* k_cache, const void* v_cache, void* k_out,
                                     void* v_out, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(idx, A4) || !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) ||
      !ptr_ok(k_out, A16) || !ptr_ok(v_out, A16))
    return SA_ERR_INVALID;
  if (M < 1 || M > shape->capacity) return SA_ERR_INVALID;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_gather_kv(c, idx, M, k_cache, v_cache, k_out, v_out), c.stream);
}

extern "C" int sparse_attn_linear_gate(const sa_shape* shape, const void* q, const void* k_new,
                                       const void* v_new, float* S, float* z,
                                       const float* w_gate, const void* o_sparse, void* out,
                                       int32_t update_state, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(q, A16) || !ptr_ok(k_new, A16) || !ptr_ok(v_new, A16) || !ptr_ok(S, A4) ||
      !ptr_ok(z, A4) || !ptr_ok(w_gate, A4) || !ptr_ok(o_sparse, A16) || !ptr_ok(out, A16))
    return SA_ERR_INVALID;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_linear_gate(c, q, k_new, v_new, S, z, w_gate, o_sparse, out, update_state),
                c.stream);
}

extern "C" int sparse_attn_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                       void* stream) {
  if (!ptr_ok(buf, A16) || !ptr_ok(sink, A4)) return SA_ERR_INVALID;
  if (bytes == 0 || bytes % ((size_t)4 << 20) != 0 || bytes / ((size_t)4 << 20) > INT32_MAX)
    return SA_ERR_INVALID;
  return finish(run_stream_read(buf, bytes, sink, (hipStream_t)stream), (hipStream_t)stream);
}

extern "C" int sparse_attn_selection_fallbacks(const sa_shape* shape, int32_t n_max, int32_t M,
                                               const void* workspace, size_t ws_bytes,
                                               int32_t* count, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(count, A4)) return SA_ERR_INVALID;
  if (n_max < 1 || n_max > shape->capacity || M < 1 || M > n_max) return SA_ERR_INVALID;
  if (!ptr_ok(workspace, kAlign) || ws_bytes < workspace_bytes(*shape, n_max, M))
    return SA_ERR_WORKSPACE;
  FilterPlan fplan;
  st = plan_filter(*shape, n_max, M, &fplan, unit_cu_count(), scores_plan_on());
  if (st != SA_OK) return st;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_count_fallbacks(c, fplan, workspace, count), c.stream);
}

extern "C" int sparse_attn_selection_plan(const sa_shape* shape, int32_t n_max, int32_t M) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (n_max < 1 || n_max > shape->capacity || M < 1 || M > n_max) return SA_ERR_INVALID;
  TopmPlan tplan;
  st = plan_topm(*shape, n_max, M, &tplan);
  if (st != SA_OK) return st;
  FilterPlan fplan;
  st = plan_filter(*shape, n_max, M, &fplan, unit_cu_count(), scores_plan_on());
  if (st != SA_OK) return st;
  if (!fplan.enabled) return SA_PLAN_CHUNK_EXACT;
  if (fplan.all_scores) return SA_PLAN_SCORES;
  return fplan.unit_wg ? SA_PLAN_UNIT : SA_PLAN_FILTER;
}

extern "C" int sparse_attn_row_read(const sa_shape* shape, const int32_t* idx, int32_t M,
                                    const void* k_cache, const void* v_cache, int32_t mode,
                                    uint32_t* sink, void* stream) {
  int st = check_shape(shape);
  if (st != SA_OK) return st;
  if (!ptr_ok(idx, A4) || !ptr_ok(k_cache, A16) || !ptr_ok(v_cache, A16) || !ptr_ok(sink, A4))
    return SA_ERR_INVALID;
  if (M < 1 || (mode != 0 && mode != 1)) return SA_ERR_INVALID;
  const LaunchCommon c = common(*shape, stream);
  return finish(run_row_read(c, idx, M, k_cache, v_cache, mode, sink), c.stream);
}
