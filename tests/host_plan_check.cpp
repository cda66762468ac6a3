// Host planning code under AddressSanitizer and UndefinedBehaviorSanitizer
// (built with g++ by tests/test_host_plan_sanitized.py; no GPU, no HIP).
//
// Sweeps the shapes check_shape admits up to its limits (2^24 units,
// capacity * head_dim * 2 up to INT32_MAX) with n_max and M at and around the
// planners' thresholds, and checks every plan's invariants: workspace offsets
// 256-byte aligned, ascending and inside the reported size; chunks cover the
// positions; attention splits cover the budget with no empty split; every
// per-unit quantity the kernels index with 32-bit arithmetic fits in int32.
// Signed overflow anywhere in the planning arithmetic aborts (UBSan).
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <vector>

#include "host_plan.h"

using namespace sa;

static int failures = 0;

#define CHECK(cond, ...)                                          \
  do {                                                            \
    if (!(cond)) {                                                \
      ++failures;                                                 \
      std::fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                          \
      std::fprintf(stderr, "\n");                                 \
    }                                                             \
  } while (0)

static bool aligned(size_t x) { return x % kAlign == 0; }

static void check_one(const sa_shape& s, int n_max, int M) {
  const size_t ws = sparse_attn_workspace_size(&s, n_max, M);
  const bool args_ok = n_max >= 1 && n_max <= s.capacity && M >= 1;
  if (!args_ok) {
    CHECK(ws == 0, "n_max %d M %d cap %d: size %zu for invalid arguments", n_max, M, s.capacity, ws);
    return;
  }
  const int64_t units = (int64_t)s.batch * s.num_kv_heads;
  const int G = s.num_q_heads / s.num_kv_heads;
  DecodePlan dp;
  CHECK(plan_decode(s, M, &dp) == SA_OK, "plan_decode M %d", M);
  CHECK(dp.units == units, "units");
  CHECK((int64_t)dp.splits * dp.rows_per_split >= M, "splits cover M");
  CHECK((int64_t)(dp.splits - 1) * dp.rows_per_split < M, "no empty split");
  CHECK(dp.splits >= 1 && dp.splits <= 256, "splits %d within the combine's limit", dp.splits);
  CHECK(units * dp.splits <= INT32_MAX, "decode grid fits");
  CHECK(aligned(dp.off_m) && aligned(dp.off_l) && aligned(dp.off_o) && aligned(dp.end), "align");
  CHECK(dp.off_m <= dp.off_l && dp.off_l <= dp.off_o && dp.off_o <= dp.end, "order");
  CHECK(dp.end >= dp.off_o + (size_t)units * dp.splits * G * s.head_dim * 4, "partials fit");
  CHECK(ws >= dp.end, "ws %zu >= decode %zu", ws, dp.end);
  if (M > n_max) return;

  TopmPlan tp;
  const int st = plan_topm(s, n_max, M, &tp);
  CHECK(st == SA_OK, "plan_topm n_max %d M %d -> %d (size %zu)", n_max, M, st, ws);
  if (st != SA_OK) return;
  CHECK((int64_t)tp.splits * tp.chunk >= n_max, "chunks cover n_max");
  CHECK(tp.splits <= kMaxSplits && tp.chunk % kChunkBlock == 0, "chunk shape");
  CHECK(tp.ms >= tp.mc && tp.ms % kMergeThreadsHost == 0 && tp.ms <= tp.chunk + 1024, "slots");
  CHECK(units * tp.splits <= INT32_MAX, "chunk grid fits");
  CHECK(aligned(tp.off_cnt) && aligned(tp.off_key) && aligned(tp.off_pos) && aligned(tp.end),
        "topm align");
  CHECK(tp.off_key >= tp.off_cnt + (size_t)units * tp.splits * 4, "counts fit");
  CHECK(tp.off_pos >= tp.off_key + (size_t)units * tp.splits * tp.ms * 4, "keys fit");
  CHECK(tp.end >= tp.off_pos + (size_t)units * tp.splits * tp.ms * 4, "positions fit");
  CHECK(ws >= tp.end, "ws covers the chunk-exact plan");

  FilterPlan fp;
  CHECK(plan_filter(s, n_max, M, &fp) == SA_OK, "plan_filter");
  const bool want = n_max <= kFilterMaxN && M <= kFilterMaxM && M < n_max;
  CHECK(fp.enabled == want, "filter enabled %d for n_max %d M %d", (int)fp.enabled, n_max, M);
  if (!fp.enabled) return;
  CHECK((int64_t)fp.splits * fp.chunk >= n_max && fp.chunk % kChunkBlock == 0, "filter chunks");
  CHECK(fp.splits >= 1 && fp.splits <= kFilterSlots / (kFilterWaves * kFilterMinCap),
        "filter splits %d", fp.splits);
  CHECK(fp.cap >= kFilterMinCap && fp.cap <= kFilterMaxCap && (fp.cap & (fp.cap - 1)) == 0,
        "cap %d", fp.cap);
  CHECK(fp.cslots == fp.cap * kFilterWaves, "cslots");
  CHECK(fp.ustride == (int64_t)fp.splits * fp.cslots + fp.spill_cap, "ustride");
  // in-unit candidate offsets are formed in 32 bits by the kernels
  CHECK(fp.ustride * 2 <= INT32_MAX, "ustride fits");
  CHECK(units * fp.splits <= INT32_MAX, "filter grid fits");
  CHECK(aligned(fp.off_thr) && aligned(fp.off_qt) && aligned(fp.off_path) &&
            aligned(fp.off_cnt) && aligned(fp.off_cand) && aligned(fp.end), "filter align");
  CHECK(fp.off_qt >= fp.off_thr + (size_t)units * 4, "thr fits");
  CHECK(fp.off_path >= fp.off_qt + (size_t)units * 32 * 4, "qt fits");
  CHECK(fp.off_cnt >= fp.off_path + (size_t)units * 4, "path fits");
  CHECK(fp.off_cand >= fp.off_cnt + (size_t)units * (fp.splits + 1) * 4, "counts fit");
  CHECK(fp.end >= fp.off_cand + (size_t)units * fp.ustride * 8, "candidates fit");
  CHECK(ws >= fp.end, "ws covers the filter plan");
  if (fused_attend_ok(s, fp))
    CHECK(ws >= fused_partials_offset(fp) + dp.end, "ws covers the fused partials");
  // the plan that scores every position
  {
    FilterPlan sp;
    CHECK(plan_filter(s, n_max, M, &sp, 0, true) == SA_OK, "plan_filter(all_scores)");
    CHECK(sp.enabled, "the scores plan keeps the filter path enabled");
    CHECK(sp.all_scores == (n_max <= kScoresMaxN), "scores plan for n_max %d", n_max);
    if (sp.all_scores) {
      CHECK(!sp.unit_wg, "one plan at a time");
      CHECK(sp.chunk >= kScoreChunkMin && sp.chunk % kChunkBlock == 0, "score chunk %d", sp.chunk);
      CHECK((int64_t)sp.splits * sp.chunk >= n_max && (int64_t)(sp.splits - 1) * sp.chunk < n_max,
            "score chunks cover n_max with none empty");
      CHECK(units * sp.splits <= INT32_MAX, "score grid fits");
      CHECK(sp.sstride >= n_max && sp.sstride % 4096 == 0, "score stride: whole rows of the layout");
      CHECK(aligned(sp.off_cand) && aligned(sp.end), "scores align");
      CHECK(sp.off_thr == fp.off_thr && sp.off_qt == fp.off_qt && sp.off_path == fp.off_path,
            "thr, qt and path flags where the chunked plan has them");
      CHECK(sp.off_cand >= sp.off_path + (size_t)units * 4, "scores after the path flags");
      CHECK(sp.end >= sp.off_cand + (size_t)units * sp.sstride * 4, "scores fit");
      // positions and offsets inside a unit's scores are formed in 32 bits
      CHECK(sp.sstride <= INT32_MAX, "score offsets fit");
      CHECK(ws >= sp.end, "ws %zu covers the scores plan %zu", ws, sp.end);
      if (fused_attend_ok(s, sp))
        CHECK(ws >= fused_partials_offset(sp) + dp.end, "ws covers the scores plan's partials");
    } else {
      CHECK(sp.end == fp.end && sp.splits == fp.splits, "no scores plan: the filter plan");
    }
  }
  // the one-workgroup-per-unit plan (on devices of these compute-unit counts)
  for (int cus : {80, 256, 304}) {
    FilterPlan up;
    CHECK(plan_filter(s, n_max, M, &up, cus) == SA_OK, "plan_filter(cu)");
    CHECK(up.enabled, "unit plan keeps the filter path enabled");
    if (!up.unit_wg) continue;
    CHECK(up.splits == 1 && up.cap == kUnitCap && up.ustride == up.spill_cap, "unit plan shape");
    CHECK(units >= kDecodeTargetBlocks && dp.splits == 1, "unit plan: attention unsplit");
    CHECK(up.off_thr == fp.off_thr && up.off_qt == fp.off_qt && up.off_path == fp.off_path,
          "thr, qt and path flags where the chunked plan has them");
    CHECK(up.off_cand >= up.off_cnt + (size_t)units * 2 * 4, "unit counts fit");
    CHECK(up.end >= up.off_cand + (size_t)units * up.ustride * 8, "spill pools fit");
    CHECK(up.end <= ws, "the workspace size covers the unit plan");
  }
}

int main() {
  // check_shape: limits
  sa_shape bad{1, 4, 1, 96, 16, 100};
  CHECK(check_shape(&bad) == SA_ERR_UNSUPPORTED, "head_dim 96");
  sa_shape big_g{1, 34, 2, 128, 32, 100};
  CHECK(check_shape(&big_g) == SA_ERR_UNSUPPORTED, "G 17");
  sa_shape too_many{(1 << 13) + 1, 1 << 11, 1 << 11, 128, 32, 100};   // units > 2^24
  CHECK(check_shape(&too_many) == SA_ERR_UNSUPPORTED, "units > 2^24");
  sa_shape too_long{1, 4, 1, 128, 32, (1 << 23)};          // 2^23 * 256 = 2^31 > INT32_MAX
  CHECK(check_shape(&too_long) == SA_ERR_UNSUPPORTED, "capacity * d * 2 > INT32_MAX");
  CHECK(check_shape(nullptr) == SA_ERR_INVALID, "null shape");

  const std::vector<sa_shape> shapes = {
      {1, 4, 1, 64, 16, 1024},
      {32, 32, 8, 128, 32, 131072},
      {8, 28, 4, 128, 32, 16384},
      {1, 16, 1, 64, 16, (1 << 24) - 1},          // longest admitted context, d = 64
      {1, 16, 1, 128, 32, (1 << 23) - 1},         // longest admitted context, d = 128
      {1 << 12, 1 << 12, 1 << 12, 64, 16, 4096},  // 2^24 units, G = 1
      {1 << 16, 1024, 256, 128, 32, 8192},        // 2^24 units, G = 4
      {3, 48, 3, 128, 16, 600001},
  };
  for (const sa_shape& s : shapes) {
    CHECK(check_shape(&s) == SA_OK, "shape admitted");
    const int cap = s.capacity;
    const std::vector<int> ns = {1, 2, 511, 512, 513, 2048, 6144, 6145, 65536, (1 << 19) - 1,
                                 1 << 19, (1 << 19) + 1, cap - 1, cap, cap + 1};
    for (int n : ns) {
      if (n < 1 || n > cap + 1) continue;
      const std::vector<int> ms = {1, 2, 64, 2047, 2048, 6143, 6144, 6145, n - 1, n, n + 1};
      for (int m : ms) {
        if (m < 0) continue;
        check_one(s, n, m);
      }
    }
  }
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("host plan checks passed\n");
  return 0;
}
