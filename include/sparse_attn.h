/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) indexer-selected sparse decode
 * library (libsparse_attn.so).
 *
 * One decode step of token-sparse attention over a long KV cache, as the JSSA
 * article (rit.work blog, "Joint Subspace Sparse Attention for Efficient
 * Long-Context Decoding") describes it in "How JSSA preserves token order":
 *
 *   1. append the new token's key/value rows to the bf16 KV cache and its
 *      low-rank projection (k . P, rounded to FP8 E4M3) to the projected-key
 *      cache;                                        -> sparse_attn_append_kv
 *   2. average the GQA group's queries, project them onto the KV head's basis
 *      P and score every cached position against the FP8 cache;
 *                                                    -> sparse_attn_index_score
 *   3. keep the M highest-scoring positions per KV head (the "top-k" of the
 *      DeepSeek Sparse Attention indexer in the IndexCache article, "DeepSeek
 *      Sparse Attention: a step towards efficiency");  -> sparse_attn_topm
 *      (steps 2 and 3 fused, scores never written:    -> sparse_attn_index_topm)
 *   4. run exact softmax attention over only the selected full-size bf16 rows,
 *      read in place from the cache, with a separate index set per KV head, all
 *      heads in one launch (JSSA article, same section, last paragraph).
 *                                                    -> sparse_attn_decode
 *   Extension: the gated linear-attention branch of LISA (aikraft.ru news item,
 *   "LISA architecture").                            -> sparse_attn_linear_gate
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to dense row-major arrays in the
 *   layouts stated per argument, except `shape`, which is a host pointer.
 *   The caller owns every buffer; the library allocates nothing and keeps no
 *   state between calls.
 * - bf16 is IEEE bfloat16 stored as uint16; FP8 is the OCP E4M3 format
 *   ("e4m3fn": bias 7, max 448, NaN codes 0x7F/0xFF, no infinities).
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on `stream`; none synchronises the host (unless the
 *   environment variable SPARSE_ATTN_SYNC=1 is set, a debugging aid that
 *   synchronises after each call and reports asynchronous errors).
 * - Return value: SA_OK (0) or a negative sa_status.  Arguments are checked on
 *   the host before anything is launched; a call that fails a check launches
 *   nothing and changes no memory.  Launch failures return SA_ERR_HIP.
 * - Pointer alignment: 16 bytes for bf16 and FP8 tensors, 4 bytes for int32
 *   and fp32 tensors; a misaligned pointer is SA_ERR_INVALID.
 * - Shape limits: head_dim in {64, 128}; rank in {16, 32}; num_q_heads a
 *   multiple of num_kv_heads with G = num_q_heads / num_kv_heads <= 16;
 *   batch, num_kv_heads >= 1; capacity >= 1.
 * - Results are bitwise deterministic run to run (no floating-point atomics).
 * - Calls that share a workspace must be ordered on one stream.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one attention layer's caches.  B = batch, Hq = num_q_heads,
 * Hkv = num_kv_heads, d = head_dim, r = rank (indexer basis width),
 * Ncap = capacity (rows per (batch row, KV head) in every cache). */
typedef struct sa_shape {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t rank;
  int32_t capacity;
} sa_shape;

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID = -1,     /* bad argument: null/misaligned pointer, bad size */
  SA_ERR_UNSUPPORTED = -2, /* valid but outside the supported shape limits */
  SA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  SA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  SA_ERR_TOO_LARGE = -5    /* the shape needs more scratch than the no-allocation
                              entry point holds (SA_NOALLOC_SCRATCH_BYTES) */
} sa_status;

/* ---------------------------------------------------------------------------
 * sparse_attn_append_kv -- append T tokens per batch row (step 1).
 *
 * JSSA article, "How JSSA preserves token order": each key gets a projection
 * onto its KV head's basis, stored as FP8 beside the bf16 KV cache.
 *
 * pos      [B] int32: first cache row written for batch row b.
 * T        tokens per batch row (T = 0 is a no-op).
 * k_new, v_new [B][Hkv][T][d] bf16.
 * P        [Hkv][d][r] fp32 basis per KV head.
 * k_cache, v_cache [B][Hkv][Ncap][d] bf16 (row pos[b]+t <- token t).
 * kp_cache [B][Hkv][Ncap][r] uint8 FP8 codes:
 *          kp[n][j] = e4m3( sum_i k[i] * P[h][i][j] ), the sum formed in fp64
 *          (8 fused multiply-add chains from +0 over d/8 consecutive i each,
 *          added in order to +0) and rounded once, to nearest-even,
 *          saturating at +-448.
 * Rows pos[b]+t outside [0, Ncap) are skipped (device data is not checked on
 * the host).
 * ------------------------------------------------------------------------- */
int sparse_attn_append_kv(const sa_shape* shape, const int32_t* pos, int32_t T,
                          const void* k_new, const void* v_new, const float* P,
                          void* k_cache, void* v_cache, uint8_t* kp_cache,
                          void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_project_keys -- (re)build the FP8 projected-key cache from rows
 * already in k_cache: rows [n_begin, n_begin + n_count) of every (b, KV head),
 * with the same arithmetic as sparse_attn_append_kv.  Used to fill the
 * indexer cache after a prefill wrote K.  Requires 0 <= n_begin and
 * n_begin + n_count <= Ncap.
 * ------------------------------------------------------------------------- */
int sparse_attn_project_keys(const sa_shape* shape, const void* k_cache,
                             const float* P, int32_t n_begin, int32_t n_count,
                             uint8_t* kp_cache, void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_index_score -- indexer scores of every position (step 2).
 *
 * JSSA article, "How JSSA preserves token order": the queries of one KV head's
 * group are averaged and projected, then every position is scored.
 *
 * q        [B][Hq][d] bf16; query head hq belongs to KV head hq / G.
 * seq_lens [B] int32 valid positions per batch row, or NULL (= n_max);
 *          values are clamped to [0, n_max].
 * n_max    positions scored per (b, KV head); 1 <= n_max <= Ncap.
 * scores   [B][Hkv][n_max] fp32 out:
 *          s[n] = sum_j qt[j] * dec(kp[n][j]) for n < len, -inf otherwise,
 *          where qt = P[h]^T * mean_g q[h*G+g] is formed in fp64 and rounded
 *          to fp32, and each score is accumulated in fp32 as one 16-term fused
 *          multiply-add chain per 16 codes (r = 32: j < 16 and j >= 16, the
 *          two chains then added).
 * ------------------------------------------------------------------------- */
int sparse_attn_index_score(const sa_shape* shape, const void* q, const float* P,
                            const uint8_t* kp_cache, const int32_t* seq_lens,
                            int32_t n_max, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_topm -- exact top-M positions per (b, KV head) (step 3).
 *
 * IndexCache article, "DeepSeek Sparse Attention": keep the k most relevant
 * positions; JSSA article: every KV head (GQA group) selects its own set.
 *
 * scores   [B][Hkv][n_max] fp32 (as written by sparse_attn_index_score; no
 *          NaN among the first len_b of a row), read in place.
 * idx      [B][Hkv][M] int32 out: the positions n < len with the M largest
 *          scores, equal scores ordered by lower position; ascending; when
 *          fewer than M positions are valid, all of them followed by -1.
 * M        1 <= M <= n_max.
 * workspace device buffer of >= sparse_attn_workspace_size(shape, n_max, M)
 *          bytes, 256-byte aligned; scratch for the per-chunk candidates.
 *          Its contents need no initialisation and are not meaningful after
 *          the call.
 * ------------------------------------------------------------------------- */
int sparse_attn_topm(const sa_shape* shape, const float* scores,
                     const int32_t* seq_lens, int32_t n_max, int32_t M,
                     int32_t* idx, void* workspace, size_t ws_bytes,
                     void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_index_topm -- steps 2 and 3 fused: at most three launches,
 * listed under sparse_attn_index_topm_stage; the scores stay on chip, except
 * under SA_PLAN_SCORES, which writes them to the workspace (4 bytes per
 * position) for its merge.  Produces exactly the idx that
 * sparse_attn_index_score followed by sparse_attn_topm produces.
 * Arguments as in those two calls.
 * ------------------------------------------------------------------------- */
int sparse_attn_index_topm(const sa_shape* shape, const void* q, const float* P,
                           const uint8_t* kp_cache, const int32_t* seq_lens,
                           int32_t n_max, int32_t M, int32_t* idx,
                           void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_index_topm_stage -- sparse_attn_index_topm as its three
 * launches, one call each, for callers that time, overlap or schedule them
 * separately.  Same selection and arguments as sparse_attn_index_topm; run
 * the stages in order on one stream with the same shape, n_max, M and
 * workspace, and let nothing else use the workspace in between.
 *
 *   SA_STAGE_BOUND       per (b, KV head): a lower bound on the M-th largest
 *                        score from a sample of the positions (a no-op for
 *                        shapes that use the chunk-exact method below);
 *   SA_STAGE_CANDIDATES  score every position; keep, per position chunk, the
 *                        keys at or above the bound (or the chunk's exact
 *                        top-M, chunk-exact method);
 *   SA_STAGE_MERGE       exact top-M over the kept keys, written to idx (a
 *                        head whose bound turned out too high, or that kept
 *                        more keys than the merge holds, is selected again
 *                        exactly from the FP8 cache).
 * idx is only written by SA_STAGE_MERGE (and may be NULL for the others).
 * Where one workgroup per unit serves the shape (sparse_attn_selection_plan
 * gives SA_PLAN_UNIT), SA_STAGE_CANDIDATES is the whole selection in one
 * launch (bound, filter and merge: it writes idx) and the other two stages
 * launch nothing.  Where every position is scored (SA_PLAN_SCORES),
 * SA_STAGE_BOUND writes every position's score to the workspace,
 * SA_STAGE_CANDIDATES launches nothing and SA_STAGE_MERGE selects exactly
 * over the scores.
 * Returns SA_ERR_INVALID for an unknown stage.
 * ------------------------------------------------------------------------- */
enum sa_stage { SA_STAGE_BOUND = 1, SA_STAGE_CANDIDATES = 2, SA_STAGE_MERGE = 3 };

int sparse_attn_index_topm_stage(const sa_shape* shape, int32_t stage, const void* q,
                                 const float* P, const uint8_t* kp_cache,
                                 const int32_t* seq_lens, int32_t n_max, int32_t M,
                                 int32_t* idx, void* workspace, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_decode -- gather-free sparse attention (step 4).
 *
 * JSSA article, "How JSSA preserves token order": final attention uses the
 * original full-size keys and values of the selected positions, read directly
 * from the cache without an intermediate buffer, with separate index sets per
 * head in a single launch.
 *
 * q        [B][Hq][d] bf16.
 * k_cache, v_cache [B][Hkv][Ncap][d] bf16.
 * idx      [B][Hkv][M] int32; entries outside [0, Ncap) are padding and
 *          skipped (duplicates count once per occurrence).
 * softmax_scale  multiplies q.k (normally 1/sqrt(d)); must be finite.
 * out      [B][Hq][d] bf16: softmax(scale * q.K[idx]) . V[idx], rounded to
 *          nearest-even; all-zero when no entry is valid.
 * lse      [B][Hq] fp32 natural-log log-sum-exp of the scaled logits, or NULL;
 *          -inf when no entry is valid.
 * workspace as for sparse_attn_topm.
 * ------------------------------------------------------------------------- */
int sparse_attn_decode(const sa_shape* shape, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* idx, int32_t M,
                       float softmax_scale, void* out, float* lse,
                       void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_decode_step -- one whole decode step of one layer: exactly
 * sparse_attn_append_kv (T new tokens), then sparse_attn_index_topm, then
 * sparse_attn_decode, with the same arguments, but with fewer launches (the
 * append shares a launch with the bound stage of the selection).
 *
 * JSSA article, "How JSSA preserves token order": append with projection,
 * indexer scoring and top-M selection per KV head, then gather-free
 * attention over the selected rows.
 *
 * idx is written (the step's selection, e.g. for IndexCache reuse by later
 * layers), then out and lse as sparse_attn_decode writes them.  Arguments
 * and checks are those of the three calls; the workspace is sized by
 * sparse_attn_workspace_size(shape, n_max, M).
 * ------------------------------------------------------------------------- */
int sparse_attn_decode_step(const sa_shape* shape, const int32_t* pos, int32_t T,
                            const void* k_new, const void* v_new, const void* q,
                            const float* P, void* k_cache, void* v_cache,
                            uint8_t* kp_cache, const int32_t* seq_lens, int32_t n_max,
                            int32_t M, float softmax_scale, int32_t* idx, void* out,
                            float* lse, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_decode_step_noalloc -- sparse_attn_decode_step for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments and results (the
 * same kernels), but no workspace argument: the workspace is a static device
 * array of SA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU,
 * held from the library's load until the process ends.  The call allocates
 * nothing; its first call on a device (that device current in the calling
 * thread, the device the stream and buffers belong to) looks the array's
 * address up once.
 * Limit: shapes with sparse_attn_workspace_size(shape, n_max, M) >
 * SA_NOALLOC_SCRATCH_BYTES return SA_ERR_TOO_LARGE and launch nothing.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (they need no clearing: the step initialises what it reads), so
 * calls that overlap on one GPU (other streams, other threads) race; order
 * them on one stream.
 * ------------------------------------------------------------------------- */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int sparse_attn_decode_step_noalloc(const sa_shape* shape, const int32_t* pos, int32_t T,
                                    const void* k_new, const void* v_new, const void* q,
                                    const float* P, void* k_cache, void* v_cache,
                                    uint8_t* kp_cache, const int32_t* seq_lens, int32_t n_max,
                                    int32_t M, float softmax_scale, int32_t* idx, void* out,
                                    float* lse, void* stream);

/* sparse_attn_decode_step_stage -- the launches of sparse_attn_decode_step,
 * one call each (for timing or scheduling): SA_STEP_APPEND_BOUND, then
 * SA_STEP_CANDIDATES, then either SA_STEP_SELECT_ATTEND (writes idx, out,
 * lse; what sparse_attn_decode_step itself runs) or SA_STEP_MERGE (writes
 * idx) followed by SA_STEP_ATTEND (writes out, lse).  Both endings give the
 * same bits.  SA_STEP_SELECT_ATTEND is one launch (plus the split merge when
 * the attention is split) when the filter path serves the shape and
 * G * head_dim <= 1024, else the two stages' launches.  Where one workgroup
 * per unit serves the shape (sparse_attn_selection_plan gives SA_PLAN_UNIT),
 * SA_STEP_APPEND_BOUND is the whole step in one launch (append, bound,
 * filter, merge and attention: it writes the caches, idx, out and lse) and
 * the later stages launch nothing.  Where every position is scored
 * (SA_PLAN_SCORES), SA_STEP_APPEND_BOUND appends and scores every position,
 * SA_STEP_CANDIDATES launches nothing, and the merge selects over the
 * scores.  Run the stages in order on one stream with identical arguments.
 * Returns SA_ERR_INVALID for an unknown stage. */
enum sa_step_stage {
  SA_STEP_APPEND_BOUND = 1,
  SA_STEP_CANDIDATES = 2,
  SA_STEP_MERGE = 3,
  SA_STEP_ATTEND = 4,
  SA_STEP_SELECT_ATTEND = 5
};

int sparse_attn_decode_step_stage(const sa_shape* shape, int32_t stage, const int32_t* pos,
                                  int32_t T, const void* k_new, const void* v_new,
                                  const void* q, const float* P, void* k_cache,
                                  void* v_cache, uint8_t* kp_cache, const int32_t* seq_lens,
                                  int32_t n_max, int32_t M, float softmax_scale, int32_t* idx,
                                  void* out, float* lse, void* workspace, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * sparse_attn_linear_gate -- LISA-style gated linear branch.
 *
 * LISA news items (aikraft.ru "LISA architecture"; opennieuws.be "Hybrid
 * architecture for efficiency"): a linear-attention branch with linear-time
 * memory is merged with the sparse branch by a gate.  Feature map
 * phi(x) = x + 1 (x > 0), exp(x) (x <= 0).
 *
 * q        [B][Hq][d] bf16; k_new, v_new [B][Hkv][d] bf16 (the new token).
 * S        [B][Hkv][d][d] fp32 in/out, S[i][j] = sum phi(k)[i] * v[j].
 * z        [B][Hkv][d] fp32 in/out, z = sum phi(k).
 * update_state != 0: first S += phi(k_new) v_new^T, z += phi(k_new).
 * w_gate   [Hq][d] fp32; g = 1 / (1 + exp(-(w[hq] . q[hq]))).
 * o_sparse [B][Hq][d] bf16 (output of sparse_attn_decode).
 * out      [B][Hq][d] bf16: g * o_sparse + (1 - g) * (phi(q)^T S) / (phi(q)^T z).
 *          With an empty state (phi(q)^T z == 0, i.e. z == 0: no token was ever
 *          added) the linear read-out is 0 and out = g * o_sparse.
 * ------------------------------------------------------------------------- */
int sparse_attn_linear_gate(const sa_shape* shape, const void* q,
                            const void* k_new, const void* v_new, float* S,
                            float* z, const float* w_gate, const void* o_sparse,
                            void* out, int32_t update_state, void* stream);

/* ---------------------------------------------------------------------------
 * Comparison baselines (not on the decode path).  The JSSA article (rit.work
 * blog) measures its decoding throughput against full attention (opening
 * paragraph: 6.43x at 128K context and a 2048-token budget on B200) and
 * reports, in "Why token selection is not enough", that with the usual
 * gather-then-attend scheme the copy into a contiguous buffer took more than
 * half of the remaining sparse-attention time at large batch.  These two
 * calls let both comparisons be measured on this GPU.
 *
 * sparse_attn_dense_decode -- exact attention of every query head over ALL
 * valid rows n < len_b of its KV head (len_b = seq_lens[b] clamped to
 * [0, n_max], or n_max when seq_lens is NULL), read as consecutive rows of
 * the bf16 cache.  q, k_cache, v_cache, out, lse and softmax_scale as in
 * sparse_attn_decode (len_b = 0 gives out = 0 and lse = -inf).  Workspace:
 * sparse_attn_dense_workspace_size(shape, n_max) bytes, 256-byte aligned.
 * Returns SA_ERR_INVALID for bad pointers or n_max outside [1, capacity],
 * SA_ERR_WORKSPACE when the workspace is missing or too small.
 * ------------------------------------------------------------------------- */
int sparse_attn_dense_decode(const sa_shape* shape, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* seq_lens, int32_t n_max,
                             float softmax_scale, void* out, float* lse, void* workspace,
                             size_t ws_bytes, void* stream);
size_t sparse_attn_dense_workspace_size(const sa_shape* shape, int32_t n_max);

/* sparse_attn_gather_kv -- the copy of gather-then-attend: for every unit u
 * and j < M, k_out[u][j] = k_cache[u][idx[u][j]] and v_out likewise (d bf16
 * values per row), zero rows where idx[u][j] is -1 (or outside the cache).
 * idx [B][Hkv][M] int32 (as sparse_attn_topm writes it); k_out, v_out
 * [B][Hkv][M][d] bf16, caller-owned, 16-byte aligned.  Attending over the
 * gathered rows is sparse_attn_dense_decode on a shape of capacity M with
 * seq_lens min(len_b, M) and n_max = M.  Returns SA_ERR_INVALID for bad
 * pointers or M outside [1, capacity]. */
int sparse_attn_gather_kv(const sa_shape* shape, const int32_t* idx, int32_t M,
                          const void* k_cache, const void* v_cache, void* k_out, void* v_out,
                          void* stream);

/* sparse_attn_stream_read -- measurement helper, not part of the method:
 * reads the `bytes` bytes at `buf` once, front to back, with the fastest
 * streaming pattern measured on this GPU (512-thread workgroups of 4 MiB
 * each, every wave load 1 KB of contiguous bytes, four 16-byte loads per
 * thread in flight, non-temporal), so that a caller can time the device's
 * streaming-read rate beside the kernels' (the practical ceiling under the
 * nominal HBM peak).  buf: 16-byte aligned device memory; bytes: a positive
 * multiple of 4 MiB; sink: one device uint32 that a value derived from the
 * data may be written to (it keeps the loads from being optimised away and
 * means nothing).  Returns SA_ERR_INVALID for anything else. */
int sparse_attn_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* sparse_attn_row_read -- measurement helper, not part of the method: reads
 * the rows the gather-free attention reads -- for every unit u and j < M, the
 * d bf16 values of k_cache[u][idx[u][j]] and of v_cache[u][idx[u][j]]
 * (entries outside [0, Ncap) skipped) -- once each, non-temporal, one
 * 16-wave workgroup per unit, and computes nothing: the random-row floor the
 * attention is measured against.  mode 0: into registers, with the
 * attention's lane layout; mode 1: straight into LDS (buffer loads to LDS,
 * whole rows per wave load).  idx, k_cache, v_cache as for
 * sparse_attn_decode; sink as for sparse_attn_stream_read.  Returns
 * SA_ERR_INVALID for a bad pointer, M < 1 or another mode. */
int sparse_attn_row_read(const sa_shape* shape, const int32_t* idx, int32_t M,
                         const void* k_cache, const void* v_cache, int32_t mode, uint32_t* sink,
                         void* stream);

/* sparse_attn_selection_fallbacks -- diagnostic, not part of the method: of
 * the (b, KV head) units of the last selection that ran in `workspace` with
 * this shape, n_max and M (sparse_attn_topm, sparse_attn_index_topm(_stage),
 * sparse_attn_decode_step(_stage)), how many were selected by the exact
 * streaming pass over the unit's codes or scores (taken when the sampled
 * bound kept fewer than M positions, or more than the merge holds) rather
 * than from the kept candidates.  Either way the selection is exact; the
 * count shows which path served a shape.  count: one device int32, written
 * on `stream` (-1 when the shape uses the chunk-exact method, which has no
 * such fallback).  Returns SA_ERR_INVALID for a bad pointer, n_max or M,
 * SA_ERR_WORKSPACE when the workspace is missing or too small. */
int sparse_attn_selection_fallbacks(const sa_shape* shape, int32_t n_max, int32_t M,
                                    const void* workspace, size_t ws_bytes, int32_t* count,
                                    void* stream);

/* sparse_attn_selection_plan -- diagnostic, host only: which method the fused
 * selection (sparse_attn_index_topm, sparse_attn_decode_step) uses for this
 * shape, n_max and M on the calling thread's current device:
 *   SA_PLAN_CHUNK_EXACT (0)  chunks hand over their exact top-M, then a merge
 *                            launch (n_max > 2^19, M > 6144 or M = n_max);
 *   SA_PLAN_FILTER (1)       sampled bound, filtering chunks, merge (and, in
 *                            the decode step, attention in the merge launch);
 *   SA_PLAN_UNIT (2)         one workgroup per (b, KV head) unit appends,
 *                            bounds, streams, merges and attends in one launch
 *                            (when the units fill whole rounds of the device's
 *                            compute units, units >= 256, G d <= 1024, M <= 2048);
 *   SA_PLAN_SCORES (3)       every position is scored and written out (fp32,
 *                            4 bytes per position of workspace), then an exact
 *                            merge over all of a unit's scores (and, in the
 *                            decode step, attention in the merge launch): no
 *                            bound, no filter (n_max <= 16384, where the unit
 *                            plan does not apply).
 * Every plan gives the same idx, out and lse bits.  The environment variables
 * SPARSE_ATTN_UNIT_WG=0 and SPARSE_ATTN_SCORES_PLAN=0 turn SA_PLAN_UNIT and
 * SA_PLAN_SCORES off (testing aids).  Returns the plan, or SA_ERR_INVALID /
 * SA_ERR_UNSUPPORTED for arguments the selection rejects. */
enum sa_plan {
  SA_PLAN_CHUNK_EXACT = 0,
  SA_PLAN_FILTER = 1,
  SA_PLAN_UNIT = 2,
  SA_PLAN_SCORES = 3
};

int sparse_attn_selection_plan(const sa_shape* shape, int32_t n_max, int32_t M);

/* Bytes of workspace that sparse_attn_topm, sparse_attn_index_topm(_stage),
 * sparse_attn_decode and sparse_attn_decode_step(_stage) need for this shape,
 * n_max and M (host only, pure).
 * Returns 0 when the arguments are invalid. */
size_t sparse_attn_workspace_size(const sa_shape* shape, int32_t n_max, int32_t M);

/* Static description of a status code (never NULL). */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
