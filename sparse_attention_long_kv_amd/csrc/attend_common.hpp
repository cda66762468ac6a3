// Gather-free sparse attention over selected rows of the bf16 KV cache: the
// per-workgroup machinery shared by the attention kernel and the fused
// select-and-attend kernel (so both form the same bits).
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
// workgroups ("split-K"); each wave of a workgroup takes tiles of 16 selected
// rows, tile t going to wave t mod W.  Both products of a tile run on the
// matrix cores:
//
//  * logits: one 16x16x32 bf16 MFMA per 32 dims, A = the 16 K rows (each
//    lane loads 16 bytes of one row straight from the cache), B = the GQA
//    group's queries (heads as columns, zero past G).  Lane (q4, n) receives
//    the logits of head n for rows 4v + q4, v = 0..3, because the lane that
//    supplies A row m loads tile row 4(m % 4) + m / 4.
//  * values: 16x16x4 fp32 MFMAs, A = the softmax weights exactly as the logit
//    product left them (head n, row 4v + q4), B = fp32 V rows (lane (q4, n)
//    loads d/16 dims, n*d/16 onward, of row 4v + q4; one MFMA per dim).  The
//    output tile holds heads as rows, so lane (q4, n) accumulates heads
//    4 q4 + v for dims n*d/16 + j.
//
// The online softmax runs in base 2 per head; each tile's maximum is shared
// by the four lanes of a head with two cross-lane steps, and the accumulated
// outputs are rescaled only when some head's running maximum moves.  States
// merge across waves in LDS and across the S workgroups with the log-sum-exp
// rule  m = max m_s,  l = sum l_s 2^(m_s - m),  o = sum o_s 2^(m_s - m) / l,
// the cross-workgroup merge being a small second launch (none when S = 1).
#pragma once

#include "device_common.hpp"

namespace sa {

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  int M, Ncap, Hq, Hkv, G, S, rps;
  float qscale;        // softmax_scale * log2(e)
  uint16_t* out;
  float* lse;
  float* pm;           // [units][S][G] partial states when S > 1
  float* pl;
  float* po;           // [units][S][G][d]
  const int32_t* lens; // dense attention: valid rows per batch row (null = n_max)
  int n_max;
};

typedef __bf16 sa_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sa_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int sa_u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxHeads = 16;        // MFMA tile width: G <= 16
constexpr int kAttendWaves = 16;     // waves per attention workgroup (4 per SIMD)
constexpr int kAttendThreads = kAttendWaves * kWave;
constexpr int kDecodeIdxTile = 2048; // selected rows staged in LDS at a time (multiple of 16 W)
constexpr uint32_t kOffNone = 0x80000000u;   // past any unit's range: loads return zero

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, l) merge weights of two base-2 states; -inf states weigh 0.
__device__ __forceinline__ float merge_scale(float m_part, float m_tot) {
  return m_part == -__builtin_inff() ? 0.0f : fast_exp2(m_part - m_tot);
}

// Row loads of the attention carry the non-temporal cache policy: each
// selected row is read once, so keeping it in the caches only displaces other
// lines (measured at 128K: select + attend 66 -> 63 us).
constexpr int kRowLoadPolicy = 2;      // nt

__device__ __forceinline__ uint4 row_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const sa_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kRowLoadPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One lane's share of a V row: 8 bf16 (d = 128) or 4 bf16 (d = 64).
template <int D> struct VRaw { using type = uint4; };
template <> struct VRaw<64> { using type = sa_u32x2; };

template <int D>
__device__ __forceinline__ typename VRaw<D>::type load_v_raw(__amdgpu_buffer_rsrc_t r,
                                                             uint32_t off) {
  if constexpr (D == 128) return row_load16(r, off);
  else return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kRowLoadPolicy);
}

template <int D>
__device__ __forceinline__ void v_raw_to_f32(const typename VRaw<D>::type& x, float* f) {
  if constexpr (D == 128) {
    bf16x8_to_f32(x, f);
  } else {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
  }
}

// Registers of one loaded 16-row tile.
template <int D>
struct TileRaw {
  uint4 k[D / 32];
  typename VRaw<D>::type v[4];
  int nr[4];
};

// One wave's share of a (unit, split) attention: W waves per workgroup, one
// 16-row tile in flight per wave.  Call init, then rows() once per staged
// run of selected rows (runs of a multiple of 16 W rows keep the tile ->
// wave assignment of one long run), then finish with the whole workgroup.
template <int D, int W>
struct AttendWave {
  static constexpr int KS = D / 32;    // logit MFMAs per tile
  static constexpr int DL = D / 16;    // value dims per lane (one MFMA each)
  int G, b, h, w, lane, q4, n16, tk;
  bool head_ok;
  uint32_t koff, voff;
  __amdgpu_buffer_rsrc_t rk, rv;
  sa_bf16x8 qb[KS];                    // B operand: head n16's dims 32i + 8 q4 .. + 8
  float m_run, l_run;
  sa_f32x4 o[DL];

  __device__ __forceinline__ void init(const DecodeArgs& a, int u) {
    G = a.G;
    b = u / a.Hkv;
    h = u % a.Hkv;
    w = threadIdx.x / kWave;
    lane = lane_id();
    q4 = lane >> 4;
    n16 = lane & 15;
    head_ok = n16 < G;
    const uint16_t* qp =
        a.q + ((size_t)b * a.Hq + (size_t)h * G + min(n16, G - 1)) * D + 8 * q4;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      uint4 raw = *reinterpret_cast<const uint4*>(qp + 32 * i);
      if (!head_ok) raw = make_uint4(0u, 0u, 0u, 0u);
      qb[i] = __builtin_bit_cast(sa_bf16x8, raw);
    }
    m_run = -__builtin_inff();
    l_run = 0.0f;
#pragma unroll
    for (int j = 0; j < DL; ++j) o[j] = sa_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t unit_bytes = (uint32_t)a.Ncap * D * 2;
    rk = make_rsrc(a.k + (size_t)u * a.Ncap * D, unit_bytes);
    rv = make_rsrc(a.v + (size_t)u * a.Ncap * D, unit_bytes);
    tk = 4 * (n16 & 3) + (n16 >> 2);          // tile row whose K this lane loads
    koff = (uint32_t)(8 * q4) * 2;            // bytes of dims 8 q4
    voff = (uint32_t)(DL * n16) * 2;          // bytes of dims DL n16
  }

  // row loads of one 16-row tile: run row j is cache row row_of(j), rows at
  // or past cnt are none
  template <class RowOf>
  __device__ __forceinline__ void issue(const DecodeArgs& a, RowOf row_of, int cnt, int tt,
                                        TileRaw<D>& t) const {
    const int rb = tt * 16;
    const int nk = rb + tk < cnt ? row_of(rb + tk) : -1;
#pragma unroll
    for (int v = 0; v < 4; ++v) t.nr[v] = rb + 4 * v + q4 < cnt ? row_of(rb + 4 * v + q4) : -1;
    const uint32_t kb =
        (unsigned)nk < (unsigned)a.Ncap ? (uint32_t)nk * (D * 2) + koff : kOffNone;
#pragma unroll
    for (int i = 0; i < KS; ++i) t.k[i] = row_load16(rk, kb + 64u * i);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t vb =
          (unsigned)t.nr[v] < (unsigned)a.Ncap ? (uint32_t)t.nr[v] * (D * 2) + voff : kOffNone;
      t.v[v] = load_v_raw<D>(rv, vb);
    }
  }

  // logits, online softmax and value products of one loaded tile
  __device__ __forceinline__ void consume(const DecodeArgs& a, const TileRaw<D>& t) {
    sa_f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < KS; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sa_bf16x8, t.k[i]), qb[i], c,
                                                  0, 0, 0);
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      s[v] = (head_ok && (unsigned)t.nr[v] < (unsigned)a.Ncap) ? c[v] * a.qscale
                                                                : -__builtin_inff();
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    if (ballot(m_new != m_run)) {                     // wave-uniform
      const float alpha = merge_scale(m_run, m_new);
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) al[v] = __shfl(alpha, 4 * q4 + v, kWave);
#pragma unroll
      for (int j = 0; j < DL; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[j][v] *= al[v];
      m_run = m_new;
    }
    const float mref = m_run == -__builtin_inff() ? 0.0f : m_run;
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = fast_exp2(s[v] - mref);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float vf[DL];
      v_raw_to_f32<D>(t.v[v], vf);
#pragma unroll
      for (int j = 0; j < DL; ++j)
        o[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[v], vf[j], o[j], 0, 0, 0);
    }
  }

  // the cnt selected rows sidx[0, cnt) (LDS); trip counts are wave-uniform
  __device__ __forceinline__ void rows(const DecodeArgs& a, const int32_t* sidx, int cnt) {
    const int ntile = (cnt + 15) >> 4;
    for (int tt = w; tt < ntile; tt += W) {
      TileRaw<D> t;
      issue(a, [&](int j) { return sidx[j]; }, cnt, tt, t);
      consume(a, t);
    }
  }

  // the cnt consecutive cache rows r0, r0 + 1, ... (dense attention)
  __device__ __forceinline__ void rows_dense(const DecodeArgs& a, int r0, int cnt) {
    const int ntile = (cnt + 15) >> 4;
    for (int tt = w; tt < ntile; tt += W) {
      TileRaw<D> t;
      issue(a, [&](int j) { return r0 + j; }, cnt, tt, t);
      consume(a, t);
    }
  }

  // Merge the waves' states (sm, sl: [W][kMaxHeads]; so: [W][G][D] floats of
  // LDS) and write out/lse (S == 1) or this split's partial state.
  __device__ __forceinline__ void finish(const DecodeArgs& a, int u, int split,
                                         float (*sm)[kMaxHeads], float (*sl)[kMaxHeads],
                                         float* so) {
    constexpr int NT = W * kWave;
    l_run += __shfl_xor(l_run, 16, kWave);
    l_run += __shfl_xor(l_run, 32, kWave);
    if (lane < kMaxHeads) {
      sm[w][lane] = m_run;
      sl[w][lane] = l_run;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int hd = 4 * q4 + v;
      if (hd < G) {
#pragma unroll
        for (int j = 0; j < DL; ++j) so[((size_t)w * G + hd) * D + DL * n16 + j] = o[j][v];
      }
    }
    __syncthreads();
    // thread -> (g, dim)
    const size_t part0 = ((size_t)u * a.S + split) * G;
    for (int t = threadIdx.x; t < G * D; t += NT) {
      const int g = t / D, dd = t % D;
      float mt = sm[0][g];
#pragma unroll
      for (int ww = 1; ww < W; ++ww) mt = fmaxf(mt, sm[ww][g]);
      float lt = 0.0f, ot = 0.0f;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const float sc = merge_scale(sm[ww][g], mt);
        lt += sl[ww][g] * sc;
        ot += so[((size_t)ww * G + g) * D + dd] * sc;
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
};

}  // namespace sa
