"""Comparison helpers for the GPU parity tests (test infrastructure).

The tolerances come from the correctness contract of the decode step:
* top-M index sets equal the oracle's except for swaps among positions whose
  scores lie within 1e-5 (relative) of the M-th score;
* attention outputs within 2e-2 absolute + 1e-2 relative (bf16 inputs, fp32
  accumulation).
Score tolerance (index_score) is derived from the arithmetic: qt is rounded
once to fp32 (relative 2^-24) and each score is at most 17 fp32 roundings deep
over terms bounded by sum_j |qt_j dec(c_j)|, so
|s_gpu - s_exact| <= 18 * 2^-24 * sum_j |qt_j dec(c_j)| ~ 1.07e-6 * that sum;
the tests use 2e-6 times the sum.
"""

import numpy as np
import torch

import oracle

SCORE_REL = 2e-6
BAND_REL = 1e-5
ATT_ABS = 2e-2
ATT_REL = 1e-2


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def oracle_kp(K64, P64):
    """oracle FP8 projected keys for K [B, Hkv, N, d] (float64), P [Hkv, d, r]."""
    B, H, N, _ = K64.shape
    r = P64.shape[2]
    out = np.zeros((B, H, N, r), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            out[b, h] = oracle.project_keys(K64[b, h], P64[h])
    return out


def kp_codes_match(gpu, orc, K64, P64):
    """GPU codes equal the oracle's except where the fp64 pre-image lies within
    1e-5 * sum_i |K_i P_ij| of an FP8 rounding midpoint (then either neighbour)."""
    if np.array_equal(gpu, orc):
        return True, 0
    bad = np.argwhere(gpu != orc)
    table = oracle.decode_table()
    for idx in bad:
        b, h, n, j = idx
        x = float(K64[b, h, n] @ P64[h][:, j])
        mag = float(np.abs(K64[b, h, n]) @ np.abs(P64[h][:, j]))
        lo, hi = sorted((table[gpu[b, h, n, j]], table[orc[b, h, n, j]]))
        if not (np.isfinite(lo) and np.isfinite(hi)):
            return False, len(bad)
        mid = (lo + hi) / 2
        if abs(x - mid) > 1e-5 * mag:
            return False, len(bad)
    return True, len(bad)


def score_tolerance(q_tilde, kp_unit):
    return SCORE_REL * (np.abs(oracle.fp8_decode(kp_unit)) @ np.abs(q_tilde)) + 1e-30


def check_topm_unit(idx_gpu, scores_exact, M, L):
    """Assert the GPU index set of one unit satisfies the contract.

    idx_gpu: [M] int32 from the GPU; scores_exact: oracle fp64 scores [>= L];
    L: number of valid positions.  Returns the number of band swaps.
    """
    idx_gpu = np.asarray(idx_gpu)
    k = min(M, L)
    sel = idx_gpu[:k]
    assert np.all(idx_gpu[k:] == -1), "padding must be -1"
    assert np.all(sel >= 0) and np.all(sel < L), "indices out of range"
    assert np.all(np.diff(sel) > 0), "indices must be ascending and unique"
    want = oracle.top_m(scores_exact[:L], M)[:k]
    if L <= M:
        assert np.array_equal(sel, want)
        return 0
    s = scores_exact[:L]
    sM = np.sort(s)[::-1][M - 1]
    band = np.abs(s - sM) <= BAND_REL * abs(sM)
    g = set(sel.tolist())
    o = set(want.tolist())
    outside_g = {n for n in g if not band[n]}
    outside_o = {n for n in o if not band[n]}
    assert outside_g == outside_o, "sets differ outside the band: %s vs %s" % (
        sorted(outside_g - outside_o)[:10], sorted(outside_o - outside_g)[:10])
    return len(g - o)


def check_attention(out_gpu, out_orc, what=""):
    out_gpu = np.asarray(out_gpu, dtype=np.float64)
    err = np.abs(out_gpu - out_orc)
    lim = ATT_ABS + ATT_REL * np.abs(out_orc)
    assert np.all(err <= lim), "%s max excess %.3g at %s" % (
        what, float((err - lim).max()), np.unravel_index(np.argmax(err - lim), err.shape))
