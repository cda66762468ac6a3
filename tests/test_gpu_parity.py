"""GPU parity: every C-ABI entry point against the fp64 oracle.

Inputs are seeded and synthetic (``workloads``); every input the oracle sees is
either generated or computed by the oracle itself (the FP8 projected-key cache
handed to the scoring tests is the oracle's, never the GPU's).  Sizes span
several chunks/tiles and ragged tails; edge cases cover empty rows, M = 1,
M = N, ties and multi-tile merges.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_kv_amd as sa
from workloads import WORKLOADS, make_decode_inputs, orthonormal_basis, scaled, default_scale
from _helpers import (f64, oracle_kp, kp_codes_match, score_tolerance, check_topm_unit,
                      check_attention, plant_miss_bound)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sa.load()
    yield
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(x, dtype=None):
    t = torch.as_tensor(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def _shape_of(B, Hq, Hkv, d, r, Ncap):
    return sa.make_shape(B, Hq, Hkv, d, r, Ncap)


def _fallbacks(sh, n_max, M, ws):
    """Units of the last selection in ws that took the exact streaming pass
    (-1: the shape uses the chunk-exact method)."""
    cnt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    sa.sparse_attn_selection_fallbacks(sh, n_max, M, ws, cnt)
    return int(cnt.item())


def _use_plan(monkeypatch, plan):
    """plan "filter": keep the sampled-bound filter plan where the plan that
    scores every position would serve the shape (both give the same bits)."""
    if plan == "filter":
        monkeypatch.setenv("SPARSE_ATTN_SCORES_PLAN", "0")


def _scores_shape(n_max, M):
    """Whether the plan that scores every position serves a selection of
    these sizes (on the chunked plans' shapes)."""
    return n_max <= 16384 and M <= 6144 and M < n_max


def _rand_inputs(B, Hq, Hkv, d, r, N, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    K = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    V = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    P = torch.from_numpy(np.stack([orthonormal_basis(d, r, seed * 31 + h)
                                   for h in range(Hkv)]).astype(np.float32))
    return q, K, V, P


# ------------------------------------------------------------------ FP8 decode

def test_fp8_decode_of_every_code_via_scores():
    """score[n] = dec(code n) exactly when qt = e_0 (G = 1, P = identity)."""
    _say("case: fp8 decode table via index_score")
    d, r, N = 64, 16, 256
    sh = _shape_of(1, 1, 1, d, r, N)
    q = torch.zeros(1, 1, d, dtype=torch.bfloat16)
    q[0, 0, 0] = 1.0
    P = torch.zeros(1, d, r, dtype=torch.float32)
    P[0, :r, :r] = torch.eye(r)
    kp = torch.zeros(1, 1, N, r, dtype=torch.uint8)
    kp[0, 0, :, 0] = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    scores = torch.empty(1, 1, N, dtype=torch.float32, device="cuda")
    sa.sparse_attn_index_score(sh, _dev(q), _dev(P), _dev(kp), None, N, scores)
    got = scores.cpu().double().numpy()[0, 0]
    want = oracle.decode_table()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------------------ append / project

@pytest.mark.parametrize("d,r", [(128, 32), (64, 16), (128, 16), (64, 32)])
def test_append_kv_matches_oracle(d, r):
    _say("case: append d=%d r=%d" % (d, r))
    B, Hq, Hkv, Ncap, T = 2, 8, 2, 64, 5
    sh = _shape_of(B, Hq, Hkv, d, r, Ncap)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, Ncap, seed=d + r)
    g = torch.Generator().manual_seed(7)
    kn = (3 * torch.randn(B, Hkv, T, d, generator=g)).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([3, 61], dtype=torch.int32)       # second row: 3 of 5 fit
    kp0 = torch.full((B, Hkv, Ncap, r), 0x11, dtype=torch.uint8)
    Kd, Vd, kpd = _dev(K), _dev(V), _dev(kp0)
    sa.sparse_attn_append_kv(sh, _dev(pos), _dev(kn), _dev(vn), _dev(P), Kd, Vd, kpd)
    K2, V2, kp2 = oracle.append_kv(f64(K), f64(V), kp0.numpy(), pos.numpy(), f64(kn), f64(vn),
                                   P.double().numpy())
    assert np.array_equal(f64(Kd), K2) and np.array_equal(f64(Vd), V2)
    ok, nbad = kp_codes_match(kpd.cpu().numpy(), kp2, K2, P.double().numpy())
    assert ok, "projected-key codes differ outside the rounding-midpoint band (%d)" % nbad


def test_project_keys_matches_oracle():
    _say("case: project_keys bulk")
    B, Hq, Hkv, d, r, Ncap = 2, 4, 2, 128, 32, 3000
    sh = _shape_of(B, Hq, Hkv, d, r, Ncap)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, Ncap, seed=5)
    kpd = torch.zeros(B, Hkv, Ncap, r, dtype=torch.uint8, device="cuda")
    sa.sparse_attn_project_keys(sh, _dev(K), _dev(P), 37, 2900, kpd)
    want = oracle_kp(f64(K), P.double().numpy())
    got = kpd.cpu().numpy()
    assert np.all(got[:, :, :37] == 0) and np.all(got[:, :, 2937:] == 0)
    ok, nbad = kp_codes_match(got[:, :, 37:2937], want[:, :, 37:2937], f64(K)[:, :, 37:2937],
                              P.double().numpy())
    assert ok, nbad


# ------------------------------------------------------------------ scores

@pytest.mark.parametrize("case", ["tiny", "gqa7"])
def test_index_score_matches_oracle(case):
    _say("case: index_score", case)
    if case == "tiny":
        B, Hq, Hkv, d, r, N, lens = 1, 4, 1, 64, 16, 1024, [1000]
    else:
        B, Hq, Hkv, d, r, N, lens = 2, 14, 2, 128, 32, 9000, [9000, 1234]
    n_max = N - 5
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=11)
    P64 = P.double().numpy()
    kp = oracle_kp(f64(K), P64)
    scores = torch.empty(B, Hkv, n_max, dtype=torch.float32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32)
    sa.sparse_attn_index_score(sh, _dev(q), _dev(P), _dev(kp), _dev(sl), n_max, scores)
    got = scores.cpu().double().numpy()
    G = Hq // Hkv
    for b in range(B):
        L = min(lens[b], n_max)
        for h in range(Hkv):
            qt = oracle.indexer_query(f64(q)[b, h * G:(h + 1) * G], P64[h])
            want = oracle.index_scores(qt, kp[b, h, :L])
            tol = score_tolerance(qt, kp[b, h, :L])
            assert np.all(np.abs(got[b, h, :L] - want) <= tol)
            assert np.all(np.isneginf(got[b, h, L:]))


# ------------------------------------------------------------------ top-M

TOPM_CASES = {
    # name: (B, Hq, Hkv, d, r, N(cap), n_max, seq_lens, M)
    "tiny": (1, 4, 1, 64, 16, 1024, 1024, None, 64),
    "ragged": (3, 8, 2, 128, 32, 20000, 19997, [19997, 300, 0], 512),
    "multitile": (1, 2, 1, 128, 32, 65613, 65613, None, 256),
    "m_equals_n": (2, 4, 2, 64, 32, 700, 700, None, 700),
    "m_one": (2, 4, 2, 64, 16, 5000, 5000, [5000, 17], 1),
    "many_chunks": (2, 28, 4, 128, 32, 16384, 16384, [16384, 9000], 2048),
    # M a quarter of N: the sampled bound is a negative score, and the filter
    # chunks' last load batch reaches past their rows (positions of the next
    # chunk, loaded as zero) -- none of those may be kept
    "low_bound": (1, 4, 1, 128, 32, 16384, 16384, None, 4096),
    "low_bound_r16": (2, 8, 2, 64, 16, 12288, 12288, [12288, 10000], 3000),
    # the limits of the filter path (n_max <= 2^19, M <= 6144) and one past
    # each, where the fused selection takes the chunk-exact path instead
    "filter_max_n": (1, 4, 1, 128, 32, 524288, 524288, None, 2048),
    "past_filter_n": (1, 4, 1, 64, 16, 600000, 600000, None, 2048),
    "filter_max_m": (1, 8, 2, 128, 32, 65536, 65536, None, 6144),
    "past_filter_m": (1, 8, 2, 128, 32, 65536, 65536, None, 6145),
}


def _topm_case(name, seed=3):
    B, Hq, Hkv, d, r, N, n_max, lens, M = TOPM_CASES[name]
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=seed)
    G = Hq // Hkv
    # plant rows aligned with the group-mean query, as in the workloads
    qbar = f64(q).reshape(B, Hkv, G, d).mean(axis=2)
    rng = np.random.default_rng(seed)
    K64 = f64(K)
    for b in range(B):
        for h in range(Hkv):
            rows = rng.choice(N, size=max(1, N // 100), replace=False)
            K64[b, h, rows] += 2.0 * qbar[b, h]
    K = torch.from_numpy(K64).to(torch.bfloat16)
    return (B, Hq, Hkv, d, r, N, n_max, lens, M), q, K, V, P


# every case as planned, and the short ones also with the filter plan
TOPM_PARAMS = [(n, "planned") for n in TOPM_CASES] + [
    (n, "filter") for n, c in TOPM_CASES.items() if _scores_shape(c[6], c[8])]


@pytest.mark.parametrize("name,plan", TOPM_PARAMS)
def test_topm_fused_and_unfused_match_oracle(name, plan, monkeypatch):
    (B, Hq, Hkv, d, r, N, n_max, lens, M), q, K, V, P = _topm_case(name)
    _say("case: topm", name, plan, "B=%d Hkv=%d n_max=%d M=%d" % (B, Hkv, n_max, M))
    _use_plan(monkeypatch, plan)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    want_plan = (sa.SA_PLAN_SCORES if plan == "planned" and _scores_shape(n_max, M) else
                 sa.SA_PLAN_FILTER if n_max <= 2 ** 19 and M <= 6144 and M < n_max else
                 sa.SA_PLAN_CHUNK_EXACT)
    assert sa.sparse_attn_selection_plan(sh, n_max, M) == want_plan
    P64 = P.double().numpy()
    kp = oracle_kp(f64(K), P64)
    qd, Pd, kpd = _dev(q), _dev(P), _dev(kp)
    sl = None if lens is None else _dev(torch.tensor(lens, dtype=torch.int32))
    ws = sa.alloc_workspace(sh, n_max, M)
    scores = torch.empty(B, Hkv, n_max, dtype=torch.float32, device="cuda")
    idx_u = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    idx_f = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    sa.sparse_attn_index_score(sh, qd, Pd, kpd, sl, n_max, scores)
    sa.sparse_attn_topm(sh, scores, sl, n_max, M, idx_u, ws)
    sa.sparse_attn_index_topm(sh, qd, Pd, kpd, sl, n_max, M, idx_f, ws)
    idx_s = torch.full_like(idx_f, -7)
    for stage in (sa.SA_STAGE_BOUND, sa.SA_STAGE_CANDIDATES, sa.SA_STAGE_MERGE):
        sa.sparse_attn_index_topm_stage(sh, stage, qd, Pd, kpd, sl, n_max, M, idx_s, ws)
    # which method served the shape: the merge over the kept keys or the
    # scores (no unit falls back to the exact streaming pass) inside the
    # filter path's limits, else chunk-exact
    fb = _fallbacks(sh, n_max, M, ws)
    filter_path = n_max <= 2 ** 19 and M <= 6144 and M < n_max
    assert fb == (0 if filter_path else -1), (name, fb)
    gu, gf = idx_u.cpu().numpy(), idx_f.cpu().numpy()
    assert np.array_equal(gu, gf), "fused and unfused index sets differ"
    assert np.array_equal(idx_s.cpu().numpy(), gf), "two-call selection differs"
    G = Hq // Hkv
    swaps = 0
    for b in range(B):
        L = n_max if lens is None else min(lens[b], n_max)
        for h in range(Hkv):
            qt = oracle.indexer_query(f64(q)[b, h * G:(h + 1) * G], P64[h])
            s = oracle.index_scores(qt, kp[b, h, :L])
            swaps += check_topm_unit(gf[b, h], s, M, L)
    _say("  band swaps:", swaps)


def test_topm_ties_take_lowest_positions():
    _say("case: topm ties")
    B, Hq, Hkv, d, r, N, M = 1, 1, 1, 64, 16, 4096, 100
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16)
    q[0, 0, 0] = 1.0
    P = torch.zeros(Hkv, d, r, dtype=torch.float32)
    P[0, :r, :r] = torch.eye(r)
    # score = dec(code in column 0): 300 rows share the top code, so the top-100
    # are the 100 lowest of those rows
    rng = np.random.default_rng(0)
    col = np.full(N, 0x30, dtype=np.uint8)                 # 0.5 everywhere
    top_rows = np.sort(rng.choice(N, 300, replace=False))
    col[top_rows] = 0x40                                   # 2.0
    kp = np.zeros((B, Hkv, N, r), dtype=np.uint8)
    kp[0, 0, :, 0] = col
    ws = sa.alloc_workspace(sh, N, M)
    idx = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), _dev(kp), None, N, M, idx, ws)
    assert idx.cpu().numpy()[0, 0].tolist() == top_rows[:M].tolist()
    scores = torch.empty(B, Hkv, N, dtype=torch.float32, device="cuda")
    sa.sparse_attn_index_score(sh, _dev(q), _dev(P), _dev(kp), None, N, scores)
    idx2 = torch.empty_like(idx)
    sa.sparse_attn_topm(sh, scores, None, N, M, idx2, ws)
    assert torch.equal(idx, idx2)


# ------------------------------------------------------------------ attention

DECODE_CASES = [
    # (B, Hq, Hkv, d, Ncap, M, pad_mode)
    (2, 8, 2, 128, 3000, 2048, "none"),
    (2, 28, 4, 128, 5000, 1000, "pad"),
    (1, 16, 16, 64, 700, 97, "dups"),
    (1, 16, 1, 64, 4000, 3000, "oob"),
    (3, 4, 1, 128, 500, 1, "none"),
    (2, 12, 4, 128, 300, 300, "all"),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_matches_oracle(case):
    B, Hq, Hkv, d, Ncap, M, mode = case
    _say("case: decode", case)
    r = 16
    sh = _shape_of(B, Hq, Hkv, d, r, Ncap)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, Ncap, seed=B * 100 + Hq)
    rng = np.random.default_rng(M)
    idx = np.zeros((B, Hkv, M), dtype=np.int32)
    for b in range(B):
        for h in range(Hkv):
            if mode == "all":
                idx[b, h] = np.arange(M)
            else:
                idx[b, h] = np.sort(rng.choice(Ncap, M, replace=False))
            if mode == "pad":
                idx[b, h, M - 1 - b * 300:] = -1
            elif mode == "dups":
                idx[b, h, ::3] = idx[b, h, 0]
            elif mode == "oob":
                idx[b, h, ::7] = Ncap + 5
    if mode == "pad" and B > 1:
        idx[B - 1, 0, :] = -1                    # a unit with no valid row
    scale = default_scale(d)
    ws = sa.alloc_workspace(sh, min(M, Ncap), M)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    sa.sparse_attn_decode(sh, _dev(q), _dev(K), _dev(V), _dev(idx), M, scale, out, lse, ws)
    G = Hq // Hkv
    got, gl = f64(out), lse.cpu().double().numpy()
    for b in range(B):
        for h in range(Hkv):
            o, l = oracle.sparse_attention(f64(q)[b, h * G:(h + 1) * G], f64(K)[b, h],
                                           f64(V)[b, h], idx[b, h], scale)
            check_attention(got[b, h * G:(h + 1) * G], o, "decode %s b=%d h=%d" % (case, b, h))
            fin = np.isfinite(l)
            assert np.array_equal(np.isfinite(gl[b, h * G:(h + 1) * G]), fin)
            assert np.all(np.abs(gl[b, h * G:(h + 1) * G][fin] - l[fin]) <= 1e-3 * (1 + np.abs(l[fin])))
            if M == 1 and idx[b, h, 0] >= 0:
                assert np.array_equal(got[b, h * G:(h + 1) * G],
                                      np.repeat(f64(V)[b, h, idx[b, h, 0]][None], G, 0))


def test_decode_split_count_and_order_invariance():
    _say("case: decode invariances")
    B, Hq, Hkv, d, Ncap, M = 1, 4, 1, 128, 5000, 2048
    sh = _shape_of(B, Hq, Hkv, d, 16, Ncap)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, 16, Ncap, seed=9)
    rng = np.random.default_rng(1)
    idx = np.sort(rng.choice(Ncap, M, replace=False)).astype(np.int32)[None, None]
    ws = sa.alloc_workspace(sh, M, M)
    outs = []
    for perm in (None, rng.permutation(M)):
        ii = idx if perm is None else idx[:, :, perm]
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        sa.sparse_attn_decode(sh, _dev(q), _dev(K), _dev(V), _dev(ii), M, default_scale(d),
                              out, None, ws)
        outs.append(f64(out))
    o, _ = oracle.sparse_attention(f64(q)[0], f64(K)[0, 0], f64(V)[0, 0], idx[0, 0],
                                   default_scale(d))
    for x in outs:
        check_attention(x[0], o)


# ------------------------------------------------------------------ linear + gate

@pytest.mark.parametrize("G,d", [(4, 128), (7, 128), (2, 64)])
def test_linear_gate_matches_oracle(G, d):
    _say("case: linear_gate G=%d d=%d" % (G, d))
    B, Hkv, N = 2, 2, 300
    Hq = G * Hkv
    sh = _shape_of(B, Hq, Hkv, d, 16, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, 16, N, seed=G)
    g = torch.Generator().manual_seed(3)
    w = (0.5 * torch.randn(Hq, d, generator=g)).float()
    o_sp = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    K64, V64, q64 = f64(K), f64(V), f64(q)
    S0 = np.zeros((B, Hkv, d, d))
    z0 = np.zeros((B, Hkv, d))
    for b in range(B):
        for h in range(Hkv):
            S0[b, h], z0[b, h] = oracle.linear_state(K64[b, h, :N - 1], V64[b, h, :N - 1])
    Sd = _dev(torch.from_numpy(S0).float())
    zd = _dev(torch.from_numpy(z0).float())
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    sa.sparse_attn_linear_gate(sh, _dev(q), _dev(K[:, :, N - 1]), _dev(V[:, :, N - 1]), Sd, zd,
                               _dev(w), _dev(o_sp), out, True)
    got = f64(out)
    for b in range(B):
        for h in range(Hkv):
            S, z = oracle.linear_state(K64[b, h], V64[b, h])
            np.testing.assert_allclose(Sd[b, h].cpu().double().numpy(), S, rtol=1e-5, atol=1e-3)
            np.testing.assert_allclose(zd[b, h].cpu().double().numpy(), z, rtol=1e-5)
            o, _, _ = oracle.linear_gate(q64[b, h * G:(h + 1) * G], S, z,
                                         w.double().numpy()[h * G:(h + 1) * G],
                                         f64(o_sp)[b, h * G:(h + 1) * G])
            check_attention(got[b, h * G:(h + 1) * G], o, "linear gate")
    # read-only call leaves the state untouched
    S_before = Sd.clone()
    sa.sparse_attn_linear_gate(sh, _dev(q), _dev(K[:, :, N - 1]), _dev(V[:, :, N - 1]), Sd, zd,
                               _dev(w), _dev(o_sp), out, False)
    assert torch.equal(S_before, Sd)


def test_linear_gate_empty_state_reads_out_zero():
    """A fresh state (S = 0, z = 0) read without an update: the linear read-out
    is defined as 0, so out = g * o_sparse (the oracle's reading), finite."""
    _say("case: linear_gate empty state")
    B, Hkv, G, d = 2, 2, 4, 128
    Hq = G * Hkv
    sh = _shape_of(B, Hq, Hkv, d, 16, 8)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, 16, 8, seed=3)
    g = torch.Generator().manual_seed(4)
    w = (0.5 * torch.randn(Hq, d, generator=g)).float()
    o_sp = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    Sd = torch.zeros(B, Hkv, d, d, dtype=torch.float32, device="cuda")
    zd = torch.zeros(B, Hkv, d, dtype=torch.float32, device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    sa.sparse_attn_linear_gate(sh, _dev(q), _dev(K[:, :, 0]), _dev(V[:, :, 0]), Sd, zd,
                               _dev(w), _dev(o_sp), out, False)
    got = f64(out)
    assert np.all(np.isfinite(got))
    for b in range(B):
        for h in range(Hkv):
            o, o_lin, _ = oracle.linear_gate(f64(q)[b, h * G:(h + 1) * G], np.zeros((d, d)),
                                             np.zeros(d), w.double().numpy()[h * G:(h + 1) * G],
                                             f64(o_sp)[b, h * G:(h + 1) * G])
            assert np.all(o_lin == 0.0)
            check_attention(got[b, h * G:(h + 1) * G], o, "empty state")


# ------------------------------------------------------------------ whole step

def _run_step(inp, sh, M, ws, fused=True):
    wl = inp.wl
    kp = torch.zeros(wl.B, wl.Hkv, sh.capacity, wl.r, dtype=torch.uint8, device="cuda")
    sa.sparse_attn_project_keys(sh, inp.k_cache, inp.P, 0, sh.capacity, kp)
    sa.sparse_attn_append_kv(sh, inp.pos, inp.k_new, inp.v_new, inp.P, inp.k_cache,
                             inp.v_cache, kp)
    idx = torch.empty(wl.B, wl.Hkv, M, dtype=torch.int32, device="cuda")
    n_max = int(inp.seq_lens.max().item())
    if fused:
        sa.sparse_attn_index_topm(sh, inp.q, inp.P, kp, inp.seq_lens, n_max, M, idx, ws)
    else:
        scores = torch.empty(wl.B, wl.Hkv, n_max, dtype=torch.float32, device="cuda")
        sa.sparse_attn_index_score(sh, inp.q, inp.P, kp, inp.seq_lens, n_max, scores)
        sa.sparse_attn_topm(sh, scores, inp.seq_lens, n_max, M, idx, ws)
    out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device="cuda")
    sa.sparse_attn_decode(sh, inp.q, inp.k_cache, inp.v_cache, idx, M, default_scale(wl.d),
                          out, lse, ws)
    return kp, idx, out, lse


@pytest.mark.parametrize("name,N", [("tiny", None), ("gqa7_16k", 4096)])
def test_decode_step_end_to_end(name, N):
    wl = WORKLOADS[name] if N is None else scaled(WORKLOADS[name], N=N, M=512)
    _say("case: step", wl.name, wl.N, wl.M)
    inp = make_decode_inputs(wl, seed=4, device="cuda")
    K0, V0 = f64(inp.k_cache), f64(inp.v_cache)
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    ws = sa.alloc_workspace(sh, wl.N, wl.M)
    kp, idx, out, lse = _run_step(inp, sh, wl.M, ws)
    _, idx2, out2, _ = _run_step(make_decode_inputs(wl, seed=4, device="cuda"), sh, wl.M, ws,
                                 fused=False)
    assert torch.equal(idx, idx2)
    P64 = inp.P.double().cpu().numpy()
    kp0 = oracle_kp(K0, P64)
    K2, V2, kp2 = oracle.append_kv(K0, V0, kp0, inp.pos.cpu().numpy(), f64(inp.k_new),
                                   f64(inp.v_new), P64)
    G = wl.G
    gi, go = idx.cpu().numpy(), f64(out)
    q64 = f64(inp.q)
    for b in range(wl.B):
        for h in range(wl.Hkv):
            qg = q64[b, h * G:(h + 1) * G]
            oi, oo, ol, s = oracle.decode_step_unit(qg, K2[b, h], V2[b, h], kp2[b, h], P64[h],
                                                    wl.N, wl.M, default_scale(wl.d))
            check_topm_unit(gi[b, h], s, wl.M, wl.N)
            if not np.array_equal(gi[b, h], oi):
                # a band swap: the oracle attends over the GPU's (equally valid) set
                oo, _ = oracle.sparse_attention(qg, K2[b, h], V2[b, h], gi[b, h],
                                                default_scale(wl.d))
            check_attention(go[b, h * G:(h + 1) * G], oo, "step unit %s" % ((b, h),))
            if (b, h) in inp.plants and wl.plant_mode == "replace":
                assert set(inp.plants[(b, h)].tolist()) <= set(gi[b, h].tolist())


def test_determinism():
    _say("case: determinism")
    wl = scaled(WORKLOADS["gqa7_16k"], N=8192, M=1024, B=2)
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    ws = sa.alloc_workspace(sh, wl.N, wl.M)
    res = [_run_step(make_decode_inputs(wl, seed=1, device="cuda"), sh, wl.M, ws)
           for _ in range(2)]
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ cross-layer reuse

def test_cross_layer_reuse_equals_decode_with_source_indices():
    _say("case: cross-layer reuse")
    wl = scaled(WORKLOADS["reuse8_64k"], N=4096, B=2, M=256)
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    ws = sa.alloc_workspace(sh, wl.N, wl.M)
    idx_of = {}
    for layer in range(wl.layers):
        inp = make_decode_inputs(wl, seed=2, layer=layer, device="cuda")
        src = oracle.reuse_source_layer(layer, wl.full_layers)
        if layer == src:
            kp, idx, out, lse = _run_step(inp, sh, wl.M, ws)
            idx_of[layer] = idx
        else:
            idx = idx_of[src]
            out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device="cuda")
            sa.sparse_attn_append_kv(sh, inp.pos, inp.k_new, inp.v_new, inp.P, inp.k_cache,
                                     inp.v_cache, torch.zeros(wl.B, wl.Hkv, wl.N, wl.r,
                                                              dtype=torch.uint8, device="cuda"))
            sa.sparse_attn_decode(sh, inp.q, inp.k_cache, inp.v_cache, idx, wl.M,
                                  default_scale(wl.d), out, None, ws)
        G = wl.G
        gi = idx.cpu().numpy()
        q64, K64, V64 = f64(inp.q), f64(inp.k_cache), f64(inp.v_cache)
        for b in range(wl.B):
            for h in range(wl.Hkv):
                o, _ = oracle.sparse_attention(q64[b, h * G:(h + 1) * G], K64[b, h], V64[b, h],
                                               gi[b, h], default_scale(wl.d))
                check_attention(f64(out)[b, h * G:(h + 1) * G], o, "layer %d" % layer)


# ------------------------------------------------------------------ full size

def _bench_sequence(inp, sh, M, ws):
    """The calls, in the order and launch configuration bench.py times: the
    three stages of sparse_attn_decode_step."""
    wl = inp.wl
    kp = torch.empty(wl.B, wl.Hkv, wl.N, wl.r, dtype=torch.uint8, device="cuda")
    sa.sparse_attn_project_keys(sh, inp.k_cache, inp.P, 0, wl.N, kp)
    idx = torch.empty(wl.B, wl.Hkv, M, dtype=torch.int32, device="cuda")
    out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device="cuda")
    for stage in (sa.SA_STEP_APPEND_BOUND, sa.SA_STEP_CANDIDATES, sa.SA_STEP_SELECT_ATTEND):
        sa.sparse_attn_decode_step_stage(sh, stage, inp.pos, inp.k_new, inp.v_new, inp.q,
                                         inp.P, inp.k_cache, inp.v_cache, kp, inp.seq_lens,
                                         wl.N, M, default_scale(wl.d), idx, out, lse, ws)
    return kp, idx, out, lse


@pytest.mark.parametrize("name,over", [("longctx_128k", {}), ("gqa7_16k", {}),
                                       ("longctx_128k", {"d": 64, "r": 16})])
def test_full_size_step_on_sampled_units(name, over):
    """Whole workload at its real size.  The oracle checks 16 units (first,
    last and 14 seeded ones) exactly: the index set against the top-M
    contract and the output against the oracle's attention.  Every unit is
    checked for properties that hold at any size: idx ascending, distinct,
    in range and -1-padded only past the valid count; the two-call selection
    equals the one-call selection; and, per unit, the planted rows missing
    from the selection stay under the bound the input recipe implies
    (_helpers.plant_miss_bound)."""
    wl = scaled(WORKLOADS[name], **over) if over else WORKLOADS[name]
    _say("case: full size", wl.name, "B=%d Hkv=%d d=%d r=%d N=%d M=%d"
         % (wl.B, wl.Hkv, wl.d, wl.r, wl.N, wl.M))
    inp = make_decode_inputs(wl, seed=7, device="cuda")
    picks = _picks(wl, np.random.default_rng(11), extra=14, distinct=16)
    # the generator's cache rows of the checked units, before the HIP append
    saved = {(b, h): (inp.k_cache[b, h].cpu(), inp.v_cache[b, h].cpu()) for b, h in picks}
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    ws = sa.alloc_workspace(sh, wl.N, wl.M)
    kp, idx, out, lse = _bench_sequence(inp, sh, wl.M, ws)
    idx1 = torch.empty_like(idx)
    sa.sparse_attn_index_topm(sh, inp.q, inp.P, kp, inp.seq_lens, wl.N, wl.M, idx1, ws)
    assert torch.equal(idx, idx1)
    gi = idx.cpu().numpy()
    assert np.all(gi >= 0) and np.all(gi < wl.N)
    assert np.all(np.diff(gi, axis=-1) > 0), "indices must ascend strictly"
    assert np.all(np.isfinite(lse.cpu().numpy()))
    P64 = inp.P.double().cpu().numpy()
    q64, go, gl = f64(inp.q), f64(out), lse.cpu().double().numpy()
    G = wl.G
    # the recipe's planted rows, per unit, against the bound the recipe implies
    qbar = q64.reshape(wl.B, wl.Hkv, G, wl.d).mean(axis=2)
    worst = 0.0
    for (b, h), rows in inp.plants.items():
        sigma = float(np.linalg.norm(qbar[b, h] @ P64[h]))
        bound, _ = plant_miss_bound(sigma, wl.N, wl.M, rows.size, wl.plant_alpha,
                                    wl.recent_rows, wl.recent_beta)
        miss = rows.size - np.intersect1d(rows, gi[b, h]).size
        assert miss <= bound, ((b, h), miss, bound, sigma)
        worst = max(worst, miss / bound)
    _say("  plants: worst unit at %.2f of its bound" % worst)
    for b, h in picks:
        K2, V2, kp2, P64h = _unit_after_append(inp, f64(saved[(b, h)][0]),
                                               f64(saved[(b, h)][1]), b, h)
        qg = q64[b, h * G:(h + 1) * G]
        oi, oo, ol, s = oracle.decode_step_unit(qg, K2, V2, kp2, P64h, wl.N, wl.M,
                                                default_scale(wl.d))
        swaps = check_topm_unit(gi[b, h], s, wl.M, wl.N)
        _say("  unit", (b, h), "band swaps", swaps)
        if not np.array_equal(gi[b, h], oi):
            oo, ol = oracle.sparse_attention(qg, K2, V2, gi[b, h], default_scale(wl.d))
        check_attention(go[b, h * G:(h + 1) * G], oo, "full-size unit %s" % ((b, h),))
        assert np.all(np.abs(gl[b, h * G:(h + 1) * G] - ol) <= 1e-3 * (1 + np.abs(ol)))


def _picks(wl, rng, extra=1, distinct=None):
    """First and last unit plus ``extra`` seeded ones (drawn until ``distinct``
    different units are picked, when given)."""
    got = {(0, 0), (wl.B - 1, wl.Hkv - 1)}
    want = min(distinct, wl.B * wl.Hkv) if distinct else None
    for _ in range(extra):
        got.add((int(rng.integers(wl.B)), int(rng.integers(wl.Hkv))))
    while want is not None and len(got) < want:
        got.add((int(rng.integers(wl.B)), int(rng.integers(wl.Hkv))))
    return sorted(got)


def _unit_after_append(inp, K0, V0, b, h):
    """The oracle's rows and FP8 codes of unit (b, h) after the step's append,
    from the generator's rows K0, V0 (before the HIP append)."""
    P64 = inp.P.double().cpu().numpy()
    pos = inp.pos.cpu().numpy()
    kp0 = oracle.project_keys(K0, P64[h])[None, None]
    K2, V2, kp2 = oracle.append_kv(K0[None, None], V0[None, None], kp0, pos[b:b + 1],
                                   f64(inp.k_new[b:b + 1, h:h + 1]),
                                   f64(inp.v_new[b:b + 1, h:h + 1]), P64[h:h + 1])
    return K2[0, 0], V2[0, 0], kp2[0, 0], P64[h]


def test_full_size_cross_layer_reuse_on_sampled_units():
    """reuse8_64k at its real size (B16, Hkv8, N65536, M2048; eight layers with
    their own caches and queries).  The full layers 0 and 4 run the decode
    step as bench.py launches it; layers 1-3 and 5-7 append their token and
    attend, with sparse_attn_decode, over the index sets of their full layer.
    In every layer the first and last unit and a seeded one are checked: the
    full layers' sets against the exact top-M contract, every layer's output
    against the oracle's attention over that layer's rows at the indices it
    used, and every layer's appended FP8 code row against the oracle's."""
    wl = WORKLOADS["reuse8_64k"]
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    ws = sa.alloc_workspace(sh, wl.N, wl.M)
    rng = np.random.default_rng(17)
    idx_of = {}
    G = wl.G
    for layer in range(wl.layers):
        src = oracle.reuse_source_layer(layer, wl.full_layers)
        _say("case: full-size reuse, layer", layer, "indices of layer", src)
        inp = make_decode_inputs(wl, seed=9, layer=layer, device="cuda")
        picks = _picks(wl, rng)
        saved = {(b, h): (f64(inp.k_cache[b, h]), f64(inp.v_cache[b, h])) for b, h in picks}
        if layer == src:
            kp, idx, out, lse = _bench_sequence(inp, sh, wl.M, ws)
            idx_of[layer] = idx
        else:
            idx = idx_of[src]
            kp = torch.zeros(wl.B, wl.Hkv, wl.N, wl.r, dtype=torch.uint8, device="cuda")
            sa.sparse_attn_append_kv(sh, inp.pos, inp.k_new, inp.v_new, inp.P, inp.k_cache,
                                     inp.v_cache, kp)
            out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device="cuda")
            sa.sparse_attn_decode(sh, inp.q, inp.k_cache, inp.v_cache, idx, wl.M,
                                  default_scale(wl.d), out, lse, ws)
        torch.cuda.synchronize()
        gi, go, gl = idx.cpu().numpy(), f64(out), lse.cpu().double().numpy()
        pos = inp.pos.cpu().numpy()
        q64 = f64(inp.q)
        for b, h in picks:
            K2, V2, kp2, P64h = _unit_after_append(inp, *saved[(b, h)], b, h)
            qg = q64[b, h * G:(h + 1) * G]
            row = kp[b, h, pos[b]].cpu().numpy()[None, None, None]
            ok, _ = kp_codes_match(row, kp2[pos[b]][None, None, None],
                                   K2[pos[b]][None, None, None], P64h[None])
            assert ok, "layer %d unit %s: appended code row" % (layer, (b, h))
            if layer == src:
                s = oracle.index_scores(oracle.indexer_query(qg, P64h), kp2[:wl.N])
                swaps = check_topm_unit(gi[b, h], s, wl.M, wl.N)
                _say("  unit", (b, h), "band swaps", swaps)
            o, l = oracle.sparse_attention(qg, K2, V2, gi[b, h], default_scale(wl.d))
            check_attention(go[b, h * G:(h + 1) * G], o, "layer %d unit %s" % (layer, (b, h)))
            assert np.all(np.abs(gl[b, h * G:(h + 1) * G] - l) <= 1e-3 * (1 + np.abs(l)))
        del inp, kp, out, lse


def test_full_size_gated_hybrid_on_sampled_units():
    """lisa_32k at its real size (B16, Hq32, Hkv8, N32768, M1024): the sparse
    branch is the decode step as bench.py launches it; the linear branch's
    state is prefilled over the rows before the new token (fp32, torch, as a
    serving stack would have carried it) and sparse_attn_linear_gate adds the
    new token and mixes the two branches.  On the first and last unit and a
    seeded one: the index set against the top-M contract, the updated state
    against the oracle's sums over all N rows, and the mixed output against
    the oracle's gate applied to its own sparse attention at the same
    indices."""
    wl = WORKLOADS["lisa_32k"]
    B, Hq, Hkv, d, N, G = wl.B, wl.Hq, wl.Hkv, wl.d, wl.N, wl.G
    _say("case: full-size gated hybrid", wl.name)
    inp = make_decode_inputs(wl, seed=5, device="cuda")
    picks = _picks(wl, np.random.default_rng(19))
    saved = {(b, h): (f64(inp.k_cache[b, h]), f64(inp.v_cache[b, h])) for b, h in picks}
    S = torch.empty(B, Hkv, d, d, dtype=torch.float32, device="cuda")
    z = torch.empty(B, Hkv, d, dtype=torch.float32, device="cuda")
    for b in range(B):
        Kf = inp.k_cache[b, :, :N - 1].float()
        phi = torch.where(Kf > 0, Kf + 1.0, torch.exp(torch.clamp(Kf, max=0.0)))
        S[b] = torch.matmul(phi.transpose(1, 2).contiguous(), inp.v_cache[b, :, :N - 1].float())
        z[b] = phi.sum(dim=1)
    del Kf, phi
    sh = _shape_of(B, Hq, Hkv, d, wl.r, N)
    ws = sa.alloc_workspace(sh, N, wl.M)
    kp, idx, o_sp, lse = _bench_sequence(inp, sh, wl.M, ws)
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    sa.sparse_attn_linear_gate(sh, inp.q, inp.k_new.view(B, Hkv, d), inp.v_new.view(B, Hkv, d),
                               S, z, inp.w_gate, o_sp, out, True)
    torch.cuda.synchronize()
    gi, go = idx.cpu().numpy(), f64(out)
    q64, w64 = f64(inp.q), inp.w_gate.double().cpu().numpy()
    for b, h in picks:
        K2, V2, kp2, P64h = _unit_after_append(inp, *saved[(b, h)], b, h)
        qg = q64[b, h * G:(h + 1) * G]
        s = oracle.index_scores(oracle.indexer_query(qg, P64h), kp2[:N])
        swaps = check_topm_unit(gi[b, h], s, wl.M, N)
        _say("  unit", (b, h), "band swaps", swaps)
        S64, z64 = oracle.linear_state(K2[:N], V2[:N])
        # fp32 sums of N terms in blocks: error well inside 64 ulp of the sum
        # of the terms' magnitudes
        phi_abs = np.abs(oracle.elu_plus_one(K2[:N]))
        tol_S = 64 * 2.0 ** -24 * (phi_abs.T @ np.abs(V2[:N]))
        assert np.all(np.abs(S[b, h].cpu().double().numpy() - S64) <= tol_S + 1e-6)
        tol_z = 64 * 2.0 ** -24 * phi_abs.sum(axis=0)
        assert np.all(np.abs(z[b, h].cpu().double().numpy() - z64) <= tol_z)
        o_sp64, _ = oracle.sparse_attention(qg, K2, V2, gi[b, h], default_scale(d))
        want, _, g = oracle.linear_gate(qg, S64, z64, w64[h * G:(h + 1) * G], o_sp64)
        assert np.all((g > 0.2) & (g < 0.8)), g      # both branches weigh in
        check_attention(go[b, h * G:(h + 1) * G], want, "hybrid unit %s" % ((b, h),))


# ------------------------------------------------------------------ exact fallbacks

def _topm_check_against_oracle(q, P, kp, M, n_max, lens=None):
    B, Hkv = kp.shape[0], kp.shape[1]
    Hq, d = q.shape[1], q.shape[2]
    r, N = kp.shape[3], kp.shape[2]
    G = Hq // Hkv
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    ws = sa.alloc_workspace(sh, n_max, M)
    idx = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    sl = None if lens is None else _dev(torch.tensor(lens, dtype=torch.int32))
    sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), _dev(kp), sl, n_max, M, idx, ws)
    fb_fused = _fallbacks(sh, n_max, M, ws)
    scores = torch.empty(B, Hkv, n_max, dtype=torch.float32, device="cuda")
    sa.sparse_attn_index_score(sh, _dev(q), _dev(P), _dev(kp), sl, n_max, scores)
    idx2 = torch.empty_like(idx)
    sa.sparse_attn_topm(sh, scores, sl, n_max, M, idx2, ws)
    assert _fallbacks(sh, n_max, M, ws) == fb_fused, "the two sources took different paths"
    _topm_check_against_oracle.fallbacks = fb_fused
    assert torch.equal(idx, idx2), "index_topm and index_score + topm differ"
    gi = idx.cpu().numpy()
    P64 = P.double().numpy()
    for b in range(B):
        L = n_max if lens is None else min(lens[b], n_max)
        for h in range(Hkv):
            qt = oracle.indexer_query(f64(q)[b, h * G:(h + 1) * G], P64[h])
            s = oracle.index_scores(qt, kp[b, h, :L])
            check_topm_unit(gi[b, h], s, M, L)
    return gi


def test_topm_all_scores_equal_takes_lowest_positions():
    """Every score equal: every candidate list overflows, so the exact
    streaming selection of the unit runs; ties go to the lowest positions."""
    _say("case: topm all equal")
    B, Hq, Hkv, d, r, N, M = 1, 4, 1, 64, 16, 65536, 100
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16)
    q[0, :, 0] = 1.0
    P = torch.zeros(Hkv, d, r, dtype=torch.float32)
    P[0, :r, :r] = torch.eye(r)
    kp = np.zeros((B, Hkv, N, r), dtype=np.uint8)
    kp[..., 0] = 0x38                                      # 1.0 everywhere
    gi = _topm_check_against_oracle(q, P, kp, M, N)
    assert _topm_check_against_oracle.fallbacks == 1        # the exact pass served it
    assert gi[0, 0].tolist() == list(range(M))


@pytest.mark.parametrize("plan", ["planned", "filter"])
def test_topm_ties_cut_by_m_take_lowest_positions(plan, monkeypatch):
    """97 distinct FP8 rows repeated along the context: scores come in tie
    groups of ~169 and M cuts one; the merge over all scores (as planned)
    and the filter path's merge (no list can overflow here) must take, of
    the tied group, exactly the lowest positions, as the chunk-exact path and
    the oracle do."""
    _say("case: topm ties cut by M", plan)
    _use_plan(monkeypatch, plan)
    B, Hq, Hkv, d, r, N, M = 1, 4, 1, 128, 32, 16384, 1000
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, 97, seed=23)
    P64 = P.double().numpy()
    base = oracle_kp(f64(K), P64)                           # [1, 1, 97, r]
    kp = np.ascontiguousarray(base[:, :, np.arange(N) % 97, :])
    gi = _topm_check_against_oracle(q, P, kp, M, N)
    assert _topm_check_against_oracle.fallbacks == 0        # the merge served it
    qt = oracle.indexer_query(f64(q)[0], P64[0])
    s = oracle.index_scores(qt, kp[0, 0])
    v = np.sort(s)[::-1][M - 1]
    above = np.flatnonzero(s > v)
    tied = np.flatnonzero(s == v)
    need = M - above.size
    assert 0 < need < tied.size, (need, tied.size)          # M really cuts a tie group
    assert gi[0, 0].tolist() == sorted(above.tolist() + tied[:need].tolist())


def test_topm_sample_overestimate_falls_back_exactly():
    """High scores planted exactly on positions the bound's sample reads (its
    128 evenly spread blocks of 8 rows; 16 of them here, 128 rows, more than
    the k = 96 sample keys the bound ranks down to) push the sampled bound
    above the M-th score, so fewer than M positions reach it; the merge must
    detect it and select exactly."""
    _say("case: topm sample overestimate")
    B, Hq, Hkv, d, r, N, M = 1, 4, 1, 128, 32, 65536, 2048
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=21)
    K64 = f64(K)
    qbar = f64(q).reshape(B, Hkv, Hq // Hkv, d).mean(axis=2)
    starts = [(j * (N - 8)) // 127 for j in range(128)]
    rows = np.concatenate([np.arange(s0, s0 + 8) for s0 in starts[::8]])   # 128 rows
    K64[0, 0, rows] += 6.0 * qbar[0, 0]
    P64 = P.double().numpy()
    kp = oracle_kp(K64, P64)
    gi = _topm_check_against_oracle(q, P, kp, M, N)
    assert _topm_check_against_oracle.fallbacks == 1        # the bound overshot: exact pass
    assert set(rows.tolist()) <= set(gi[0, 0].tolist())


@pytest.mark.parametrize("d,r", [(128, 32), (64, 16)])
def test_topm_clustered_high_scores(d, r):
    """Runs of consecutive high-scoring positions (a relevant passage) fill the
    filter's per-wave candidate lists, which then go to the unit's spill pool;
    the selection must stay exact.  Unit (0, 0): 3000 rows inside one chunk;
    (0, 1): 1500 rows across a chunk boundary; (1, 0): none; (1, 1): 40000 rows,
    more candidates than the merge holds, so the exact fallback runs."""
    _say("case: topm clustered d=%d r=%d" % (d, r))
    B, Hq, Hkv, N, M = 2, 8, 2, 65536, 2048
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=23)
    K64 = f64(K)
    qbar = f64(q).reshape(B, Hkv, Hq // Hkv, d).mean(axis=2)
    runs = {(0, 0): (10000, 13000), (0, 1): (7500, 9000), (1, 1): (20000, 60000)}
    for (b, h), (lo, hi) in runs.items():
        K64[b, h, lo:hi] += 3.0 * qbar[b, h]
    P64 = P.double().numpy()
    kp = oracle_kp(K64, P64)
    gi = _topm_check_against_oracle(q, P, kp, M, N)
    # unit (1, 1) may overflow the merge (then the exact pass serves it); the
    # other units' runs go through the spill pool and the merge
    assert _topm_check_against_oracle.fallbacks in (0, 1)
    # the recipe does what it is for: the runs dominate their units' selections
    assert np.isin(np.arange(7500, 9000), gi[0, 1]).mean() > 0.98
    assert np.isin(gi[0, 0], np.arange(10000, 13000)).mean() > 0.98


def test_decode_step_with_clustered_high_scores():
    """The fused decode step (append + bound, candidates, select + attend in
    one workgroup) over units whose high scores come in runs, so that wave
    lists spill: the same caches, idx, out and lse as the three separate
    calls, and the oracle's selection and attention on the checked units."""
    _say("case: decode step, clustered")
    B, Hq, Hkv, d, r, N, M = 2, 8, 2, 128, 32, 65536, 2048
    G = Hq // Hkv
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=29)
    K64 = f64(K)
    qbar = f64(q).reshape(B, Hkv, G, d).mean(axis=2)
    runs = {(0, 0): (10000, 13000), (1, 1): (31000, 34500)}     # one across a chunk boundary
    for (b, h), (lo, hi) in runs.items():
        K64[b, h, lo:hi] += 3.0 * qbar[b, h]
    K = torch.from_numpy(K64).to(torch.bfloat16)
    K64 = f64(K)                        # the cache holds the bf16-rounded keys
    g = torch.Generator().manual_seed(31)
    k_new = torch.randn(B, Hkv, 1, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, 1, d, generator=g).to(torch.bfloat16)
    pos = torch.full((B,), N - 1, dtype=torch.int32)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    res = []
    for fused in (False, True):
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        if fused:
            sa.sparse_attn_decode_step(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(q), _dev(P),
                                       Kd, Vd, kp, None, N, M, default_scale(d), idx, out, lse,
                                       ws)
        else:
            sa.sparse_attn_append_kv(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(P), Kd, Vd, kp)
            sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), kp, None, N, M, idx, ws)
            sa.sparse_attn_decode(sh, _dev(q), Kd, Vd, idx, M, default_scale(d), out, lse, ws)
        torch.cuda.synchronize()
        res.append((Kd, Vd, kp, idx, out, lse))
    for x, y in zip(res[0], res[1]):
        assert torch.equal(x, y)
    _, _, _, idx, out, _ = res[1]
    gi, go = idx.cpu().numpy(), f64(out)
    P64 = P.double().numpy()
    q64 = f64(q)
    for (b, h), (lo, hi) in runs.items():
        K0, V0 = K64[b, h], f64(V)[b, h]
        kp0 = oracle.project_keys(K0, P64[h])[None, None]
        K2, V2, kp2 = oracle.append_kv(K0[None, None], V0[None, None], kp0,
                                       pos.numpy()[b:b + 1], f64(k_new)[b:b + 1, h:h + 1],
                                       f64(v_new)[b:b + 1, h:h + 1], P64[h:h + 1])
        qg = q64[b, h * G:(h + 1) * G]
        oi, oo, _, sc = oracle.decode_step_unit(qg, K2[0, 0], V2[0, 0], kp2[0, 0], P64[h], N, M,
                                                default_scale(d))
        swaps = check_topm_unit(gi[b, h], sc, M, N)
        _say("  unit", (b, h), "band swaps", swaps)
        assert np.isin(gi[b, h], np.arange(lo, hi)).mean() > 0.9
        if not np.array_equal(gi[b, h], oi):
            oo, _ = oracle.sparse_attention(qg, K2[0, 0], V2[0, 0], gi[b, h], default_scale(d))
        check_attention(go[b, h * G:(h + 1) * G], oo, "clustered unit %s" % ((b, h),))


# ------------------------------------------------------------------ decode step

SELECT_ATTEND_CASES = [
    (2, 8, 2, 128, 32, 8192, 512),     # G d = 512: one launch, then the split merge
    (1, 16, 1, 128, 16, 4096, 256),    # G d = 2048: merge and attention launched apart
    (3, 12, 1, 64, 16, 6000, 700),     # G d = 768, ragged tiles
    (1, 4, 1, 128, 32, 20000, 6144),   # the largest M the merge stages in LDS
]


@pytest.mark.parametrize("B,Hq,Hkv,d,r,N,M,plan", [
    c + (p,) for c in SELECT_ATTEND_CASES for p in ("planned", "filter")
    if p == "planned" or _scores_shape(c[5], c[6])])
def test_select_attend_stage_equals_merge_then_attend(B, Hq, Hkv, d, r, N, M, plan, monkeypatch):
    """SA_STEP_SELECT_ATTEND (the merge workgroups go on to attend over the
    selection they hold) writes the same idx, out and lse, bit for bit, as
    SA_STEP_MERGE followed by SA_STEP_ATTEND; the attention of two units is
    checked against the oracle over the selected rows."""
    _say("case: select+attend", B, Hq, Hkv, d, r, N, M, plan)
    _use_plan(monkeypatch, plan)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=41)
    g = torch.Generator().manual_seed(42)
    k_new = torch.randn(B, Hkv, 1, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, 1, d, generator=g).to(torch.bfloat16)
    pos = torch.full((B,), N - 1, dtype=torch.int32)
    res = []
    for ending in ((sa.SA_STEP_MERGE, sa.SA_STEP_ATTEND), (sa.SA_STEP_SELECT_ATTEND,)):
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        for stage in (sa.SA_STEP_APPEND_BOUND, sa.SA_STEP_CANDIDATES) + ending:
            sa.sparse_attn_decode_step_stage(sh, stage, _dev(pos), _dev(k_new), _dev(v_new),
                                             _dev(q), _dev(P), Kd, Vd, kp, None, N, M,
                                             default_scale(d), idx, out, lse, ws)
        torch.cuda.synchronize()
        res.append((idx, out, lse, Kd, Vd))
    for x, y in zip(res[0][:3], res[1][:3]):
        assert torch.equal(x, y)
    assert _fallbacks(sh, N, M, ws) == 0, "the merge, not the exact pass, must serve these"
    idx, out, _, Kd, Vd = res[1]
    gi = idx.cpu().numpy()
    assert np.all(np.diff(gi, axis=-1) > 0) and gi.min() >= 0 and gi.max() < N
    G = Hq // Hkv
    q64, K64, V64 = f64(q), f64(Kd), f64(Vd)
    for b, h in {(0, 0), (B - 1, Hkv - 1)}:
        o, _ = oracle.sparse_attention(q64[b, h * G:(h + 1) * G], K64[b, h], V64[b, h], gi[b, h],
                                       default_scale(d))
        check_attention(f64(out)[b, h * G:(h + 1) * G], o, "unit (%d, %d)" % (b, h))


@pytest.mark.parametrize("name,N,T,lens,M", [
    ("tiny", None, 1, None, None),
    ("gqa7_16k", 8192, 1, [8192, 5000, 1, 0, 8192, 300, 8100, 7000], None),
    ("longctx_128k", 16384, 2, None, None),
    # at the filter path's limits (one fused select + attend launch) and past
    # them (chunk-exact selection, then the attention launch)
    ("tiny", 524288, 1, None, 6144),
    ("tiny", 600000, 1, None, 2048),
    ("tiny", 65536, 1, None, 6145),
])
def test_decode_step_equals_the_three_calls(name, N, T, lens, M):
    """sparse_attn_decode_step (fused prologue) writes the same caches, idx,
    out and lse, bit for bit, as append_kv + index_topm + decode."""
    wl = WORKLOADS[name] if N is None else scaled(WORKLOADS[name], N=N, B=min(8, WORKLOADS[name].B))
    if M is not None:
        wl = scaled(wl, M=M)
    _say("case: decode step", wl.name, wl.N, "T=%d" % T)
    sh = _shape_of(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, wl.N)
    res = []
    for fused in (False, True):
        inp = make_decode_inputs(wl, seed=13, device="cuda", seq_lens=lens)
        g = torch.Generator(device="cuda").manual_seed(5)
        k_new = torch.randn(wl.B, wl.Hkv, T, wl.d, generator=g, device="cuda").to(torch.bfloat16)
        v_new = torch.randn(wl.B, wl.Hkv, T, wl.d, generator=g, device="cuda").to(torch.bfloat16)
        pos = (inp.seq_lens - T).clamp(min=0).to(torch.int32)
        kp = torch.empty(wl.B, wl.Hkv, wl.N, wl.r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, inp.k_cache, inp.P, 0, wl.N, kp)
        if not fused:        # the generator's rows of the units the oracle checks
            picks = sorted({(0, 0), (wl.B - 1, wl.Hkv - 1)})
            saved = {(b, h): (f64(inp.k_cache[b, h]), f64(inp.v_cache[b, h])) for b, h in picks}
            host = (f64(inp.q), inp.P.double().cpu().numpy(), inp.seq_lens.cpu().numpy(),
                    pos.cpu().numpy(), f64(k_new), f64(v_new))
        ws = sa.alloc_workspace(sh, wl.N, wl.M)
        idx = torch.full((wl.B, wl.Hkv, wl.M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(wl.B, wl.Hq, wl.d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(wl.B, wl.Hq, dtype=torch.float32, device="cuda")
        scale = default_scale(wl.d)
        if fused:
            sa.sparse_attn_decode_step(sh, pos, k_new, v_new, inp.q, inp.P, inp.k_cache,
                                       inp.v_cache, kp, inp.seq_lens, wl.N, wl.M, scale, idx, out,
                                       lse, ws)
        else:
            sa.sparse_attn_append_kv(sh, pos, k_new, v_new, inp.P, inp.k_cache, inp.v_cache, kp)
            sa.sparse_attn_index_topm(sh, inp.q, inp.P, kp, inp.seq_lens, wl.N, wl.M, idx, ws)
            sa.sparse_attn_decode(sh, inp.q, inp.k_cache, inp.v_cache, idx, wl.M, scale, out,
                                  lse, ws)
        torch.cuda.synchronize()
        res.append((inp.k_cache.clone(), inp.v_cache.clone(), kp, idx, out, lse))
        del inp
    for x, y in zip(res[0], res[1]):
        assert torch.equal(x, y)
    # and the oracle, on the first and last unit
    q64, P64, lens_h, pos_h, kn, vn = host
    gi, go = res[1][3].cpu().numpy(), f64(res[1][4])
    G = wl.G
    for b, h in picks:
        K0, V0 = saved[(b, h)]
        L = int(lens_h[b])
        if L == 0:
            continue
        kp0 = oracle.project_keys(K0, P64[h])[None, None]
        K2, V2, kp2 = oracle.append_kv(K0[None, None], V0[None, None], kp0, pos_h[b:b + 1],
                                       kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], P64[h:h + 1])
        qg = q64[b, h * G:(h + 1) * G]
        oi, oo, _, s = oracle.decode_step_unit(qg, K2[0, 0], V2[0, 0], kp2[0, 0], P64[h], L,
                                               wl.M, default_scale(wl.d))
        swaps = check_topm_unit(gi[b, h], s, wl.M, L)
        _say("  unit", (b, h), "band swaps", swaps)
        if not np.array_equal(gi[b, h], oi):
            oo, _ = oracle.sparse_attention(qg, K2[0, 0], V2[0, 0], gi[b, h],
                                            default_scale(wl.d))
        check_attention(go[b, h * G:(h + 1) * G], oo, "unit %s" % ((b, h),))


# ------------------------------------------------------------------ one workgroup per unit

UNIT_CASES = [
    # (B, Hq, Hkv, d, r, N, M, seq_lens[, T]): 256 units each, so the units
    # fill the chip's 256 compute units and the decode step runs one workgroup
    # per unit; T new rows per batch row (1 unless given)
    (32, 32, 8, 128, 32, 8192, 1024, None),
    (16, 128, 16, 64, 16, 5000, 700, "ragged"),       # G = 8, d = 64, short and empty rows
    (64, 16, 4, 128, 32, 4096, 2048, None),           # M at the plan's limit
    # three new rows per unit, some of them inside the chunks the streaming
    # waves load before the bound is known (rows below 2048)
    (32, 32, 8, 128, 32, 8192, 1024, "ragged", 3),
]


def _unit_inputs(B, Hq, Hkv, d, r, N, seed):
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=seed)
    G = Hq // Hkv
    qbar = f64(q).reshape(B, Hkv, G, d).mean(axis=2)
    rng = np.random.default_rng(seed)
    K64 = f64(K)
    for b in range(B):
        for h in range(Hkv):
            rows = rng.choice(N, size=max(1, N // 100), replace=False)
            K64[b, h, rows] += 2.0 * qbar[b, h]
    # a run of high scores in two units: their wave lists fill and spill
    K64[0, 0, 1000:2500] += 3.0 * qbar[0, 0]
    K64[B - 1, Hkv - 1, 100:3100] += 3.0 * qbar[B - 1, Hkv - 1]
    return q, torch.from_numpy(K64).to(torch.bfloat16), V, P


@pytest.mark.parametrize("case", UNIT_CASES)
def test_unit_workgroup_plan_equals_chunked_plan(case, monkeypatch):
    """The one-workgroup-per-unit plan (stream, merge over LDS wave lists and
    attend in one launch) writes the same caches, idx, out and lse, bit for
    bit, as the chunked filter plan (SPARSE_ATTN_UNIT_WG=0), for the whole
    step and for the selection alone; the oracle checks three units."""
    B, Hq, Hkv, d, r, N, M, lens = case[:8]
    T = case[8] if len(case) > 8 else 1
    _say("case: unit plan", case)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    G = Hq // Hkv
    q, K, V, P = _unit_inputs(B, Hq, Hkv, d, r, N, seed=B + Hkv + T - 1)
    if lens == "ragged":
        lens = [N, 0, 700, 1, N - 3, 2000] + [N] * (B - 6)
    sl = None if lens is None else _dev(torch.tensor(lens, dtype=torch.int32))
    g = torch.Generator().manual_seed(3)
    k_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    Ls = [N if lens is None else lens[b] for b in range(B)]
    pos = torch.tensor([max(L - T, 0) for L in Ls], dtype=torch.int32)
    res, plans = {}, {}
    for flag in ("1", "0"):
        monkeypatch.setenv("SPARSE_ATTN_UNIT_WG", flag)
        monkeypatch.setenv("SPARSE_ATTN_SCORES_PLAN", flag)   # "0": the sampled-bound filter
        plans[flag] = sa.sparse_attn_selection_plan(sh, N, M)
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        for stage in (sa.SA_STEP_APPEND_BOUND, sa.SA_STEP_CANDIDATES, sa.SA_STEP_SELECT_ATTEND):
            sa.sparse_attn_decode_step_stage(sh, stage, _dev(pos), _dev(k_new), _dev(v_new),
                                             _dev(q), _dev(P), Kd, Vd, kp, sl, N, M,
                                             default_scale(d), idx, out, lse, ws)
        fb = _fallbacks(sh, N, M, ws)
        idx2 = torch.full_like(idx, -9)
        sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), kp, sl, N, M, idx2, ws)
        torch.cuda.synchronize()
        res[flag] = (Kd, Vd, kp, idx, out, lse, idx2)
        assert fb == 0, (flag, fb)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert plans["1"] == sa.SA_PLAN_UNIT, plans
    assert plans["0"] == sa.SA_PLAN_FILTER, plans
    for name, x, y in zip(("k", "v", "kp", "idx", "out", "lse", "idx_topm"), res["1"], res["0"]):
        assert torch.equal(x, y), name
    Kd, Vd, kp, idx, out, lse, idx2 = res["1"]
    assert torch.equal(idx, idx2)
    gi, go = idx.cpu().numpy(), f64(out)
    q64, P64, K64, V64 = f64(q), P.double().numpy(), f64(K), f64(V)
    for b, h in sorted({(0, 0), (B - 1, Hkv - 1), (min(2, B - 1), 1 % Hkv)}):
        L = Ls[b]
        # the oracle's own caches of the unit: its projection of the rows,
        # then its append of the new token
        kp0 = oracle.project_keys(K64[b, h], P64[h])[None, None]
        K2, V2, kp2 = oracle.append_kv(K64[b, h][None, None], V64[b, h][None, None], kp0,
                                       pos.numpy()[b:b + 1], f64(k_new)[b:b + 1, h:h + 1],
                                       f64(v_new)[b:b + 1, h:h + 1], P64[h:h + 1])
        qg = q64[b, h * G:(h + 1) * G]
        oi, oo, _, sc = oracle.decode_step_unit(qg, K2[0, 0], V2[0, 0], kp2[0, 0], P64[h], L, M,
                                                default_scale(d))
        swaps = check_topm_unit(gi[b, h], sc, M, L)
        _say("  unit", (b, h), "L", L, "band swaps", swaps)
        if not np.array_equal(gi[b, h], oi):
            oo, _ = oracle.sparse_attention(qg, K2[0, 0], V2[0, 0], gi[b, h], default_scale(d))
        check_attention(go[b, h * G:(h + 1) * G], oo, "unit plan %s" % ((b, h),))


def test_unit_workgroup_plan_falls_back_exactly():
    """All scores equal in one unit of a unit-plan shape: its wave lists fill,
    the spill pool runs out, and the workgroup selects exactly by streaming
    the unit again (the lowest positions); the other units are unaffected."""
    _say("case: unit plan, exact fallback")
    B, Hq, Hkv, d, r, N, M = 32, 32, 8, 64, 16, 32768, 512
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=51)
    P64 = P.double().numpy()
    kp = oracle_kp(f64(K), P64)
    kp[3, 5] = 0x38                                       # every code 1.0 in unit (3, 5)
    ws = sa.alloc_workspace(sh, N, M)
    idx = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), _dev(kp), None, N, M, idx, ws)
    fb = _fallbacks(sh, N, M, ws)
    gi = idx.cpu().numpy()
    G = Hq // Hkv
    assert fb == 1, fb
    for b, h in ((3, 5), (0, 0), (B - 1, Hkv - 1)):
        qt = oracle.indexer_query(f64(q)[b, h * G:(h + 1) * G], P64[h])
        s = oracle.index_scores(qt, kp[b, h])
        check_topm_unit(gi[b, h], s, M, N)
    # unit (3, 5): every score equal, so the M lowest positions
    assert gi[3, 5].tolist() == list(range(M))


@pytest.mark.parametrize("d,r", [(128, 32), (64, 16)])
def test_unit_workgroup_step_scores_the_new_token(d, r):
    """With one workgroup per unit the append, the bound and the stream share
    one launch: the stream must score the codes the append just wrote, not
    what the row held before.  Each unit's new token is k_new = 5 qbar (far
    above every cached row's score) over a cached row that scores low, so it
    must be selected (and first, being the largest); the step must equal the
    three separate calls bit for bit."""
    B, Hq, Hkv, N, M = 32, 32, 8, 4096, 256
    _say("case: unit plan appends and scores the new token d=%d r=%d" % (d, r))
    G = Hq // Hkv
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=61)
    qbar = f64(q).reshape(B, Hkv, G, d).mean(axis=2)
    K64 = f64(K)
    K64[:, :, N - 1] = -3.0 * qbar                          # the row before the append: low
    K = torch.from_numpy(K64).to(torch.bfloat16)
    k_new = torch.from_numpy(5.0 * qbar[:, :, None, :]).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, 1, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    pos = torch.full((B,), N - 1, dtype=torch.int32)
    res = []
    for fused in (True, False):
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        if fused:
            sa.sparse_attn_decode_step(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(q), _dev(P),
                                       Kd, Vd, kp, None, N, M, default_scale(d), idx, out, lse, ws)
        else:
            sa.sparse_attn_append_kv(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(P), Kd, Vd, kp)
            sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), kp, None, N, M, idx, ws)
            sa.sparse_attn_decode(sh, _dev(q), Kd, Vd, idx, M, default_scale(d), out, lse, ws)
        torch.cuda.synchronize()
        res.append((Kd, Vd, kp, idx, out, lse))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert sa.sparse_attn_selection_plan(sh, N, M) == sa.SA_PLAN_UNIT
    for name, x, y in zip(("k", "v", "kp", "idx", "out", "lse"), res[0], res[1]):
        assert torch.equal(x, y), name
    gi = res[0][3].cpu().numpy()
    assert np.all(gi[:, :, -1] == N - 1), "the new token must be selected in every unit"


# ------------------------------------------------------------------ every position scored

SCORES_CASES = [
    # (B, Hq, Hkv, d, r, N, M, T, seq_lens): few units, short enough that every
    # position is scored and the merge selects over all of a unit's scores
    (8, 28, 4, 128, 32, 16384, 2048, 1, None),              # the 16K GQA workload's shape
    (3, 8, 2, 128, 32, 6000, 512, 3, [6000, 300, 2049]),    # new rows across a chunk edge; len <= M
    (2, 8, 2, 64, 16, 16384, 1, 1, [16384, 9000]),          # d = 64, M = 1
    (1, 4, 1, 128, 32, 3000, 2999, 1, None),                # M = n_max - 1
    (2, 12, 2, 128, 16, 5000, 700, 2, [0, 1]),              # an empty unit, a unit of one row
    # more new rows in a chunk than are scored from their codes in LDS: the
    # chunk's code loads wait for the rows' stores instead
    (2, 8, 2, 128, 32, 6000, 512, 20, [6000, 2100]),
]


@pytest.mark.parametrize("case", SCORES_CASES)
def test_scores_plan_equals_filter_plan(case, monkeypatch):
    """The plan that scores every position (the scores written out, then an
    exact merge over all of a unit's scores with the attention in the merge
    launch) writes the same caches, idx, out and lse, bit for bit, as the
    sampled-bound filter plan (SPARSE_ATTN_SCORES_PLAN=0): through the staged
    decode step, the staged fused selection and sparse_attn_topm over the
    scores sparse_attn_index_score writes; the oracle checks three units."""
    B, Hq, Hkv, d, r, N, M, T, lens = case
    _say("case: scores plan", case)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    G = Hq // Hkv
    q, K, V, P = _unit_inputs(B, Hq, Hkv, d, r, N, seed=B + Hkv + T)
    sl = None if lens is None else _dev(torch.tensor(lens, dtype=torch.int32))
    Ls = [N if lens is None else lens[b] for b in range(B)]
    g = torch.Generator().manual_seed(7)
    k_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([max(L - T, 0) for L in Ls], dtype=torch.int32)
    scale = default_scale(d)
    res, plans = {}, {}
    for flag in ("1", "0"):
        monkeypatch.setenv("SPARSE_ATTN_SCORES_PLAN", flag)
        plans[flag] = sa.sparse_attn_selection_plan(sh, N, M)
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        for stage in (sa.SA_STEP_APPEND_BOUND, sa.SA_STEP_CANDIDATES, sa.SA_STEP_SELECT_ATTEND):
            sa.sparse_attn_decode_step_stage(sh, stage, _dev(pos), _dev(k_new), _dev(v_new),
                                             _dev(q), _dev(P), Kd, Vd, kp, sl, N, M, scale, idx,
                                             out, lse, ws)
        fb = _fallbacks(sh, N, M, ws)
        idx2 = torch.full_like(idx, -9)
        for stage in (sa.SA_STAGE_BOUND, sa.SA_STAGE_CANDIDATES, sa.SA_STAGE_MERGE):
            sa.sparse_attn_index_topm_stage(sh, stage, _dev(q), _dev(P), kp, sl, N, M, idx2, ws)
        scores = torch.empty(B, Hkv, N, dtype=torch.float32, device="cuda")
        sa.sparse_attn_index_score(sh, _dev(q), _dev(P), kp, sl, N, scores)
        idx3 = torch.full_like(idx, -9)
        sa.sparse_attn_topm(sh, scores, sl, N, M, idx3, ws)
        torch.cuda.synchronize()
        res[flag] = (Kd, Vd, kp, idx, out, lse, idx2, idx3)
        if flag == "1":
            assert fb == 0, fb                                # no bound, so no fallback
    assert plans == {"1": sa.SA_PLAN_SCORES, "0": sa.SA_PLAN_FILTER}, plans
    names = ("k", "v", "kp", "idx", "out", "lse", "idx_topm_stages", "idx_topm_scores")
    for name, x, y in zip(names, res["1"], res["0"]):
        assert torch.equal(x, y), name
    Kd, Vd, kp, idx, out, lse, idx2, idx3 = res["1"]
    assert torch.equal(idx, idx2) and torch.equal(idx, idx3)
    gi, go = idx.cpu().numpy(), f64(out)
    q64, P64, K64, V64 = f64(q), P.double().numpy(), f64(K), f64(V)
    for b, h in sorted({(0, 0), (B - 1, Hkv - 1), (min(2, B - 1), 1 % Hkv)}):
        L = Ls[b]
        if L == 0:
            assert np.all(gi[b, h] == -1)
            continue
        kp0 = oracle.project_keys(K64[b, h], P64[h])[None, None]
        K2, V2, kp2 = oracle.append_kv(K64[b, h][None, None], V64[b, h][None, None], kp0,
                                       pos.numpy()[b:b + 1], f64(k_new)[b:b + 1, h:h + 1],
                                       f64(v_new)[b:b + 1, h:h + 1], P64[h:h + 1])
        qg = q64[b, h * G:(h + 1) * G]
        oi, oo, _, sc = oracle.decode_step_unit(qg, K2[0, 0], V2[0, 0], kp2[0, 0], P64[h], L, M,
                                                scale)
        swaps = check_topm_unit(gi[b, h], sc, M, L)
        _say("  unit", (b, h), "L", L, "band swaps", swaps)
        if not np.array_equal(gi[b, h], oi):
            oo, _ = oracle.sparse_attention(qg, K2[0, 0], V2[0, 0], gi[b, h], scale)
        check_attention(go[b, h * G:(h + 1) * G], oo, "scores plan %s" % ((b, h),))


def test_scores_plan_all_equal_takes_lowest_positions():
    """Every score of one unit equal (every code 1.0) under the plan that
    scores every position: the merge's threshold is that score and the tie
    goes to the M lowest positions; a unit of random scores beside it is
    checked against the oracle's top-M."""
    _say("case: scores plan, all equal")
    B, Hq, Hkv, d, r, N, M = 1, 8, 2, 64, 16, 16384, 1000
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=61)
    P64 = P.double().numpy()
    kp = oracle_kp(f64(K), P64)
    kp[0, 1] = 0x38
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    assert sa.sparse_attn_selection_plan(sh, N, M) == sa.SA_PLAN_SCORES
    ws = sa.alloc_workspace(sh, N, M)
    idx = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
    sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), _dev(kp), None, N, M, idx, ws)
    gi = idx.cpu().numpy()
    assert _fallbacks(sh, N, M, ws) == 0
    assert gi[0, 1].tolist() == list(range(M))
    G = Hq // Hkv
    qt = oracle.indexer_query(f64(q)[0, 0:G], P64[0])
    check_topm_unit(gi[0, 0], oracle.index_scores(qt, kp[0, 0]), M, N)


def _sweep_shapes(n, seed=97):
    """Seeded small shapes across the plans' parameters: batch, KV heads,
    group size, head dim, rank, context, budget, new rows and ragged rows."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B = int(rng.choice([1, 2, 3, 5]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 4, 7, 8]))
        d = int(rng.choice([64, 128]))
        r = int(rng.choice([16, 32]))
        N = int(rng.choice([700, 2049, 5000, 12288, 16384, 20000]))
        M = int(rng.choice([1, 64, 777, 2048]))
        T = int(rng.choice([1, 2, 3]))
        if M >= N:
            continue
        lens = [int(N if rng.random() < 0.5 else rng.integers(0, N + 1)) for _ in range(B)]
        out.append((B, G * Hkv, Hkv, d, r, N, M, T, lens))
    return out


@pytest.mark.parametrize("case", _sweep_shapes(12))
def test_plans_agree_across_a_shape_sweep(case, monkeypatch):
    """Seeded shapes across the selection plans' parameters: the decode step
    as planned, the decode step with the score-all plan turned off, and
    append_kv + index_topm + decode write the same caches, idx, out and lse,
    bit for bit; idx is ascending, in range and -1 padded in every unit; the
    oracle checks the last unit's selection and attention."""
    B, Hq, Hkv, d, r, N, M, T, lens = case
    _say("case: sweep", case)
    G = Hq // Hkv
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    q, K, V, P = _rand_inputs(B, Hq, Hkv, d, r, N, seed=B * 131 + N + M)
    g = torch.Generator().manual_seed(N + T)
    k_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, T, d, generator=g).to(torch.bfloat16)
    pos = torch.tensor([max(L - T, 0) for L in lens], dtype=torch.int32)
    sl = _dev(torch.tensor(lens, dtype=torch.int32))
    scale = default_scale(d)
    res = []
    for mode in ("planned", "filter", "calls"):
        monkeypatch.setenv("SPARSE_ATTN_SCORES_PLAN", "0" if mode == "filter" else "1")
        Kd, Vd = _dev(K), _dev(V)
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, Kd, _dev(P), 0, N, kp)
        ws = sa.alloc_workspace(sh, N, M)
        idx = torch.full((B, Hkv, M), -9, dtype=torch.int32, device="cuda")
        out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        if mode == "calls":
            sa.sparse_attn_append_kv(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(P), Kd, Vd, kp)
            sa.sparse_attn_index_topm(sh, _dev(q), _dev(P), kp, sl, N, M, idx, ws)
            sa.sparse_attn_decode(sh, _dev(q), Kd, Vd, idx, M, scale, out, lse, ws)
        else:
            sa.sparse_attn_decode_step(sh, _dev(pos), _dev(k_new), _dev(v_new), _dev(q), _dev(P),
                                       Kd, Vd, kp, sl, N, M, scale, idx, out, lse, ws)
        torch.cuda.synchronize()
        res.append((Kd, Vd, kp, idx, out, lse))
    for other in res[1:]:
        for name, x, y in zip(("k", "v", "kp", "idx", "out", "lse"), res[0], other):
            assert torch.equal(x, y), name
    gi, go = res[0][3].cpu().numpy(), f64(res[0][4])
    for b in range(B):
        n_sel = min(lens[b], M)
        for h in range(Hkv):
            row = gi[b, h]
            assert np.all(row[n_sel:] == -1) and np.all(np.diff(row[:n_sel]) > 0), (b, h)
            assert n_sel == 0 or (row[0] >= 0 and row[n_sel - 1] < lens[b]), (b, h)
    b, h = B - 1, Hkv - 1
    L = lens[b]
    if L == 0:
        return
    P64 = P.double().numpy()
    kp0 = oracle.project_keys(f64(K)[b, h], P64[h])[None, None]
    K2, V2, kp2 = oracle.append_kv(f64(K)[b, h][None, None], f64(V)[b, h][None, None], kp0,
                                   pos.numpy()[b:b + 1], f64(k_new)[b:b + 1, h:h + 1],
                                   f64(v_new)[b:b + 1, h:h + 1], P64[h:h + 1])
    qg = f64(q)[b, h * G:(h + 1) * G]
    oi, oo, _, sc = oracle.decode_step_unit(qg, K2[0, 0], V2[0, 0], kp2[0, 0], P64[h], L, M,
                                            scale)
    swaps = check_topm_unit(gi[b, h], sc, M, L)
    _say("  unit", (b, h), "L", L, "band swaps", swaps)
    if not np.array_equal(gi[b, h], oi):
        oo, _ = oracle.sparse_attention(qg, K2[0, 0], V2[0, 0], gi[b, h], scale)
    check_attention(go[b, h * G:(h + 1) * G], oo, "sweep unit %s" % ((b, h),))


def _order_key(x):
    """The order-preserving unsigned key of float32 values (IEEE bits, sign
    flipped for positives, all bits flipped for negatives)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    return np.where(b >> 31, 0xFFFFFFFF - b, b | 0x80000000)


def test_unit_plan_candidates_far_above_the_sample():
    """Candidates over a huge range under one workgroup per unit: rows planted
    between the sampled blocks (codes of magnitude 448 with the query's signs)
    score far above every sampled row, so the merge's first radix level, spread
    over the candidates' range, puts every ordinary candidate into a few
    bins.  In unit (0, 0) 1500 equal planted rows: the M-th key is theirs and
    ties cut it; in (0, 1) 1500 rows of graded scores; in (0, 2) 500 rows, all
    selected, and the M-th key is an ordinary one among the crowded low bins.
    Every unit's selection is the oracle's."""
    _say("case: unit plan, candidates far above the sample")
    B, Hq, Hkv, d, r, N, M = 32, 32, 8, 128, 32, 16384, 1024
    G = Hq // Hkv
    g = torch.Generator().manual_seed(71)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    P = torch.from_numpy(np.stack([orthonormal_basis(d, r, 71 * 31 + h)
                                   for h in range(Hkv)]).astype(np.float32))
    rng = np.random.default_rng(71)
    # codes of magnitude below 2, either sign (no NaN codes)
    kp = (rng.integers(0, 0x40, size=(B, Hkv, N, r)) |
          (rng.integers(0, 2, size=(B, Hkv, N, r)) << 7)).astype(np.uint8)
    starts = [(j * (N - 8)) // 127 for j in range(128)]
    sampled = np.zeros(N, dtype=bool)
    for s0 in starts:
        sampled[s0:s0 + 8] = True
    gaps = np.flatnonzero(~sampled)
    P64 = P.double().numpy()
    plants = {(0, 0): (1500, False), (0, 1): (1500, True), (0, 2): (500, False)}
    for (b, h), (n_rows, graded) in plants.items():
        qt = oracle.indexer_query(f64(q)[b, h * G:(h + 1) * G], P64[h])
        sign = np.where(qt < 0, 0x80, 0).astype(np.uint8)
        rows = gaps[:n_rows]
        mag = np.full(n_rows, 0x7E, dtype=np.uint8)            # 448
        if graded:
            mag = (0x70 + rng.integers(0, 15, size=n_rows)).astype(np.uint8)   # 128 .. 448
        kp[b, h, rows] = mag[:, None] | sign[None, :]
        # the recipe does what it is for: the bound is the k-th largest of the
        # 1024 sampled keys (k = 3 M 1024 / N, rounded up: 192), and every
        # planted key lies more than four times the range from the bound to
        # the largest sampled key above the bound (order-preserving keys)
        s = oracle.index_scores(qt, kp[b, h])
        ks = _order_key(s.astype(np.float32))
        top = np.sort(ks[sampled])[::-1]
        thr, smax = top[-(-3 * M * 1024 // N) - 1], top[0]
        assert ks[rows].min() - thr > 4 * (smax - thr), (b, h)
    sh = _shape_of(B, Hq, Hkv, d, r, N)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert sa.sparse_attn_selection_plan(sh, N, M) == sa.SA_PLAN_UNIT
    gi = _topm_check_against_oracle(q, P, kp, M, N)
    assert _topm_check_against_oracle.fallbacks == 0
    assert gi[0, 0].tolist() == gaps[:M].tolist()              # ties: the lowest positions
    assert set(gaps[:500].tolist()) <= set(gi[0, 2].tolist())
