"""Pins of the oracle's decode step against things other than itself.

Each test ties a function of ``oracle/jssa.py`` to a hand-derived example
(``tests/golden``), a library routine computing a special case, brute force on
tiny inputs, or an identity of the mathematics, so that a dropped term, a wrong
sign or index, or a transposed operand fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import (project_keys, append_kv, indexer_query, index_scores, top_m,
                    sparse_attention, dense_attention, decode_step_unit, decode_step,
                    reuse_source_layer, elu_plus_one, linear_state, linear_gate,
                    fp8_encode, fp8_decode, decode_table)
from workloads import WORKLOADS, make_decode_inputs, bf16_to_f64, default_scale

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ev(x):
    if isinstance(x, str):
        return eval(x, {"__builtins__": {}}, {"e": math.e, "log": math.log,
                                              "exp": math.exp})
    return float(x)


def _arr(rows):
    return np.array([[_ev(v) for v in row] for row in rows], dtype=np.float64)


# ---------------------------------------------------------------- hand examples

def test_hand_example_decode_step():
    ex = _load("hand_examples.json")["decode_step"]
    P = np.array(ex["P"], dtype=np.float64)
    K = np.array(ex["K"], dtype=np.float64)
    V = np.array(ex["V"], dtype=np.float64)
    q = np.array(ex["q"], dtype=np.float64)
    kp = project_keys(K, P)
    assert kp.tolist() == ex["expect_kP"]
    qt = indexer_query(q, P)
    assert qt.tolist() == ex["expect_q_tilde"]
    s = index_scores(qt, kp)
    assert s.tolist() == ex["expect_scores"]
    assert top_m(s, 2).tolist() == ex["expect_idx_M2"]
    assert top_m(s, 3).tolist() == ex["expect_idx_M3"]
    assert top_m(s, 8).tolist() == ex["expect_idx_M8"]
    idx, out, lse, s2 = decode_step_unit(q, K, V, kp, P, ex["N"], 2, ex["scale"])
    assert idx.tolist() == ex["expect_idx_M2"]
    np.testing.assert_allclose(out, _arr(ex["expect_out_M2"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, [_ev(v) for v in ex["expect_lse_M2"]], rtol=0,
                               atol=1e-14)


def _check_batched_golden(step_fn):
    """Run a decode_step implementation on the batched hand example; raise
    AssertionError on any difference from the hand-derived values."""
    ex = _load("hand_examples.json")["decode_step_batched"]
    K = np.array(ex["K"], dtype=np.float64)
    V = np.array(ex["V"], dtype=np.float64)
    q = np.array(ex["q"], dtype=np.float64)
    P = np.array(ex["P"], dtype=np.float64)
    kp = np.stack([np.stack([project_keys(K[b, h], P[h]) for h in range(ex["Hkv"])])
                   for b in range(ex["B"])])
    idx, out, lse = step_fn(q, K, V, kp, P, ex["seq_lens"], ex["M"], ex["scale"])
    assert idx.tolist() == ex["expect_idx"]
    want_out = np.array([[[_ev(v) for v in row] for row in rows] for rows in ex["expect_out"]])
    want_lse = np.array([[_ev(v) for v in row] for row in ex["expect_lse"]])
    np.testing.assert_allclose(out, want_out, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-13, atol=1e-13)


def test_hand_example_batched_decode_step():
    """Two batch rows of different valid lengths, two KV heads with groups of
    three query heads: every head's output is its own group's selection (see
    tests/golden/README.md for the derivation)."""
    _check_batched_golden(decode_step)


def _mutant(find, replace):
    """oracle.decode_step with one planted mistake (source text substituted)."""
    import inspect
    from oracle import jssa
    src = inspect.getsource(jssa.decode_step)
    assert find in src, find
    ns = dict(vars(jssa))
    exec(compile(src.replace(find, replace), "<mutant>", "exec"), ns)
    return ns["decode_step"]


@pytest.mark.parametrize("find,replace", [
    # query head hq read as belonging to KV head hq % Hkv instead of hq // G
    ("qg = q[b, h * G:(h + 1) * G]", "qg = q[b, h::Hkv]"),
    # every batch row scored over all cached rows instead of its own length
    ("int(seq_lens[b])", "k_cache.shape[2]"),
    # outputs written to the wrong query heads
    ("out[b, h * G:(h + 1) * G] = o", "out[b, h::Hkv] = o"),
])
def test_batched_golden_catches_planted_mistakes(find, replace):
    with pytest.raises(AssertionError):
        _check_batched_golden(_mutant(find, replace))


def test_hand_example_linear_gate():
    ex = _load("hand_examples.json")["linear_gate"]
    K = np.array(ex["K"], dtype=np.float64)
    V = np.array(ex["V"], dtype=np.float64)
    S, z = linear_state(K, V)
    assert S.tolist() == ex["expect_S"]
    assert z.tolist() == ex["expect_z"]
    out, o_lin, g = linear_gate(np.array(ex["q"], dtype=np.float64), S, z,
                                _arr(ex["w"]), np.array(ex["o_sparse"], dtype=np.float64))
    np.testing.assert_allclose(o_lin, ex["expect_o_lin"], atol=1e-15, rtol=0)
    np.testing.assert_allclose(g, ex["expect_g"], atol=1e-15, rtol=0)
    np.testing.assert_allclose(out, ex["expect_out"], atol=1e-15, rtol=0)


def test_fp8_cache_fraction_matches_page():
    fig = _load("page_figures.json")["fp8_cache_fraction_of_bf16_kv_max"]["value"]
    for wl in WORKLOADS.values():
        frac = (wl.r * 1) / (2 * wl.d * 2)      # kP row bytes / (K + V row bytes)
        assert frac <= fig + 1e-15
    wl = WORKLOADS["longctx_128k"]
    assert (wl.r * 1) / (2 * wl.d * 2) == fig


# ---------------------------------------------------------------- projection

def _brute_project(K, P):
    n, d = K.shape
    r = P.shape[1]
    table = decode_table()
    codes = np.zeros((n, r), dtype=np.uint8)
    for i in range(n):
        for j in range(r):
            x = 0.0
            for k in range(d):
                x += float(K[i, k]) * float(P[k, j])
            # nearest code by search, ties to even mantissa
            best = None
            for c in range(256):
                v = table[c]
                if np.isnan(v) or (c >> 7) != (1 if x < 0 else 0):
                    continue
                err = abs(v - x) if abs(x) < 448 else abs(abs(v) - 448.0)
                if best is None or err < best[0] or (err == best[0] and c % 2 == 0):
                    best = (err, c)
            codes[i, j] = best[1]
    return codes


def test_project_keys_identity_basis_reduces_to_codec():
    rng = np.random.default_rng(3)
    K = torch.from_numpy(rng.standard_normal((50, 16)) * 3).to(torch.bfloat16)
    K = K.to(torch.float64).numpy()
    kp = project_keys(K, np.eye(16))
    ref = torch.from_numpy(K).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kp, ref)


def test_project_keys_brute_force_tiny():
    rng = np.random.default_rng(4)
    K = torch.from_numpy(rng.standard_normal((6, 8))).to(torch.bfloat16).double().numpy()
    P = rng.standard_normal((8, 3)).astype(np.float32).astype(np.float64)
    assert np.array_equal(project_keys(K, P), _brute_project(K, P))


def test_project_keys_zero_row_is_plus_zero_code():
    K = np.zeros((1, 4))
    K[0, 0] = -0.0
    P = -np.ones((4, 2))
    assert project_keys(K, P).tolist() == [[0, 0]]


def test_append_writes_rows_and_projection():
    rng = np.random.default_rng(5)
    B, H, Ncap, d, r, T = 2, 2, 10, 8, 4, 3
    kc = rng.standard_normal((B, H, Ncap, d))
    vc = rng.standard_normal((B, H, Ncap, d))
    kp = np.zeros((B, H, Ncap, r), dtype=np.uint8)
    kn = rng.standard_normal((B, H, T, d))
    vn = rng.standard_normal((B, H, T, d))
    P = rng.standard_normal((H, d, r))
    pos = np.array([2, 8])               # second row: rows 8, 9 in range, 10 dropped
    k2, v2, kp2 = append_kv(kc, vc, kp, pos, kn, vn, P)
    assert np.array_equal(k2[0, :, 2:5], kn[0])
    assert np.array_equal(v2[1, :, 8:10], vn[1, :, :2])
    assert np.array_equal(k2[0, :, :2], kc[0, :, :2])
    for h in range(H):
        assert np.array_equal(kp2[0, h, 2:5], _brute_project(kn[0, h], P[h]))
    assert np.array_equal(kp2[1, :, :8], kp[1, :, :8])


# ---------------------------------------------------------------- indexer

def test_indexer_query_linearity_and_identity():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((7, 32))
    P = rng.standard_normal((32, 8))
    proj_then_mean = np.mean([q[g] @ P for g in range(7)], axis=0)
    np.testing.assert_allclose(indexer_query(q, P), proj_then_mean, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(indexer_query(q, np.eye(32)[:, :8]),
                               q.mean(axis=0)[:8], rtol=0, atol=1e-15)


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(20, 5)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    qt = rng.standard_normal(5)
    table = decode_table()
    ref = [sum(qt[j] * table[codes[n, j]] for j in range(5)) for n in range(20)]
    np.testing.assert_allclose(index_scores(qt, codes), ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- top-M

def test_top_m_is_max_sum_subset_with_lowest_positions_on_ties():
    rng = np.random.default_rng(8)
    for trial in range(40):
        n = 8
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        for M in (1, 3, 5):
            best = None
            for sub in itertools.combinations(range(n), M):
                key = (sum(s[list(sub)]), tuple(-i for i in sub))
                if best is None or key > best[0]:
                    best = (key, sub)
            assert top_m(s, M).tolist() == list(best[1]), (s, M)


def test_top_m_invariants_and_padding():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(1000)
    idx = top_m(s, 64)
    assert len(set(idx.tolist())) == 64 and np.all(np.diff(idx) > 0)
    chosen = np.zeros(1000, bool)
    chosen[idx] = True
    assert s[chosen].min() > s[~chosen].max()
    assert top_m(s, 1000).tolist() == list(range(1000))
    short = top_m(s, 64, valid_len=10)
    assert short[:10].tolist() == list(range(10)) and np.all(short[10:] == -1)
    assert np.all(top_m(s, 5, valid_len=0) == -1)


# ---------------------------------------------------------------- attention

def test_sparse_with_all_rows_equals_torch_sdpa():
    rng = np.random.default_rng(10)
    G, N, d = 4, 300, 64
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    scale = 1 / math.sqrt(d)
    out, lse = sparse_attention(q, K, V, np.arange(N), scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :].transpose(1, 2),
        torch.from_numpy(K)[None, None].expand(1, 1, N, d),
        torch.from_numpy(V)[None, None].expand(1, 1, N, d), scale=scale)
    ref = ref.transpose(1, 2)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    z = scale * q @ K.T
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-13)
    o2, l2 = dense_attention(q, K, V, scale)
    np.testing.assert_array_equal(o2, out)


def test_sparse_single_row_is_that_row_and_padding_is_skipped():
    rng = np.random.default_rng(11)
    K = rng.standard_normal((40, 16))
    V = rng.standard_normal((40, 16))
    q = rng.standard_normal((3, 16))
    out, _ = sparse_attention(q, K, V, np.array([17, -1, -1, 40, 99]), 0.25)
    np.testing.assert_array_equal(out, np.repeat(V[17][None], 3, axis=0))
    out0, lse0 = sparse_attention(q, K, V, np.array([-1, -1]), 0.25)
    assert np.all(out0 == 0) and np.all(np.isneginf(lse0))


def test_sparse_order_invariance_and_lse_merge():
    rng = np.random.default_rng(12)
    K = rng.standard_normal((500, 32))
    V = rng.standard_normal((500, 32))
    q = rng.standard_normal((2, 32))
    idx = rng.choice(500, 100, replace=False)
    o1, l1 = sparse_attention(q, K, V, np.sort(idx), 0.2)
    o2, l2 = sparse_attention(q, K, V, idx[::-1], 0.2)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    oa, la = sparse_attention(q, K, V, idx[:37], 0.2)
    ob, lb = sparse_attention(q, K, V, idx[37:], 0.2)
    m = np.maximum(la, lb)
    lm = m + np.log(np.exp(la - m) + np.exp(lb - m))
    om = (np.exp(la - lm)[:, None] * oa + np.exp(lb - lm)[:, None] * ob)
    np.testing.assert_allclose(lm, l1, rtol=1e-13)
    np.testing.assert_allclose(om, o1, rtol=1e-12, atol=1e-13)


def test_decode_step_with_budget_n_equals_dense():
    wl = WORKLOADS["tiny"]
    inp = make_decode_inputs(wl, seed=1)
    q = bf16_to_f64(inp.q)
    K = bf16_to_f64(inp.k_cache)
    V = bf16_to_f64(inp.v_cache)
    P = inp.P.double().numpy()
    kp = np.stack([np.stack([project_keys(K[b, h], P[h]) for h in range(wl.Hkv)])
                   for b in range(wl.B)])
    scale = default_scale(wl.d)
    idx, out, lse = decode_step(q, K, V, kp, P, [wl.N], wl.N, scale)
    assert idx[0, 0].tolist() == list(range(wl.N))
    dense, _ = dense_attention(q[0], K[0, 0], V[0, 0], scale)
    np.testing.assert_allclose(out[0], dense, rtol=1e-12, atol=1e-12)


def test_planted_rows_are_selected_tiny_workload():
    wl = WORKLOADS["tiny"]
    for seed in range(3):
        inp = make_decode_inputs(wl, seed=seed)
        K = bf16_to_f64(inp.k_cache)[0, 0]
        P = inp.P.double().numpy()[0]
        q = bf16_to_f64(inp.q)[0]
        kp = project_keys(K, P)
        idx, _, _, s = decode_step_unit(q, K, bf16_to_f64(inp.v_cache)[0, 0], kp, P,
                                        wl.N, wl.M, default_scale(wl.d))
        assert set(inp.plants[(0, 0)].tolist()) <= set(idx.tolist())


# ---------------------------------------------------------------- reuse, linear

def test_reuse_source_layer():
    assert [reuse_source_layer(l, (0, 4)) for l in range(8)] == [0, 0, 0, 0, 4, 4, 4, 4]
    with pytest.raises(ValueError):
        reuse_source_layer(0, (1,))


def test_elu_plus_one_matches_torch():
    x = np.linspace(-20, 20, 4001)
    # torch forms (exp(x) - 1) + 1, which is exact only to ~1 ulp of 1.0
    ref = (torch.nn.functional.elu(torch.from_numpy(x)) + 1).numpy()
    np.testing.assert_allclose(elu_plus_one(x), ref, rtol=1e-15, atol=2.3e-16)


def test_linear_branch_equals_kernelised_attention_sum():
    rng = np.random.default_rng(13)
    N, d, G = 50, 16, 3
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    q = rng.standard_normal((G, d))
    S, z = linear_state(K, V)
    # recurrence over tokens gives the same state
    S2 = np.zeros((d, d))
    z2 = np.zeros(d)
    for n in range(N):
        f = np.where(K[n] > 0, K[n] + 1, np.exp(np.minimum(K[n], 0)))
        S2 += np.outer(f, V[n])
        z2 += f
    np.testing.assert_allclose(S, S2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, z2, rtol=1e-12)
    w = rng.standard_normal((G, d))
    o_sp = rng.standard_normal((G, d))
    out, o_lin, g = linear_gate(q, S, z, w, o_sp)
    for gi in range(G):
        fq = np.where(q[gi] > 0, q[gi] + 1, np.exp(np.minimum(q[gi], 0)))
        wts = np.array([fq @ np.where(K[n] > 0, K[n] + 1, np.exp(np.minimum(K[n], 0)))
                        for n in range(N)])
        np.testing.assert_allclose(o_lin[gi], (wts[:, None] * V).sum(0) / wts.sum(),
                                   rtol=1e-12)
        assert g[gi] == pytest.approx(scipy.special.expit(w[gi] @ q[gi]), rel=1e-14)
    # gate limits: g -> 1 gives the sparse branch, g -> 0 the linear one
    big = 1e3 * np.sign(q)
    out1, _, g1 = linear_gate(q, S, z, big, o_sp)
    np.testing.assert_allclose(out1, o_sp, rtol=1e-12, atol=1e-12)
    out0, _, g0 = linear_gate(q, S, z, -big, o_sp)
    np.testing.assert_allclose(out0, o_lin, rtol=1e-12, atol=1e-12)


def test_linear_gate_empty_memory_reads_out_zero():
    """With no token added (S = 0, z = 0) the read-out phi(q)^T z is 0; the
    reading defines the linear branch's output as 0 then, so the mix is the
    sparse branch scaled by the gate (scipy's logistic function)."""
    rng = np.random.default_rng(5)
    G, d = 3, 8
    q = rng.standard_normal((G, d))
    w = rng.standard_normal((G, d))
    o_sp = rng.standard_normal((G, d))
    out, o_lin, g = linear_gate(q, np.zeros((d, d)), np.zeros(d), w, o_sp)
    assert np.all(o_lin == 0.0) and np.all(np.isfinite(out))
    gate = scipy.special.expit(np.sum(w * q, axis=1))
    np.testing.assert_allclose(out, gate[:, None] * o_sp, rtol=1e-14, atol=0)
