"""The decode step, written out plainly in float64.

Test infrastructure only (see the package docstring).

Notation: B batch, Hq query heads, Hkv KV heads, G = Hq / Hkv query heads per
KV head (GQA group), d head dim, r indexer rank, N valid cached positions,
Ncap cache rows, M selection budget.  Query head hq belongs to KV head
hq // G.  Key/value/query inputs are bf16 values carried as float64.

Readings taken where the pages leave a step open are marked "Reading:".
"""

import numpy as np

from .fp8_e4m3 import fp8_decode, fp8_encode


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Projected-key cache
# --------------------------------------------------------------------------

def project_keys(K, P):
    """FP8 projected keys ``e4m3(K @ P)`` for key rows ``K [..., d]``.

    JSSA article, "How JSSA preserves token order": every key has a low-rank
    projection onto its KV head's basis (d x r), and those projections are kept
    in an FP8 cache next to the bf16 KV cache.  The projection only steers the
    candidate search.

    Reading: no scale factor; the dot product is formed in float64 from the
    bf16 keys and fp32 basis (every product is exact there) and rounded once
    to FP8.  The sum starts from +0, so a zero projection encodes as 0x00.
    """
    x = 0.0 + _f64(K) @ _f64(P)
    return fp8_encode(x)


def append_kv(k_cache, v_cache, kp_cache, pos, k_new, v_new, P):
    """Write T new tokens per batch row into the caches (returns new arrays).

    k_cache, v_cache: [B, Hkv, Ncap, d]; kp_cache: [B, Hkv, Ncap, r] uint8;
    pos: [B] first row to write; k_new, v_new: [B, Hkv, T, d]; P: [Hkv, d, r].
    Row pos[b] + t receives token t; its FP8 projection is ``project_keys``.
    Rows outside [0, Ncap) are dropped (reading: the cache never grows here).
    """
    k_cache = _f64(k_cache).copy()
    v_cache = _f64(v_cache).copy()
    kp_cache = np.asarray(kp_cache, dtype=np.uint8).copy()
    k_new = _f64(k_new)
    v_new = _f64(v_new)
    B, Hkv, Ncap, _ = k_cache.shape
    T = k_new.shape[2]
    for b in range(B):
        for t in range(T):
            n = int(pos[b]) + t
            if n < 0 or n >= Ncap:
                continue
            for h in range(Hkv):
                k_cache[b, h, n] = k_new[b, h, t]
                v_cache[b, h, n] = v_new[b, h, t]
                kp_cache[b, h, n] = project_keys(k_new[b, h, t][None, :], P[h])[0]
    return k_cache, v_cache, kp_cache


# --------------------------------------------------------------------------
# Indexer: query, scores, top-M
# --------------------------------------------------------------------------

def indexer_query(q_group, P_h):
    """Indexer query of one KV head: the group's queries averaged, then projected.

    JSSA article, "How JSSA preserves token order": at decode time the queries
    tied to one KV head are averaged and projected before scoring.
    q_group: [G, d]; P_h: [d, r] -> [r].
    """
    q_bar = _f64(q_group).mean(axis=0)
    return q_bar @ _f64(P_h)


def index_scores(q_tilde, kp_codes):
    """Score of every position: ``s[n] = sum_j q_tilde[j] * dec(kP[n, j])``.

    JSSA article, "How JSSA preserves token order": the projected query is
    compared with every cached position's projected key.
    Reading: a plain dot product, no scale or nonlinearity (ranking does not
    depend on a positive scale, and the article names no other transform).
    """
    return fp8_decode(kp_codes) @ _f64(q_tilde)


def top_m(scores, M, valid_len=None):
    """Indices of the M highest scores among positions ``n < valid_len``.

    IndexCache article, "DeepSeek Sparse Attention": the indexer keeps the top-k
    positions; LISA names the budget M.  JSSA article: each KV head keeps its
    own set.
    Readings: equal scores are ordered by lower position first; the result is
    sorted ascending; with fewer than M valid positions every valid position is
    returned and the rest of the M slots hold -1.
    """
    s = _f64(scores)
    n_all = s.shape[0]
    L = n_all if valid_len is None else max(0, min(int(valid_len), n_all))
    s = s[:L]
    pos = np.arange(L)
    order = np.lexsort((pos, -s))          # primary key: -score; then position
    chosen = np.sort(order[: min(M, L)])
    out = np.full(M, -1, dtype=np.int32)
    out[: chosen.shape[0]] = chosen
    return out


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def sparse_attention(q_group, K_unit, V_unit, idx, scale):
    """Exact softmax attention of each query over the rows listed in ``idx``.

    JSSA article, "How JSSA preserves token order": after selection the final
    attention uses the original full-size keys and values, read in place; each
    KV head has its own index set.
    q_group: [G, d]; K_unit, V_unit: [Ncap, d]; idx: [M] (entries < 0 or
    >= Ncap are padding and skipped).  Returns out [G, d] and the natural-log
    log-sum-exp [G] of the scaled logits.  With no valid entry: out = 0,
    lse = -inf.
    """
    q = _f64(q_group)
    K_unit = _f64(K_unit)
    V_unit = _f64(V_unit)
    idx = np.asarray(idx, dtype=np.int64)
    Ncap = K_unit.shape[0]
    sel = idx[(idx >= 0) & (idx < Ncap)]
    G, d = q.shape
    if sel.shape[0] == 0:
        return np.zeros((G, d)), np.full(G, -np.inf)
    Ks = K_unit[sel]
    Vs = V_unit[sel]
    z = scale * (q @ Ks.T)                        # [G, m]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ Vs) / l
    lse = (zmax + np.log(l))[:, 0]
    return out, lse


def dense_attention(q_group, K, V, scale):
    """Full softmax attention over all rows of K, V (the case the method avoids)."""
    n = _f64(K).shape[0]
    return sparse_attention(q_group, K, V, np.arange(n), scale)


# --------------------------------------------------------------------------
# One decode step
# --------------------------------------------------------------------------

def decode_step_unit(q_group, K_unit, V_unit, kp_unit, P_h, N, M, scale):
    """Score, select and attend for one (batch row, KV head) unit.

    Returns (idx [M] int32, out [G, d], lse [G], scores [N]).
    """
    q_tilde = indexer_query(q_group, P_h)
    s = index_scores(q_tilde, np.asarray(kp_unit)[:N])
    idx = top_m(s, M)
    out, lse = sparse_attention(q_group, K_unit, V_unit, idx, scale)
    return idx, out, lse, s


def decode_step(q, k_cache, v_cache, kp_cache, P, seq_lens, M, scale):
    """Whole-batch decode step.

    q: [B, Hq, d]; caches [B, Hkv, Ncap, *]; P: [Hkv, d, r]; seq_lens: [B]
    (number of valid positions per batch row).  Returns idx [B, Hkv, M],
    out [B, Hq, d], lse [B, Hq].
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    idx = np.full((B, Hkv, M), -1, dtype=np.int32)
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hkv):
            qg = q[b, h * G:(h + 1) * G]
            i, o, l, _ = decode_step_unit(qg, k_cache[b, h], v_cache[b, h],
                                          kp_cache[b, h], P[h], int(seq_lens[b]),
                                          M, scale)
            idx[b, h] = i
            out[b, h * G:(h + 1) * G] = o
            lse[b, h * G:(h + 1) * G] = l
    return idx, out, lse


def reuse_source_layer(layer, full_layers):
    """Layer whose indices ``layer`` attends with.

    IndexCache article, "IndexCache: layer sharing for extreme acceleration":
    layers are grouped; a few "full" layers compute the indices and the
    "shared" layers after them reuse those indices.  Reading: a shared layer
    reuses the nearest full layer at or before it.
    """
    src = [f for f in sorted(full_layers) if f <= layer]
    if not src:
        raise ValueError("no full layer at or before layer %d" % layer)
    return src[-1]


# --------------------------------------------------------------------------
# LISA-style gated linear branch
# --------------------------------------------------------------------------

def elu_plus_one(x):
    """Feature map of the linear branch: x + 1 for x > 0, exp(x) otherwise."""
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_state(K, V):
    """Recurrent state of the linear branch over key/value rows ``K, V [n, d]``.

    LISA news items ("LISA architecture"; "Hybrid architecture for
    efficiency"): a linear-attention branch keeps a long-term memory in linear
    time.  Reading: S = sum_n phi(k_n) v_n^T  ([d, d], row index = key dim),
    z = sum_n phi(k_n), phi = elu + 1.
    """
    phi = elu_plus_one(K)
    return phi.T @ _f64(V), phi.sum(axis=0)


def linear_gate(q_group, S, z, w_gate, o_sparse):
    """Linear read-out and the gate that mixes it with the sparse branch.

    LISA news items: the linear and sparse branches are merged by a gating
    mechanism.  Reading: o_lin = (phi(q)^T S) / (phi(q)^T z); per query head
    g = sigmoid(w . q); out = g * o_sparse + (1 - g) * o_lin.  An empty
    memory (phi(q)^T z = 0, which with phi > 0 and z a sum of phi values
    means no token was ever added, so S = 0 too) reads out o_lin = 0: the
    linear branch then contributes nothing instead of 0 / 0.
    q_group, w_gate, o_sparse: [G, d]; S: [d, d]; z: [d].
    Returns (out [G, d], o_lin [G, d], g [G]).
    """
    q = _f64(q_group)
    phq = elu_plus_one(q)
    num = phq @ _f64(S)
    den = (phq @ _f64(z))[:, None]
    o_lin = np.divide(num, den, out=np.zeros_like(num), where=den != 0)
    with np.errstate(over="ignore"):
        g = 1.0 / (1.0 + np.exp(-np.sum(_f64(w_gate) * q, axis=1)))
    out = g[:, None] * _f64(o_sparse) + (1.0 - g)[:, None] * o_lin
    return out, o_lin, g
