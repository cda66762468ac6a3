"""GPU parity of the comparison baselines against the fp64 oracle.

sparse_attn_dense_decode is full attention over every valid row (the JSSA
article's throughput comparison); sparse_attn_gather_kv is the copy of the
gather-then-attend scheme ("Why token selection is not enough").  Expected
values come from the oracle (oracle.dense_attention / sparse_attention) and,
for the copy, from plain indexing of the host copies of the inputs.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_long_kv_amd as sa
from workloads import default_scale
from _helpers import f64, check_attention

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


def _inputs(B, Hq, Hkv, d, N, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g).to(torch.bfloat16)
    K = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    V = torch.randn(B, Hkv, N, d, generator=g).to(torch.bfloat16)
    return q, K, V


@pytest.mark.parametrize("B,Hq,Hkv,d,N,lens", [
    (2, 8, 2, 128, 3000, [3000, 1234]),    # ragged: the second row stops mid-split
    (1, 4, 1, 64, 700, None),              # one unit, many splits
    (3, 16, 1, 128, 520, [520, 0, 17]),    # G = 16, an empty row, a single tile
    (4, 32, 8, 128, 4096, None),           # the long-context head layout
])
def test_dense_decode_matches_oracle(B, Hq, Hkv, d, N, lens):
    """Every unit's output and log-sum-exp equal the oracle's full attention
    over its first len_b rows (empty rows: out = 0, lse = -inf)."""
    _say("case: dense decode", B, Hq, Hkv, d, N, lens)
    q, K, V = _inputs(B, Hq, Hkv, d, N, seed=51)
    sh = sa.make_shape(B, Hq, Hkv, d, 16, N)
    ws = torch.empty(sa.sparse_attn_dense_workspace_size(sh, N), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    sa.sparse_attn_dense_decode(sh, q.cuda(), K.cuda(), V.cuda(), sl, N, default_scale(d), out,
                                lse, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    q64, K64, V64 = f64(q), f64(K), f64(V)
    go, gl = f64(out), lse.cpu().double().numpy()
    for b in range(B):
        n = N if lens is None else lens[b]
        for h in range(Hkv):
            o, l = oracle.dense_attention(q64[b, h * G:(h + 1) * G], K64[b, h, :n], V64[b, h, :n],
                                          default_scale(d))
            check_attention(go[b, h * G:(h + 1) * G], o, "unit (%d, %d)" % (b, h))
            if n == 0:
                assert np.all(np.isneginf(gl[b, h * G:(h + 1) * G]))
            else:
                assert np.allclose(gl[b, h * G:(h + 1) * G], l, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("B,Hq,Hkv,d,N,M,lens", [
    (2, 8, 2, 128, 5000, 300, [5000, 120]),   # the second row has fewer rows than M
    (1, 4, 1, 64, 2048, 2048, None),          # M = N
])
def test_gather_then_attend(B, Hq, Hkv, d, N, M, lens):
    """The gathered buffers equal plain indexing of the cache (zero rows for
    -1); attending over them (dense attention on capacity M with lens
    min(len_b, M)) matches the oracle's attention over the selected rows, as
    the gather-free sparse_attn_decode does."""
    _say("case: gather then attend", B, Hq, Hkv, d, N, M, lens)
    q, K, V = _inputs(B, Hq, Hkv, d, N, seed=52)
    rng = np.random.default_rng(53)
    idx = np.full((B, Hkv, M), -1, dtype=np.int32)
    for b in range(B):
        n = N if lens is None else lens[b]
        for h in range(Hkv):
            m = min(n, M)
            idx[b, h, :m] = np.sort(rng.choice(n, size=m, replace=False))
    sh = sa.make_shape(B, Hq, Hkv, d, 16, N)
    Kg = torch.full((B, Hkv, M, d), 7.0, dtype=torch.bfloat16, device="cuda")
    Vg = torch.full((B, Hkv, M, d), 7.0, dtype=torch.bfloat16, device="cuda")
    idx_d = torch.from_numpy(idx).cuda()
    sa.sparse_attn_gather_kv(sh, idx_d, M, K.cuda(), V.cuda(), Kg, Vg)
    torch.cuda.synchronize()
    Kh = K.view(torch.int16).numpy()
    Vh = V.view(torch.int16).numpy()
    expect_k = np.zeros((B, Hkv, M, d), dtype=np.int16)
    expect_v = np.zeros((B, Hkv, M, d), dtype=np.int16)
    for b in range(B):
        for h in range(Hkv):
            ok = idx[b, h] >= 0
            expect_k[b, h, ok] = Kh[b, h, idx[b, h, ok]]
            expect_v[b, h, ok] = Vh[b, h, idx[b, h, ok]]
    assert np.array_equal(Kg.cpu().view(torch.int16).numpy(), expect_k)
    assert np.array_equal(Vg.cpu().view(torch.int16).numpy(), expect_v)
    # attention over the gathered rows
    shg = sa.make_shape(B, Hq, Hkv, d, 16, M)
    glens = torch.tensor([min(N if lens is None else lens[b], M) for b in range(B)],
                         dtype=torch.int32, device="cuda")
    ws = torch.empty(sa.sparse_attn_dense_workspace_size(shg, M), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    sa.sparse_attn_dense_decode(shg, q.cuda(), Kg, Vg, glens, M, default_scale(d), out, None, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    q64, K64, V64 = f64(q), f64(K), f64(V)
    go = f64(out)
    for b in range(B):
        for h in range(Hkv):
            o, _ = oracle.sparse_attention(q64[b, h * G:(h + 1) * G], K64[b, h], V64[b, h],
                                           idx[b, h], default_scale(d))
            check_attention(go[b, h * G:(h + 1) * G], o, "unit (%d, %d)" % (b, h))


def test_stream_read_runs_over_whole_buffers():
    """The measurement helper reads buffers of multiples of 4 MiB and
    reports no error; the sink is written only for one data-dependent value
    (never for this buffer of ones), so it keeps its contents."""
    _say("case: stream read")
    buf = torch.ones(1 << 20, dtype=torch.int32, device="cuda")      # 4 MiB
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sa.sparse_attn_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    with pytest.raises(sa.SparseAttnError):
        sa.sparse_attn_stream_read(buf[:1000], sink)


@pytest.mark.parametrize("d", [128, 64])
def test_row_read_runs_over_selected_rows(d):
    """The random-row measurement helper reads the selected rows (padding and
    out-of-range entries skipped) in both modes without error; the sink keeps
    its contents for these rows of ones."""
    _say("case: row read d=%d" % d)
    B, Hq, Hkv, N, M = 2, 8, 2, 5000, 700
    sh = sa.make_shape(B, Hq, Hkv, d, 16, N)
    K = torch.ones(B, Hkv, N, d, dtype=torch.bfloat16, device="cuda")
    V = torch.ones_like(K)
    rng = np.random.default_rng(3)
    idx = np.stack([np.stack([np.sort(rng.choice(N, M, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    idx[0, 1, -50:] = -1
    idx[1, 0, ::9] = N + 3
    idx = torch.from_numpy(idx).cuda()
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for mode in (0, 1):
        sa.sparse_attn_row_read(sh, idx, M, K, V, mode, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
