"""The attention checks of the GPU tests discriminate (CPU only).

tests/_helpers.check_attention applies the contract and a relative-L2
diagnostic.  Here the oracle's own attention plays both sides: the exact
output rounded to bf16 (what a correct kernel writes) passes both checks,
while the output with 1% of the selected rows dropped -- a plausible
value-path mistake such as a lost tail tile -- still passes the contract but
fails the diagnostic.
"""

import numpy as np
import pytest
import torch

import oracle
from _helpers import attention_errors, check_attention, ATT_REL_L2


def _unit(seed, N=4096, M=2048, G=4, d=128):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).double().numpy()
    q, K, V = bf(G, d), bf(N, d), bf(N, d)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(N, M, replace=False)).astype(np.int32)
    return q, K, V, idx


def _bf16(x):
    return torch.from_numpy(np.asarray(x)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bf16_rounded_exact_output_passes(seed):
    q, K, V, idx = _unit(seed)
    o, _ = oracle.sparse_attention(q, K, V, idx, 1.0 / np.sqrt(q.shape[1]))
    check_attention(_bf16(o), o)
    assert attention_errors(_bf16(o), o)[1] < 3e-3


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_percent_of_rows_dropped_fails_only_the_diagnostic(seed):
    q, K, V, idx = _unit(seed)
    scale = 1.0 / np.sqrt(q.shape[1])
    o, _ = oracle.sparse_attention(q, K, V, idx, scale)
    rng = np.random.default_rng(100 + seed)
    drop = idx.copy()
    drop[rng.choice(idx.size, idx.size // 100, replace=False)] = -1      # 20 of 2048 rows
    o_drop, _ = oracle.sparse_attention(q, K, V, drop, scale)
    excess, rel = attention_errors(_bf16(o_drop), o)
    assert excess <= 0.0, "the contract alone would catch it; the case is too easy"
    assert rel > ATT_REL_L2, rel
    with pytest.raises(AssertionError, match="relative L2"):
        check_attention(_bf16(o_drop), o)


def test_all_zero_outputs():
    z = np.zeros((4, 8))
    check_attention(z, z)
    with pytest.raises(AssertionError):
        check_attention(z + 1e-3, z)
