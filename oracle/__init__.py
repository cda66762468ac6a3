"""Plain CPU oracle of one indexer-selected sparse decode step (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything under ``oracle/``: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or constant
generators); the only code both sides share is the seeded input generator in
``workloads/``, which holds none of the method's arithmetic.

What it computes is written from the pages, step by step and in their order:

* the JSSA article (rit.work blog on "Joint Subspace Sparse Attention for
  Efficient Long-Context Decoding"), sections "Why token selection is not
  enough" and "How JSSA preserves token order": average the queries of one KV
  head's group, project them with the per-head basis, score every cached
  position against the FP8 projected-key cache, select, then run exact
  attention over the selected full-size keys and values;
* the DSA paragraphs of the IndexCache article (denisavetisyan.com,
  "DeepSeek Sparse Attention: a step towards efficiency"): the indexer keeps the
  top-k (here top-M) positions;
* the IndexCache article, section "IndexCache: layer sharing for extreme
  acceleration": "full" layers compute indices, "shared" layers reuse them;
* the LISA news items (aikraft.ru "LISA architecture", opennieuws.be "Hybrid
  architecture for efficiency"): a linear-attention branch mixed with the
  sparse branch by a gate.

Every function runs in float64.  Pins that tie it to something other than
itself live in ``tests/test_oracle_*.py`` and ``tests/golden/``.
"""

from .fp8_e4m3 import decode_table, fp8_decode, fp8_encode, FP8_MAX
from .jssa import (
    project_keys,
    append_kv,
    indexer_query,
    index_scores,
    top_m,
    sparse_attention,
    dense_attention,
    decode_step_unit,
    decode_step,
    reuse_source_layer,
    elu_plus_one,
    linear_state,
    linear_gate,
)

__all__ = [
    "decode_table", "fp8_decode", "fp8_encode", "FP8_MAX",
    "project_keys", "append_kv", "indexer_query", "index_scores", "top_m",
    "sparse_attention", "dense_attention", "decode_step_unit", "decode_step",
    "reuse_source_layer", "elu_plus_one", "linear_state", "linear_gate",
]
