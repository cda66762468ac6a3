"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

The library must load, export every entry point ``include/sparse_attn.h``
declares, and reject bad arguments on the host before anything is launched.
Every call below fails a host check, so no kernel is ever enqueued.
"""

import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_long_kv_amd as sa
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return sa.load()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("sparse_attn_append_kv", "sparse_attn_index_score", "sparse_attn_topm",
              "sparse_attn_decode", "sparse_attn_linear_gate"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sparse_attn_\w+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(_declared()) == set(sa.exported_symbols())


def test_library_targets_gfx950_only():
    data = open(sa.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def _shape(wl, cap=None):
    return sa.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.r, cap or wl.N)


def test_status_strings():
    assert sa.sparse_attn_status_string(0) == "ok"
    for s in (-1, -2, -3, -4, 7):
        assert len(sa.sparse_attn_status_string(s)) > 0


def test_workspace_size_rules():
    wl = WORKLOADS["longctx_128k"]
    sh = _shape(wl)
    ws = sa.sparse_attn_workspace_size(sh, wl.N, wl.M)
    assert ws > 0 and ws % 256 == 0
    # no gathered K/V buffer: far below B*Hkv*M*d*2 (K+V) bytes
    gathered = wl.B * wl.Hkv * wl.M * wl.d * 2 * 2
    assert ws < gathered / 4
    assert sa.sparse_attn_workspace_size(sh, 0, 10) == 0
    assert sa.sparse_attn_workspace_size(sh, wl.N + 1, 10) == 0
    assert sa.sparse_attn_workspace_size(sh, wl.N, 0) == 0
    bad = sa.make_shape(1, 4, 1, 96, 16, 100)
    assert sa.sparse_attn_workspace_size(bad, 100, 10) == 0


@pytest.mark.parametrize("units", [(1, 1), (2, 4), (32, 8)])
@pytest.mark.parametrize("d", [64, 128])
def test_workspace_covers_every_context_the_shape_allows(units, d):
    """Every n_max up to the largest capacity the shape admits (int32 byte
    offsets within a unit's cache) has a workspace, whatever the number of
    units: the chunk planning never asks for more chunks than a unit may have.
    Past that capacity the shape itself is unsupported."""
    B, Hkv = units
    top = (2 ** 31 - 1) // (d * 2)
    for n in (1, 2047, 524288, 524289, 600000, 1 << 22, top):
        sh = sa.make_shape(B, 4 * Hkv, Hkv, d, 32, n)
        for M in sorted({1, min(n, 2048), min(n, 6145)}):
            ws = sa.sparse_attn_workspace_size(sh, n, M)
            assert ws > 0 and ws % 256 == 0, (units, d, n, M)
    assert sa.sparse_attn_workspace_size(sa.make_shape(B, 4 * Hkv, Hkv, d, 32, top + 1),
                                         top + 1, 2048) == 0


_FAKE = 1 << 20      # aligned, never dereferenced (every call below fails a check)


def _st(lib, name, *args):
    return getattr(lib, name)(*args)


def test_bad_shapes_are_rejected(lib):
    P = ctypes.c_void_p(_FAKE)
    for sh, expect in [(sa.make_shape(1, 4, 1, 96, 16, 100), sa.SA_ERR_UNSUPPORTED),
                       (sa.make_shape(1, 4, 1, 64, 8, 100), sa.SA_ERR_UNSUPPORTED),
                       (sa.make_shape(1, 34, 2, 64, 16, 100), sa.SA_ERR_UNSUPPORTED),
                       (sa.make_shape(1, 6, 4, 64, 16, 100), sa.SA_ERR_INVALID),
                       (sa.make_shape(0, 4, 1, 64, 16, 100), sa.SA_ERR_INVALID),
                       (sa.make_shape(1, 4, 1, 64, 16, 0), sa.SA_ERR_INVALID)]:
        st = _st(lib, "sparse_attn_index_score", ctypes.byref(sh), P, P, P, None, 10, P, None)
        assert st == expect, (sh, st)
    assert _st(lib, "sparse_attn_decode", None, P, P, P, P, 4, ctypes.c_float(1.0), P, None,
               P, 1 << 20, None) == sa.SA_ERR_INVALID


def test_stream_read_rejects_bad_arguments(lib):
    """The measurement helper checks its buffer, size and sink on the host."""
    P = ctypes.c_void_p(_FAKE)
    odd = ctypes.c_void_p(_FAKE + 2)
    for buf, nbytes, sink in [(None, 1 << 22, P), (odd, 1 << 22, P), (P, 1 << 22, None),
                              (P, 0, P), (P, 100, P), (P, 1 << 20, P), (P, (1 << 22) + 16, P)]:
        assert _st(lib, "sparse_attn_stream_read", buf, ctypes.c_size_t(nbytes), sink,
                   None) == sa.SA_ERR_INVALID, (buf, nbytes, sink)


def test_row_read_rejects_bad_arguments(lib):
    wl = WORKLOADS["tiny"]
    sh = _shape(wl)
    P = ctypes.c_void_p(_FAKE)
    odd = ctypes.c_void_p(_FAKE + 2)
    by = ctypes.byref(sh)
    for idx, M, k, v, mode, sink in [(None, 4, P, P, 0, P), (P, 0, P, P, 0, P),
                                     (P, 4, odd, P, 0, P), (P, 4, P, None, 1, P),
                                     (P, 4, P, P, 2, P), (P, 4, P, P, 0, None)]:
        assert _st(lib, "sparse_attn_row_read", by, idx, M, k, v, mode, sink,
                   None) == sa.SA_ERR_INVALID, (idx, M, mode)


def test_bad_arguments_are_rejected(lib):
    wl = WORKLOADS["tiny"]
    sh = _shape(wl)
    P = ctypes.c_void_p(_FAKE)
    odd = ctypes.c_void_p(_FAKE + 2)
    by = ctypes.byref(sh)
    # null and misaligned pointers
    assert _st(lib, "sparse_attn_index_score", by, None, P, P, None, 10, P, None) == -1
    assert _st(lib, "sparse_attn_index_score", by, odd, P, P, None, 10, P, None) == -1
    assert _st(lib, "sparse_attn_append_kv", by, P, 1, P, P, P, P, P, None, None) == -1
    # sizes
    assert _st(lib, "sparse_attn_index_score", by, P, P, P, None, 0, P, None) == -1
    assert _st(lib, "sparse_attn_index_score", by, P, P, P, None, wl.N + 1, P, None) == -1
    assert _st(lib, "sparse_attn_append_kv", by, P, -1, P, P, P, P, P, P, None) == -1
    assert _st(lib, "sparse_attn_project_keys", by, P, P, wl.N - 3, 4, P, None) == -1
    assert _st(lib, "sparse_attn_topm", by, P, None, wl.N, wl.N + 1, P, P, 1 << 30, None) == -1
    assert _st(lib, "sparse_attn_topm", by, P, None, wl.N, 0, P, P, 1 << 30, None) == -1
    assert _st(lib, "sparse_attn_decode", by, P, P, P, P, 0, ctypes.c_float(1.0), P, None, P,
               1 << 30, None) == -1
    assert _st(lib, "sparse_attn_decode", by, P, P, P, P, 4, ctypes.c_float(float("inf")), P,
               None, P, 1 << 30, None) == -1
    # workspace missing / too small
    need = sa.sparse_attn_workspace_size(sh, wl.N, wl.M)
    assert _st(lib, "sparse_attn_topm", by, P, None, wl.N, wl.M, P, None, need, None) == -3
    assert _st(lib, "sparse_attn_topm", by, P, None, wl.N, wl.M, P, P, need - 1, None) == -3
    assert _st(lib, "sparse_attn_index_topm", by, P, P, P, None, wl.N, wl.M, P, P, need - 1,
               None) == -3
    step = "sparse_attn_decode_step_stage"
    f1 = ctypes.c_float(1.0)
    assert _st(lib, step, by, 0, P, 1, P, P, P, P, P, P, P, None, wl.N, wl.M, f1, P, P, None, P,
               need, None) == -1
    # baselines
    dneed = sa.sparse_attn_dense_workspace_size(sh, wl.N)
    assert dneed > 0 and sa.sparse_attn_dense_workspace_size(sh, wl.N + 1) == 0
    dense = "sparse_attn_dense_decode"
    assert _st(lib, dense, by, P, P, P, None, 0, f1, P, None, P, dneed, None) == -1
    assert _st(lib, dense, by, P, P, odd, None, wl.N, f1, P, None, P, dneed, None) == -1
    assert _st(lib, dense, by, P, P, P, None, wl.N, ctypes.c_float(float("nan")), P, None, P,
               dneed, None) == -1
    assert _st(lib, dense, by, P, P, P, None, wl.N, f1, P, None, P, dneed - 1, None) == -3
    assert _st(lib, dense, by, P, P, P, None, wl.N, f1, P, None, None, dneed, None) == -3
    gather = "sparse_attn_gather_kv"
    assert _st(lib, gather, by, P, 0, P, P, P, P, None) == -1
    assert _st(lib, gather, by, P, wl.N + 1, P, P, P, P, None) == -1
    assert _st(lib, gather, by, None, wl.M, P, P, P, P, None) == -1
    assert _st(lib, gather, by, P, wl.M, P, P, odd, P, None) == -1
    for bad in (6, -1):                                       # unknown stages
        assert _st(lib, step, by, bad, P, 1, P, P, P, P, P, P, P, None, wl.N, wl.M, f1, P, P,
                   None, P, need, None) == -1
    assert _st(lib, step, by, 1, P, 1, P, P, P, P, P, P, P, None, wl.N, wl.M, f1, P, P, None, P,
               need - 1, None) == -3
    assert _st(lib, "sparse_attn_decode_step", by, P, -1, P, P, P, P, P, P, P, None, wl.N, wl.M,
               f1, P, P, None, P, need, None) == -1
    assert _st(lib, "sparse_attn_decode_step", by, P, 1, P, P, P, P, P, P, P, None, wl.N, wl.M,
               ctypes.c_float(float("nan")), P, P, None, P, need, None) == -1
    stage = "sparse_attn_index_topm_stage"
    assert _st(lib, stage, by, 2, P, P, P, None, wl.N, wl.M, None, None, need, None) == -3
    assert _st(lib, stage, by, 3, P, P, P, None, wl.N, wl.M, P, P, need - 1, None) == -3
    assert _st(lib, stage, by, 3, P, P, P, None, wl.N, wl.M, None, P, need, None) == -1
    assert _st(lib, stage, by, 1, P, P, P, None, wl.N, wl.N + 1, None, P, need, None) == -1
    assert _st(lib, stage, by, 0, P, P, P, None, wl.N, wl.M, P, P, need, None) == -1
    assert _st(lib, stage, by, 4, P, P, P, None, wl.N, wl.M, P, P, need, None) == -1
    assert _st(lib, "sparse_attn_decode", by, P, P, P, P, wl.M, ctypes.c_float(1.0), P, None,
               P, 16, None) == -3
    # zero-size work is accepted without launching
    assert _st(lib, "sparse_attn_append_kv", by, P, 0, P, P, P, P, P, P, None) == 0
    assert _st(lib, "sparse_attn_project_keys", by, P, P, 0, 0, P, None) == 0


def test_binding_raises_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("sparse_attention_long_kv_amd._lib")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved
