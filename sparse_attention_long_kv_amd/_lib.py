"""ctypes binding of libsparse_attn.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU; it checks dtype, device, shape and
contiguity, passes raw device pointers and the current HIP stream, and raises
``SparseAttnError`` on a non-zero status.  Every step of the computation runs
in the library's HIP kernels; there is no fallback of any kind, and the
functions raise if the library has not been built.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_WORKSPACE = -3
SA_ERR_HIP = -4
SA_ERR_TOO_LARGE = -5
SA_PLAN_CHUNK_EXACT, SA_PLAN_FILTER, SA_PLAN_UNIT, SA_PLAN_SCORES = 0, 1, 2, 3
SA_NOALLOC_SCRATCH_BYTES = 64 << 20


class SparseAttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (%d)" % (fn, msg, status))
        self.status = status


class SaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("capacity", ctypes.c_int32)]

    @property
    def G(self):
        return self.num_q_heads // self.num_kv_heads

    def __repr__(self):
        return "SaShape(B=%d, Hq=%d, Hkv=%d, d=%d, r=%d, Ncap=%d)" % (
            self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim, self.rank,
            self.capacity)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, rank, capacity):
    return SaShape(batch, num_q_heads, num_kv_heads, head_dim, rank, capacity)


_lib = None

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(SaShape)

_SIGS = {
    "sparse_attn_append_kv": [_SP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "sparse_attn_project_keys": [_SP, _VP, _VP, _I32, _I32, _VP, _VP],
    "sparse_attn_index_score": [_SP, _VP, _VP, _VP, _VP, _I32, _VP, _VP],
    "sparse_attn_topm": [_SP, _VP, _VP, _I32, _I32, _VP, _VP, _SZ, _VP],
    "sparse_attn_index_topm": [_SP, _VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _SZ, _VP],
    "sparse_attn_index_topm_stage": [_SP, _I32, _VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _SZ,
                                     _VP],
    "sparse_attn_decode": [_SP, _VP, _VP, _VP, _VP, _I32, ctypes.c_float, _VP, _VP, _VP,
                           _SZ, _VP],
    "sparse_attn_decode_step": [_SP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                _I32, _I32, ctypes.c_float, _VP, _VP, _VP, _VP, _SZ, _VP],
    "sparse_attn_decode_step_stage": [_SP, _I32, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                      _VP, _I32, _I32, ctypes.c_float, _VP, _VP, _VP, _VP, _SZ,
                                      _VP],
    "sparse_attn_decode_step_noalloc": [_SP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                        _VP, _I32, _I32, ctypes.c_float, _VP, _VP, _VP, _VP],
    "sparse_attn_linear_gate": [_SP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP],
    "sparse_attn_dense_decode": [_SP, _VP, _VP, _VP, _VP, _I32, ctypes.c_float, _VP, _VP, _VP,
                                 _SZ, _VP],
    "sparse_attn_gather_kv": [_SP, _VP, _I32, _VP, _VP, _VP, _VP, _VP],
    "sparse_attn_stream_read": [_VP, _SZ, _VP, _VP],
    "sparse_attn_row_read": [_SP, _VP, _I32, _VP, _VP, _I32, _VP, _VP],
    "sparse_attn_selection_fallbacks": [_SP, _I32, _I32, _VP, _SZ, _VP, _VP],
    "sparse_attn_selection_plan": [_SP, _I32, _I32],
    "sparse_attn_workspace_size": [_SP, _I32, _I32],
    "sparse_attn_dense_workspace_size": [_SP, _I32],
    "sparse_attn_status_string": [ctypes.c_int],
}
_RESTYPES = {
    "sparse_attn_workspace_size": _SZ,
    "sparse_attn_dense_workspace_size": _SZ,
    "sparse_attn_status_string": ctypes.c_char_p,
}


def load(path=None):
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            "libsparse_attn.so is not built (%s); run "
            "`python -m sparse_attention_long_kv_amd.build_lib`" % p)
    lib = ctypes.CDLL(p)
    for name, argt in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = _RESTYPES.get(name, ctypes.c_int)
    _lib = lib
    return lib


def exported_symbols():
    return list(_SIGS)


def sparse_attn_status_string(status):
    return load().sparse_attn_status_string(int(status)).decode()


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st != SA_OK:
        raise SparseAttnError(name, st, sparse_attn_status_string(st))


def _dev_ptr(t, dtype, shape=None, name="tensor"):
    # (the cheapest form of each check: a step call checks about a dozen
    # tensors, and a Python decode loop launches at this rate)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and t.shape != (shape if isinstance(shape, tuple) else tuple(shape)):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return t.data_ptr()                  # an int; ctypes passes it as void*


def _opt_ptr(t, dtype, shape=None, name="tensor"):
    return None if t is None else _dev_ptr(t, dtype, shape, name)


def _stream(t):
    return _VP(torch.cuda.current_stream(t.device).cuda_stream)


def _sh(shape):
    return ctypes.byref(shape)


def sparse_attn_workspace_size(shape, n_max, M):
    return int(load().sparse_attn_workspace_size(_sh(shape), int(n_max), int(M)))


def alloc_workspace(shape, n_max, M, device="cuda"):
    """Workspace for calls with this (n_max, M) (contents need no initialisation)."""
    n = sparse_attn_workspace_size(shape, n_max, M)
    if n == 0:
        raise ValueError("invalid shape/n_max/M for a workspace: %r %d %d" % (shape, n_max, M))
    return torch.empty(n, dtype=torch.uint8, device=device)


def sparse_attn_append_kv(shape, pos, k_new, v_new, P, k_cache, v_cache, kp_cache):
    B, Hkv, d, r, Nc = (shape.batch, shape.num_kv_heads, shape.head_dim, shape.rank,
                        shape.capacity)
    T = k_new.shape[2]
    _call("sparse_attn_append_kv", _sh(shape),
          _dev_ptr(pos, torch.int32, (B,), "pos"), T,
          _dev_ptr(k_new, torch.bfloat16, (B, Hkv, T, d), "k_new"),
          _dev_ptr(v_new, torch.bfloat16, (B, Hkv, T, d), "v_new"),
          _dev_ptr(P, torch.float32, (Hkv, d, r), "P"),
          _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"),
          _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"), _stream(k_cache))


def sparse_attn_project_keys(shape, k_cache, P, n_begin, n_count, kp_cache):
    B, Hkv, d, r, Nc = (shape.batch, shape.num_kv_heads, shape.head_dim, shape.rank,
                        shape.capacity)
    _call("sparse_attn_project_keys", _sh(shape),
          _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(P, torch.float32, (Hkv, d, r), "P"), int(n_begin), int(n_count),
          _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"), _stream(k_cache))


def sparse_attn_index_score(shape, q, P, kp_cache, seq_lens, n_max, scores):
    B, Hq, Hkv, d, r, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads,
                            shape.head_dim, shape.rank, shape.capacity)
    _call("sparse_attn_index_score", _sh(shape),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(P, torch.float32, (Hkv, d, r), "P"),
          _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"),
          _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max),
          _dev_ptr(scores, torch.float32, (B, Hkv, n_max), "scores"), _stream(q))


def sparse_attn_topm(shape, scores, seq_lens, n_max, M, idx, workspace):
    B, Hkv = shape.batch, shape.num_kv_heads
    _call("sparse_attn_topm", _sh(shape),
          _dev_ptr(scores, torch.float32, (B, Hkv, n_max), "scores"),
          _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max), int(M),
          _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(),
          _stream(scores))


def sparse_attn_index_topm(shape, q, P, kp_cache, seq_lens, n_max, M, idx, workspace):
    B, Hq, Hkv, d, r, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads,
                            shape.head_dim, shape.rank, shape.capacity)
    _call("sparse_attn_index_topm", _sh(shape),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(P, torch.float32, (Hkv, d, r), "P"),
          _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"),
          _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max), int(M),
          _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(q))


SA_STAGE_BOUND, SA_STAGE_CANDIDATES, SA_STAGE_MERGE = 1, 2, 3


def sparse_attn_index_topm_stage(shape, stage, q, P, kp_cache, seq_lens, n_max, M, idx,
                                 workspace):
    B, Hq, Hkv, d, r, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads,
                            shape.head_dim, shape.rank, shape.capacity)
    _call("sparse_attn_index_topm_stage", _sh(shape), int(stage),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(P, torch.float32, (Hkv, d, r), "P"),
          _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"),
          _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max), int(M),
          _opt_ptr(idx, torch.int32, (B, Hkv, M), "idx"),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(q))


SA_STEP_APPEND_BOUND, SA_STEP_CANDIDATES, SA_STEP_MERGE, SA_STEP_ATTEND = 1, 2, 3, 4
SA_STEP_SELECT_ATTEND = 5


def _step_args(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache, seq_lens, n_max, M,
               softmax_scale, idx, out, lse, workspace):
    B, Hq, Hkv, d, r, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads,
                            shape.head_dim, shape.rank, shape.capacity)
    if k_new.dim() != 4 or k_new.shape[:2] != (B, Hkv) or k_new.shape[3] != d:
        raise ValueError("k_new must have shape (B, Hkv, T, d)")
    T = k_new.shape[2]
    return (_dev_ptr(pos, torch.int32, (B,), "pos"), int(T),
            _dev_ptr(k_new, torch.bfloat16, (B, Hkv, T, d), "k_new"),
            _dev_ptr(v_new, torch.bfloat16, (B, Hkv, T, d), "v_new"),
            _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
            _dev_ptr(P, torch.float32, (Hkv, d, r), "P"),
            _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
            _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"),
            _dev_ptr(kp_cache, torch.uint8, (B, Hkv, Nc, r), "kp_cache"),
            _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max), int(M),
            float(softmax_scale),
            _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"),
            _dev_ptr(out, torch.bfloat16, (B, Hq, d), "out"),
            _opt_ptr(lse, torch.float32, (B, Hq), "lse"),
            None if workspace is None else _dev_ptr(workspace, torch.uint8, name="workspace"),
            0 if workspace is None else workspace.numel(), _stream(q))


def sparse_attn_decode_step(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache,
                            seq_lens, n_max, M, softmax_scale, idx, out, lse, workspace):
    _call("sparse_attn_decode_step", _sh(shape),
          *_step_args(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache, seq_lens,
                      n_max, M, softmax_scale, idx, out, lse, workspace))


def sparse_attn_decode_step_stage(shape, stage, pos, k_new, v_new, q, P, k_cache, v_cache,
                                  kp_cache, seq_lens, n_max, M, softmax_scale, idx, out, lse,
                                  workspace):
    _call("sparse_attn_decode_step_stage", _sh(shape), int(stage),
          *_step_args(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache, seq_lens,
                      n_max, M, softmax_scale, idx, out, lse, workspace))


def sparse_attn_decode_step_noalloc(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache,
                                    seq_lens, n_max, M, softmax_scale, idx, out, lse):
    """sparse_attn_decode_step with the library's static per-GPU scratch as its
    workspace (no allocation; shapes whose workspace exceeds
    SA_NOALLOC_SCRATCH_BYTES raise with SA_ERR_TOO_LARGE)."""
    args = _step_args(shape, pos, k_new, v_new, q, P, k_cache, v_cache, kp_cache, seq_lens,
                      n_max, M, softmax_scale, idx, out, lse, None)
    _call("sparse_attn_decode_step_noalloc", _sh(shape), *(args[:16] + args[18:]))


def sparse_attn_decode(shape, q, k_cache, v_cache, idx, M, softmax_scale, out, lse, workspace):
    B, Hq, Hkv, d, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                         shape.capacity)
    _call("sparse_attn_decode", _sh(shape),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"),
          _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"), int(M), float(softmax_scale),
          _dev_ptr(out, torch.bfloat16, (B, Hq, d), "out"),
          _opt_ptr(lse, torch.float32, (B, Hq), "lse"),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(q))


def sparse_attn_dense_decode(shape, q, k_cache, v_cache, seq_lens, n_max, softmax_scale, out,
                             lse, workspace):
    """Comparison baseline: attention over every valid row (M = N)."""
    B, Hq, Hkv, d, Nc = (shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim,
                         shape.capacity)
    _call("sparse_attn_dense_decode", _sh(shape),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"),
          _opt_ptr(seq_lens, torch.int32, (B,), "seq_lens"), int(n_max), float(softmax_scale),
          _dev_ptr(out, torch.bfloat16, (B, Hq, d), "out"),
          _opt_ptr(lse, torch.float32, (B, Hq), "lse"),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(), _stream(q))


def sparse_attn_dense_workspace_size(shape, n_max):
    return int(load().sparse_attn_dense_workspace_size(_sh(shape), int(n_max)))


def sparse_attn_stream_read(buf, sink):
    """Measurement helper: one streaming read of the whole of `buf` (a device
    tensor of a multiple of 4 MiB); `sink` is a one-element int32 device
    tensor the kernel may write (it keeps the loads alive)."""
    p = _dev_ptr(buf, buf.dtype, name="buf")
    _call("sparse_attn_stream_read", p, buf.numel() * buf.element_size(),
          _dev_ptr(sink, torch.int32, (1,), "sink"), _stream(buf))


def sparse_attn_gather_kv(shape, idx, M, k_cache, v_cache, k_out, v_out):
    """Comparison baseline: copy the selected rows into contiguous buffers."""
    B, Hkv, d, Nc = shape.batch, shape.num_kv_heads, shape.head_dim, shape.capacity
    _call("sparse_attn_gather_kv", _sh(shape),
          _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"), int(M),
          _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"),
          _dev_ptr(k_out, torch.bfloat16, (B, Hkv, M, d), "k_out"),
          _dev_ptr(v_out, torch.bfloat16, (B, Hkv, M, d), "v_out"), _stream(idx))


def sparse_attn_linear_gate(shape, q, k_new, v_new, S, z, w_gate, o_sparse, out,
                            update_state=True):
    B, Hq, Hkv, d = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    _call("sparse_attn_linear_gate", _sh(shape),
          _dev_ptr(q, torch.bfloat16, (B, Hq, d), "q"),
          _dev_ptr(k_new, torch.bfloat16, (B, Hkv, d), "k_new"),
          _dev_ptr(v_new, torch.bfloat16, (B, Hkv, d), "v_new"),
          _dev_ptr(S, torch.float32, (B, Hkv, d, d), "S"),
          _dev_ptr(z, torch.float32, (B, Hkv, d), "z"),
          _dev_ptr(w_gate, torch.float32, (Hq, d), "w_gate"),
          _dev_ptr(o_sparse, torch.bfloat16, (B, Hq, d), "o_sparse"),
          _dev_ptr(out, torch.bfloat16, (B, Hq, d), "out"), int(bool(update_state)),
          _stream(q))


def sparse_attn_selection_fallbacks(shape, n_max, M, workspace, count):
    """Diagnostic: units of the last selection in `workspace` (same shape,
    n_max, M) that took the exact streaming pass, written to `count` (a
    one-element int32 device tensor); -1 for shapes without a filter path."""
    _call("sparse_attn_selection_fallbacks", _sh(shape), int(n_max), int(M),
          _dev_ptr(workspace, torch.uint8, name="workspace"), workspace.numel(),
          _dev_ptr(count, torch.int32, (1,), "count"), _stream(workspace))


def sparse_attn_selection_plan(shape, n_max, M):
    """Diagnostic: the selection method for this shape on the current device
    (SA_PLAN_CHUNK_EXACT, SA_PLAN_FILTER, SA_PLAN_UNIT or SA_PLAN_SCORES)."""
    st = load().sparse_attn_selection_plan(_sh(shape), int(n_max), int(M))
    if st < 0:
        raise SparseAttnError("sparse_attn_selection_plan", st, sparse_attn_status_string(st))
    return st


def sparse_attn_row_read(shape, idx, M, k_cache, v_cache, mode, sink):
    """Measurement helper: read the selected K and V rows once and nothing else
    (mode 0: into registers, 1: into LDS)."""
    B, Hkv, d, Nc = shape.batch, shape.num_kv_heads, shape.head_dim, shape.capacity
    _call("sparse_attn_row_read", _sh(shape), _dev_ptr(idx, torch.int32, (B, Hkv, M), "idx"),
          int(M), _dev_ptr(k_cache, torch.bfloat16, (B, Hkv, Nc, d), "k_cache"),
          _dev_ptr(v_cache, torch.bfloat16, (B, Hkv, Nc, d), "v_cache"), int(mode),
          _dev_ptr(sink, torch.int32, (1,), "sink"), _stream(idx))
