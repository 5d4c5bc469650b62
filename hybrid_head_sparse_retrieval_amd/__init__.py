"""Python binding of liblychee_decode.so (the gfx950 hybrid-head sparse decode step).

Argument marshalling only: every step of the computation runs in the HIP kernels
behind the C ABI declared in include/lychee_decode.h. PyTorch supplies device
memory and the current stream. The library must have been built
(``python -m hybrid_head_sparse_retrieval_amd.build``); importing the functions
below without it raises ``LycheeDecodeUnavailable`` -- there is no fallback path.
"""
from __future__ import annotations

import collections
import ctypes
import math
import os
from typing import Optional

__all__ = [
    "LycheeDecodeError", "LycheeDecodeUnavailable", "library_path", "load_library",
    "Shape", "workspace_bytes", "topk_workspace_bytes", "Workspace", "TopkWorkspace",
    "retrieval_decode", "sparse_decode", "hybrid_layer", "topk_select",
    "hysparse_workspace_bytes", "HySparseWorkspace", "hysparse_layer",
    "tsa_workspace_bytes", "TsaWorkspace", "tsa_attention", "TSA_CAUSAL", "TSA_ZERO_FILL", "TSA_GIVEN_IDX",
    "hybrid_layer_noalloc", "hybrid_layer_plan", "LayerPlan", "prefill_hybrid_layer", "PrefillWorkspace", "NOALLOC_SCRATCH_BYTES", "FLAG_SKIP_TOPK", "FLAG_S_CHAINED", "FLAG_SEPARATE_SELECT", "FLAG_BLOCK_SELECT", "flag_split_rows", "flag_waves", "EXPORTED_SYMBOLS",
]

LD_OK = 0
FLAG_SKIP_TOPK = 1
FLAG_S_CHAINED = 2
FLAG_SEPARATE_SELECT = 4
FLAG_BLOCK_SELECT = 8
TSA_CAUSAL = 1
TSA_ZERO_FILL = 2
TSA_GIVEN_IDX = 4
_STATUS = {1: "invalid argument", 2: "unsupported shape", 3: "workspace missing or too small",
           4: "HIP launch or copy failed", 5: "a bounded wait between workgroups gave up",
           6: "the shape needs more scratch than the library's static buffer holds"}
NOALLOC_SCRATCH_BYTES = 128 << 20     # LD_NOALLOC_SCRATCH_BYTES
EXPORTED_SYMBOLS = ("ld_status_string", "ld_workspace_size", "ld_topk_workspace_size",
                    "ld_workspace_init", "ld_workspace_check", "ld_retrieval_decode",
                    "ld_sparse_decode", "ld_hybrid_layer", "ld_topk_select",
                    "ld_hysparse_workspace_size", "ld_hysparse_layer",
                    "ld_tsa_workspace_size", "ld_tsa_attention", "ld_hybrid_layer_noalloc",
                    "ld_hybrid_layer_plan", "ld_prefill_workspace_size", "ld_prefill_hybrid_layer")


def flag_split_rows(v: int) -> int:
    """Rows per attention split = 256 << (v - 1), v in 1..5 (0 = automatic)."""
    return (int(v) & 0xF) << 8


def flag_waves(v: int) -> int:
    """Waves per attention workgroup: 1 = 4 waves, 2 = 8 waves (0 = automatic)."""
    return (int(v) & 0x3) << 12


class LycheeDecodeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, 'status %d' % status)}")


class LycheeDecodeUnavailable(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblychee_decode.so")


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("kv_indptr", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("pages_per_seq", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("s_capacity", ctypes.c_int64),
    ]


_lib = None


def load_library():
    """Load the shared library (once). Raises LycheeDecodeUnavailable if not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise LycheeDecodeUnavailable(
            f"{path} is missing; build it with `python -m hybrid_head_sparse_retrieval_amd.build`")
    # torch brings its own HIP runtime; load it first so that the library binds to the
    # same runtime (and so the same device context) as the tensors it is handed
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t)
    sp = ctypes.POINTER(Shape)
    lib.ld_status_string.restype = ctypes.c_char_p
    lib.ld_status_string.argtypes = [i32]
    lib.ld_workspace_size.restype = sz
    lib.ld_workspace_size.argtypes = [sp, i32]
    lib.ld_topk_workspace_size.restype = sz
    lib.ld_topk_workspace_size.argtypes = [i32, i32]
    lib.ld_workspace_init.restype = i32
    lib.ld_workspace_init.argtypes = [vp, sz, vp]
    lib.ld_workspace_check.restype = i32
    lib.ld_workspace_check.argtypes = [vp, sz, vp]
    lib.ld_retrieval_decode.restype = i32
    lib.ld_retrieval_decode.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.ld_sparse_decode.restype = i32
    lib.ld_sparse_decode.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, u32, vp, sz, vp]
    lib.ld_hybrid_layer.restype = i32
    lib.ld_hybrid_layer.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, vp, vp, u32, vp, sz, vp]
    lib.ld_hybrid_layer_plan.restype = i32
    lib.ld_hybrid_layer_plan.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, vp, vp, u32, vp]
    lib.ld_hybrid_layer_noalloc.restype = i32
    lib.ld_hybrid_layer_noalloc.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, vp, vp, u32, vp]
    lib.ld_hysparse_workspace_size.restype = sz
    lib.ld_hysparse_workspace_size.argtypes = [sp, i32, i32]
    lib.ld_hysparse_layer.restype = i32
    lib.ld_hysparse_layer.argtypes = [sp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, u32, vp, sz, vp]
    lib.ld_tsa_workspace_size.restype = sz
    lib.ld_tsa_workspace_size.argtypes = [sp, i32]
    lib.ld_tsa_attention.restype = i32
    lib.ld_tsa_attention.argtypes = [sp, vp, vp, vp, vp, i32, vp, vp, u32, vp, sz, vp]
    lib.ld_prefill_workspace_size.restype = sz
    lib.ld_prefill_workspace_size.argtypes = [sp, i32]
    lib.ld_prefill_hybrid_layer.restype = i32
    lib.ld_prefill_hybrid_layer.argtypes = [sp, u64, vp, vp, vp, i32, vp, vp, vp, vp, u32, vp, sz, vp]
    lib.ld_topk_select.restype = i32
    lib.ld_topk_select.argtypes = [vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != LD_OK:
        raise LycheeDecodeError(status, where)


def make_shape(q, k_cache, kv_indptr=None, seq_len=None, scale=None, block_table=None,
               page_size: int = 0, k_scale=None, v_scale=None) -> Shape:
    """ld_shape from tensors: q [B][Hq][d], k_cache [Hkv][T][d]. Paged KV: block_table is
    an int32 device tensor [B][pages_per_seq] of page ids into the T / page_size pages of
    k_cache and v_cache; seq_len (and kv_indptr for ragged lengths) give the lengths.
    Quantised KV: k_cache / v_cache of dtype uint8 (or float8_e4m3fn) hold E4M3 codes,
    and k_scale / v_scale (default 1) their per-tensor dequantisation scales."""
    B, Hq, d = q.shape
    Hkv, T, d2 = k_cache.shape
    if d2 != d:
        raise ValueError("head_dim of q and k_cache differ")
    if kv_indptr is None and block_table is None:
        n = seq_len if seq_len is not None else T // B
    else:
        if seq_len is None:
            raise ValueError("seq_len (max sequence length) is required with kv_indptr or block_table")
        n = seq_len
    s = Shape()
    s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim = B, Hq, Hkv, d
    s.seq_len = int(n)
    s.total_tokens = int(T)
    s.kv_indptr = _ptr(kv_indptr)
    s.softmax_scale = float(scale) if scale is not None else 0.0
    if _is_fp8(k_cache):
        s.kv_dtype = 1
        s.k_scale = float(k_scale) if k_scale is not None else 1.0
        s.v_scale = float(v_scale) if v_scale is not None else 1.0
    if block_table is not None:
        torch = _torch()
        _req(block_table, torch.int32, "block_table")
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B][pages_per_seq]")
        s.page_size = int(page_size)
        s.pages_per_seq = int(block_table.shape[1])
        s.block_table = block_table.data_ptr()
    return s


def workspace_bytes(shape: Shape, k_max: int) -> int:
    n = load_library().ld_workspace_size(ctypes.byref(shape), int(k_max))
    if n == 0:
        raise LycheeDecodeError(1, "ld_workspace_size")
    return int(n)


def topk_workspace_bytes(rows: int, n: int) -> int:
    v = load_library().ld_topk_workspace_size(int(rows), int(n))
    if v == 0:
        raise LycheeDecodeError(1, "ld_topk_workspace_size")
    return int(v)


class _WS:
    def __init__(self, nbytes: int, device):
        torch = _torch()
        self.nbytes = int(nbytes)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _check(load_library().ld_workspace_init(self.buf.data_ptr(), self.nbytes, _stream()),
               "ld_workspace_init")

    def ptr(self) -> int:
        return self.buf.data_ptr()

    def check(self) -> None:
        """Raise LycheeDecodeError when a bounded wait inside a launch gave up since the
        last check (then those calls' results are unreliable); clears the flag.
        Synchronises the current stream."""
        _check(load_library().ld_workspace_check(self.ptr(), self.nbytes, _stream()), "ld_workspace_check")


# Workspaces the binding keeps for calls that pass none: one per (entry point, device,
# stream, sizes that fix the workspace layout), reused by the later calls on the same
# stream, which are ordered after the earlier ones; the least recently used beyond
# _WS_CACHE_MAX are released (the allocator reuses their memory in stream order).
_WS_CACHE: "collections.OrderedDict" = collections.OrderedDict()
_WS_CACHE_MAX = 8


def _default_ws(kind: str, key: tuple, make, device):
    torch = _torch()
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    full = (kind, idx, _stream(), key)
    ws = _WS_CACHE.get(full)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"{kind}: pass a workspace to calls under graph capture (its first "
                               "use on a stream allocates and clears one)")
        ws = make()
        _WS_CACHE[full] = ws
        while len(_WS_CACHE) > _WS_CACHE_MAX:
            _WS_CACHE.popitem(last=False)
    else:
        _WS_CACHE.move_to_end(full)
    return ws


def _layout_key(shape, *extra) -> tuple:
    return (shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.seq_len,
            shape.page_size, shape.total_tokens, shape.kv_dtype) + tuple(int(x) for x in extra)


class Workspace(_WS):
    """Zero-initialised device workspace for the layer entry points."""

    def __init__(self, shape: Shape, k_max: int, device="cuda"):
        super().__init__(workspace_bytes(shape, k_max), device)


def hysparse_workspace_bytes(shape: Shape, k_max: int, window_len: int) -> int:
    n = load_library().ld_hysparse_workspace_size(ctypes.byref(shape), int(k_max), int(window_len))
    if n == 0:
        raise LycheeDecodeError(1, "ld_hysparse_workspace_size")
    return int(n)


class HySparseWorkspace(_WS):
    """Zero-initialised device workspace for hysparse_layer."""

    def __init__(self, shape: Shape, k_max: int, window_len: int, device="cuda"):
        super().__init__(hysparse_workspace_bytes(shape, k_max, window_len), device)


def tsa_shape(q, k_cache, batch: int, scale=None) -> Shape:
    """ld_shape of a prefill: q [Hq][B*T][d], k_cache [Hkv][B*T][d], B = batch."""
    Hq, BT, d = (int(x) for x in q.shape)
    if BT % batch:
        raise ValueError("q rows are not a multiple of the batch")
    s = Shape()
    s.batch, s.num_q_heads, s.num_kv_heads, s.head_dim = int(batch), Hq, int(k_cache.shape[0]), d
    s.seq_len = BT // batch
    s.total_tokens = BT
    s.softmax_scale = float(scale) if scale is not None else 0.0
    return s


def tsa_workspace_bytes(shape: Shape, k: int) -> int:
    n = load_library().ld_tsa_workspace_size(ctypes.byref(shape), int(k))
    if n == 0:
        raise LycheeDecodeError(1, "ld_tsa_workspace_size")
    return int(n)


class TsaWorkspace(_WS):
    """Zero-initialised device workspace for tsa_attention."""

    def __init__(self, shape: Shape, k: int, device="cuda"):
        super().__init__(tsa_workspace_bytes(shape, k), device)


def prefill_workspace_bytes(shape: Shape, k: int) -> int:
    n = load_library().ld_prefill_workspace_size(ctypes.byref(shape), int(k))
    if n == 0:
        raise LycheeDecodeError(1, "ld_prefill_workspace_size")
    return int(n)


class PrefillWorkspace(_WS):
    """Zero-initialised device workspace for prefill_hybrid_layer."""

    def __init__(self, shape: Shape, k: int, device="cuda"):
        super().__init__(prefill_workspace_bytes(shape, k), device)


class TopkWorkspace(_WS):
    def __init__(self, rows: int, n: int, device="cuda"):
        super().__init__(topk_workspace_bytes(rows, n), device)


def _req(t, dtype, name):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, dtype, name):
    return None if t is None else _req(t, dtype, name)


def _sizes(shape, q, out, k, kv_indptr=None, s_bufs=(), s_indptr=None, scores_out=None):
    """Sizes of the caller's buffers against the shape: the kernels write them without
    bounds of their own. CSR S rows are sized by device-side offsets, so only the offset
    array is checked for them."""
    B, Hq = int(shape.batch), int(shape.num_q_heads)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q [B][Hq][d]")
    if kv_indptr is not None and kv_indptr.numel() != B + 1:
        raise ValueError("kv_indptr must hold B+1 offsets")
    if s_indptr is not None:
        if s_indptr.numel() != B * Hq + 1:
            raise ValueError("s_indptr must hold B*Hq+1 offsets")
    else:
        for name, t in s_bufs:
            if t is not None and t.numel() < B * Hq * int(k):
                raise ValueError(f"{name} must hold B*Hq*k indices ([B][Hq][k])")
    if scores_out is not None and scores_out.numel() < B * Hq * int(shape.seq_len):
        raise ValueError("scores_out must hold B*Hq*seq_len values ([B][Hq][seq_len])")


def _clamp_k(shape, k, s_indptr, s_bufs) -> int:
    """The pages' budget clamp k = min(k, seq_len) (Token Sparse Attention skill page,
    Step 3; LycheeDecode skill page, Step 1), and, for CSR S, the S buffers' capacity
    that bounds every row on the device."""
    k = min(int(k), int(shape.seq_len))
    if k < 1:
        raise ValueError("k must be at least 1")
    if s_indptr is not None:
        caps = [t.numel() for _, t in s_bufs if t is not None]
        shape.s_capacity = min(caps) if caps else 0
    return k


def _is_fp8(t) -> bool:
    torch = _torch()
    return t.dtype == torch.uint8 or t.dtype == getattr(torch, "float8_e4m3fn", None)


def _prep(q, k_cache, v_cache, out, kv_indptr):
    torch = _torch()
    _req(q, torch.bfloat16, "q")
    kv_dtype = k_cache.dtype if _is_fp8(k_cache) else torch.bfloat16
    _req(k_cache, kv_dtype, "k_cache")
    _req(v_cache, kv_dtype, "v_cache")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if out is None:
        out = torch.empty_like(q)
    _req(out, torch.bfloat16, "out")
    _opt(kv_indptr, torch.int64, "kv_indptr")
    return out


def retrieval_decode(q, k_cache, v_cache, head_mask: int, k: int, *, s_out=None, s_indptr=None,
                     scores_out=None, out=None, workspace: Optional[Workspace] = None,
                     kv_indptr=None, seq_len=None, scale=None, block_table=None, page_size: int = 0,
                     k_scale=None, v_scale=None):
    """Retrieval heads: full attention (+ argsTopK into s_out when given). Returns out."""
    torch = _torch()
    out = _prep(q, k_cache, v_cache, out, kv_indptr)
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    _opt(s_out, torch.int32, "s_out"); _opt(s_indptr, torch.int64, "s_indptr")
    _opt(scores_out, torch.float32, "scores_out")
    k = _clamp_k(shape, k, s_indptr, [("s_out", s_out)])
    _sizes(shape, q, out, k, kv_indptr, [("s_out", s_out)], s_indptr, scores_out)
    ws = workspace or _default_ws("layer", _layout_key(shape, k), lambda: Workspace(shape, k, q.device), q.device)
    _check(load_library().ld_retrieval_decode(
        ctypes.byref(shape), int(head_mask), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        int(k), _ptr(s_out), _ptr(s_indptr), _ptr(scores_out), out.data_ptr(), ws.ptr(), ws.nbytes,
        _stream()), "ld_retrieval_decode")
    return out


def sparse_decode(q, k_cache, v_cache, head_mask: int, k: int, s_in, *, s_indptr=None, out=None,
                  flags: int = 0, workspace: Optional[Workspace] = None, kv_indptr=None,
                  seq_len=None, scale=None, block_table=None, page_size: int = 0, k_scale=None,
                  v_scale=None):
    """Sparse heads: attention over K[S], V[S]. Returns out."""
    torch = _torch()
    out = _prep(q, k_cache, v_cache, out, kv_indptr)
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    _req(s_in, torch.int32, "s_in"); _opt(s_indptr, torch.int64, "s_indptr")
    k = _clamp_k(shape, k, s_indptr, [("s_in", s_in)])
    _sizes(shape, q, out, k, kv_indptr, [("s_in", s_in)], s_indptr)
    ws = workspace or _default_ws("layer", _layout_key(shape, k), lambda: Workspace(shape, k, q.device), q.device)
    _check(load_library().ld_sparse_decode(
        ctypes.byref(shape), int(head_mask), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        int(k), s_in.data_ptr(), _ptr(s_indptr), out.data_ptr(), int(flags), ws.ptr(), ws.nbytes,
        _stream()), "ld_sparse_decode")
    return out


def hybrid_layer(q, k_cache, v_cache, retrieval_mask: int, k: int, s, *, s_out=None,
                 s_indptr=None, scores_out=None, out=None, flags: int = 0,
                 workspace: Optional[Workspace] = None, kv_indptr=None, seq_len=None,
                 scale=None, block_table=None, page_size: int = 0, k_scale=None, v_scale=None):
    """One layer of the recurrence. `s` is S^{l} (None for an all-retrieval layer);
    S^{l+1} is written to `s_out` (default: in place into `s`). Returns out."""
    torch = _torch()
    out = _prep(q, k_cache, v_cache, out, kv_indptr)
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    _opt(s, torch.int32, "s"); _opt(s_out, torch.int32, "s_out")
    _opt(s_indptr, torch.int64, "s_indptr"); _opt(scores_out, torch.float32, "scores_out")
    if s_out is None:
        s_out = s
    k = _clamp_k(shape, k, s_indptr, [("s", s), ("s_out", s_out)])
    _sizes(shape, q, out, k, kv_indptr, [("s", s), ("s_out", s_out)], s_indptr, scores_out)
    ws = workspace or _default_ws("layer", _layout_key(shape, k), lambda: Workspace(shape, k, q.device), q.device)
    _check(load_library().ld_hybrid_layer(
        ctypes.byref(shape), int(retrieval_mask), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), int(k), _ptr(s), _ptr(s_out), _ptr(s_indptr), _ptr(scores_out),
        out.data_ptr(), int(flags), ws.ptr(), ws.nbytes, _stream()), "ld_hybrid_layer")
    return out


class LayerPlan(ctypes.Structure):
    """ld_layer_plan: the launches of one ld_hybrid_layer call."""
    _fields_ = [("launches", ctypes.c_int32), ("attention_workgroups", ctypes.c_int32),
                ("split_rows_stream", ctypes.c_int32), ("split_rows_gather", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("select_in_launch", ctypes.c_int32),
                ("selector_parts", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_ if name != "reserved"}


def hybrid_layer_plan(q, k_cache, v_cache, retrieval_mask: int, k: int, s, *, s_out=None,
                      s_indptr=None, scores_out=None, out=None, flags: int = 0, kv_indptr=None,
                      seq_len=None, scale=None, block_table=None, page_size: int = 0, k_scale=None,
                      v_scale=None) -> dict:
    """What hybrid_layer would launch for the same arguments (nothing is launched):
    kernel count, attention grid, split rows, waves, and whether S is selected inside
    the attention launch."""
    torch = _torch()
    _opt(s, torch.int32, "s"); _opt(s_out, torch.int32, "s_out")
    _opt(s_indptr, torch.int64, "s_indptr"); _opt(scores_out, torch.float32, "scores_out")
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    if s_out is None:
        s_out = s
    k = _clamp_k(shape, k, s_indptr, [("s", s), ("s_out", s_out)])
    out_ptr = out.data_ptr() if out is not None else q.data_ptr()
    plan = LayerPlan()
    _check(load_library().ld_hybrid_layer_plan(
        ctypes.byref(shape), int(retrieval_mask), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), int(k), _ptr(s), _ptr(s_out), _ptr(s_indptr), _ptr(scores_out),
        out_ptr, int(flags), ctypes.byref(plan)), "ld_hybrid_layer_plan")
    return plan.as_dict()


def hybrid_layer_noalloc(q, k_cache, v_cache, retrieval_mask: int, k: int, s, *, out, s_out=None,
                         s_indptr=None, scores_out=None, flags: int = 0, kv_indptr=None, seq_len=None,
                         scale=None, block_table=None, page_size: int = 0, k_scale=None, v_scale=None):
    """hybrid_layer on the library's static per-device scratch: no workspace, and nothing
    is allocated here either (`out` is required). Calls on one device must not overlap.
    Returns out."""
    torch = _torch()
    _prep(q, k_cache, v_cache, out, kv_indptr)
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    _opt(s, torch.int32, "s"); _opt(s_out, torch.int32, "s_out")
    _opt(s_indptr, torch.int64, "s_indptr"); _opt(scores_out, torch.float32, "scores_out")
    if s_out is None:
        s_out = s
    k = _clamp_k(shape, k, s_indptr, [("s", s), ("s_out", s_out)])
    _sizes(shape, q, out, k, kv_indptr, [("s", s), ("s_out", s_out)], s_indptr, scores_out)
    _check(load_library().ld_hybrid_layer_noalloc(
        ctypes.byref(shape), int(retrieval_mask), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), int(k), _ptr(s), _ptr(s_out), _ptr(s_indptr), _ptr(scores_out),
        out.data_ptr(), int(flags), _stream()), "ld_hybrid_layer_noalloc")
    return out


def hysparse_layer(q, k_cache, v_cache, k: int, s_in, k_window, v_window, gate, *, s_indptr=None,
                   out=None, flags: int = 0, workspace: Optional[HySparseWorkspace] = None,
                   kv_indptr=None, seq_len=None, scale=None, block_table=None, page_size: int = 0,
                   k_scale=None, v_scale=None):
    """HySparse sparse layer: block-sparse attention over rows S of the shared cache,
    window attention over the layer's own cache k_window/v_window [Hkv][B*W][d] (the
    last W tokens of each sequence), combined as w*O_s + (1-w)*O_w, w = sigmoid(gate)
    with gate fp32 [B][Hq]. Returns out."""
    torch = _torch()
    out = _prep(q, k_cache, v_cache, out, kv_indptr)
    shape = make_shape(q, k_cache, kv_indptr, seq_len, scale, block_table, page_size, k_scale, v_scale)
    _req(s_in, torch.int32, "s_in"); _opt(s_indptr, torch.int64, "s_indptr")
    _req(k_window, torch.bfloat16, "k_window"); _req(v_window, torch.bfloat16, "v_window")
    _req(gate, torch.float32, "gate")
    B, Hq = q.shape[0], q.shape[1]
    if k_window.shape != v_window.shape or k_window.dim() != 3 or k_window.shape[0] != shape.num_kv_heads \
            or k_window.shape[1] % B != 0 or k_window.shape[2] != q.shape[2]:
        raise ValueError("k_window/v_window must be [Hkv][B*W][d] and match each other")
    if gate.numel() != B * Hq:
        raise ValueError("gate must hold B*Hq values")
    k = _clamp_k(shape, k, s_indptr, [("s_in", s_in)])
    _sizes(shape, q, out, k, kv_indptr, [("s_in", s_in)], s_indptr)
    W = k_window.shape[1] // B
    ws = workspace or _default_ws("hysparse", _layout_key(shape, k, W),
                                  lambda: HySparseWorkspace(shape, k, W, q.device), q.device)
    _check(load_library().ld_hysparse_layer(
        ctypes.byref(shape), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), int(k),
        s_in.data_ptr(), _ptr(s_indptr), k_window.data_ptr(), v_window.data_ptr(), int(W),
        gate.data_ptr(), out.data_ptr(), int(flags), ws.ptr(), ws.nbytes, _stream()),
        "ld_hysparse_layer")
    return out


def prefill_hybrid_layer(q, k_cache, v_cache, retrieval_mask: int, k: int, s, *, batch: int = 1,
                         s_out=None, importance_out=None, out=None, flags: int = 0,
                         workspace: Optional[PrefillWorkspace] = None, scale=None):
    """One hybrid-head layer over a causal prefill of T prompt tokens per sequence:
    q [Hq][B*T][d], k_cache / v_cache [Hkv][B*T][d] (bf16), B = batch. Retrieval heads
    run causal full attention and write argsTopK of their attention matrix's column sums
    to their rows of s_out ([B][Hq][k] int32, ascending); sparse heads attend, row by row,
    to the tokens of their row of `s` at or before the row (s is None only when every
    head retrieves). importance_out: optional fp32 [B][Hq][T] column sums. Returns out."""
    torch = _torch()
    _req(q, torch.bfloat16, "q"); _req(k_cache, torch.bfloat16, "k_cache"); _req(v_cache, torch.bfloat16, "v_cache")
    if q.dim() != 3 or k_cache.dim() != 3 or k_cache.shape != v_cache.shape:
        raise ValueError("q, k_cache, v_cache must be 3-D with equal K/V shapes")
    B = int(batch)
    Hq, BT, d = (int(x) for x in q.shape)
    if B < 1 or BT % B or k_cache.shape[1] != BT or k_cache.shape[2] != d:
        raise ValueError("q must be [Hq][B*T][d] and k_cache [Hkv][B*T][d]")
    T = BT // B
    shape = tsa_shape(q, k_cache, B, scale)
    kk = min(int(k), T)                                   # the pages' k = min(k, seq_len)
    _opt(s, torch.int32, "s"); _opt(s_out, torch.int32, "s_out")
    _opt(importance_out, torch.float32, "importance_out")
    if s_out is None:
        s_out = s
    for name, t in (("s", s), ("s_out", s_out)):
        if t is not None and t.numel() != B * Hq * kk:
            raise ValueError(f"{name} must hold B*Hq*min(k, T) = {B * Hq * kk} entries")
    if importance_out is not None and importance_out.numel() != B * Hq * T:
        raise ValueError("importance_out must hold B*Hq*T entries")
    if out is None:
        out = torch.empty_like(q)
    _req(out, torch.bfloat16, "out")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    ws = workspace or _default_ws("prefill", _layout_key(shape, kk), lambda: PrefillWorkspace(shape, kk, q.device),
                                  q.device)
    _check(load_library().ld_prefill_hybrid_layer(
        ctypes.byref(shape), int(retrieval_mask), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kk,
        _ptr(s), _ptr(s_out), _ptr(importance_out), out.data_ptr(), int(flags), ws.ptr(), ws.nbytes, _stream()),
        "ld_prefill_hybrid_layer")
    return out


def tsa_attention(q, k_cache, v_cache, scores, k: int, *, idx_out=None, out=None, causal: bool = False,
                  zero_fill: bool = True, workspace: Optional[TsaWorkspace] = None, scale=None,
                  given_idx: bool = False, batch: Optional[int] = None):
    """Token Sparse Attention over a prefill: per (sequence, head) the top-k tokens of
    `scores` [B][Hq][T] (fp32), dense attention among them, scattered to their rows of
    `out` [Hq][B*T][d]. q [Hq][B*T][d], k_cache / v_cache [Hkv][B*T][d] (bf16).
    given_idx: skip the selection and use idx_out as given (scores may be None; then
    `batch` gives B). Returns (out, idx_out [B][Hq][min(k, T)] int32 ascending)."""
    torch = _torch()
    _req(q, torch.bfloat16, "q"); _req(k_cache, torch.bfloat16, "k_cache"); _req(v_cache, torch.bfloat16, "v_cache")
    if scores is not None:
        _req(scores, torch.float32, "scores")
        if scores.dim() != 3:
            raise ValueError("scores must be [B][Hq][T]")
        B, Hq, T = (int(x) for x in scores.shape)
    elif given_idx and batch:
        B, Hq = int(batch), int(q.shape[0])
        T = int(q.shape[1]) // B
    else:
        raise ValueError("scores are required unless given_idx is set with batch")
    if q.dim() != 3 or k_cache.shape != v_cache.shape or k_cache.dim() != 3:
        raise ValueError("q, k_cache, v_cache must be 3-D with equal K/V shapes")
    if given_idx and idx_out is None:
        raise ValueError("given_idx needs idx_out")
    if q.shape[0] != Hq or q.shape[1] != B * T or k_cache.shape[1] != B * T or k_cache.shape[2] != q.shape[2]:
        raise ValueError("q must be [Hq][B*T][d] and k_cache [Hkv][B*T][d] for scores [B][Hq][T]")
    shape = tsa_shape(q, k_cache, B, scale)
    kk = min(int(k), T)
    if idx_out is None:
        idx_out = torch.empty((B, Hq, kk), dtype=torch.int32, device=q.device)
    _req(idx_out, torch.int32, "idx_out")
    if idx_out.numel() != B * Hq * kk:
        raise ValueError("idx_out must hold B*Hq*min(k, T) entries")
    if out is None:
        out = torch.empty_like(q)
    _req(out, torch.bfloat16, "out")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    flags = (TSA_CAUSAL if causal else 0) | (TSA_ZERO_FILL if zero_fill else 0) | (TSA_GIVEN_IDX if given_idx else 0)
    ws = workspace or _default_ws("tsa", _layout_key(shape, k), lambda: TsaWorkspace(shape, k, q.device), q.device)
    _check(load_library().ld_tsa_attention(
        ctypes.byref(shape), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), _ptr(scores), int(k),
        idx_out.data_ptr(), out.data_ptr(), int(flags), ws.ptr(), ws.nbytes, _stream()), "ld_tsa_attention")
    return out, idx_out


def topk_select(scores, k: int, *, idx_out=None, val_out=None, n_per_row=None, k_per_row=None,
                idx_indptr=None, workspace: Optional[TopkWorkspace] = None):
    """argsTopK of each row of a 2-D fp32 tensor [rows][n]. Row r holds
    n_r = n_per_row[r] (int32 device tensor, default n) scores and keeps
    k_r = min(k_per_row[r] (default k), n_r) indices, in ascending order. Output: dense
    [rows][k] int32 (rows with k_r < k keep their tail), or CSR into the 1-D idx_out at
    offsets idx_indptr (int64 device tensor [rows+1]; capacity per row, which also
    bounds k_r). Returns idx_out."""
    torch = _torch()
    if scores.dim() != 2:
        raise ValueError("scores must be 2-D [rows][n]")
    rows, n = scores.shape
    row_stride = scores.stride(0) if rows > 1 else n     # a size-1 dim has no meaningful stride
    if (n > 1 and scores.stride(1) != 1) or row_stride < n:
        raise ValueError("scores must have unit stride along each row")
    if not scores.is_cuda or scores.dtype != torch.float32:
        raise ValueError("scores must be a float32 device tensor")
    k = int(k)
    if k < 1:
        raise ValueError("k must be at least 1")
    for name, t in (("n_per_row", n_per_row), ("k_per_row", k_per_row)):
        _opt(t, torch.int32, name)
        if t is not None and t.numel() != rows:
            raise ValueError(f"{name} must hold one entry per row")
    if idx_indptr is not None:
        _req(idx_indptr, torch.int64, "idx_indptr")
        if idx_indptr.numel() != rows + 1:
            raise ValueError("idx_indptr must hold rows+1 offsets")
        if idx_out is None:
            raise ValueError("CSR output needs idx_out")
        # device-side offsets bound the kernels' writes: check them once here
        off = idx_indptr.cpu()
        need = int(off[-1])
        if int(off[0]) < 0 or bool((off[1:] < off[:-1]).any()):
            raise ValueError("idx_indptr must be non-negative and non-decreasing")
        cap = need
    else:
        if idx_out is None:
            idx_out = torch.empty((rows, min(k, n)), dtype=torch.int32, device=scores.device)
            k_stride = min(k, n)
        else:
            k_stride = k
        cap = rows * k_stride
        k = k_stride
    _req(idx_out, torch.int32, "idx_out"); _opt(val_out, torch.float32, "val_out")
    for name, t in (("idx_out", idx_out), ("val_out", val_out)):
        if t is not None and t.numel() < cap:
            raise ValueError(f"{name} must hold {cap} entries")
    ws = workspace or _default_ws("topk", (rows, n), lambda: TopkWorkspace(rows, n, scores.device), scores.device)
    _check(load_library().ld_topk_select(
        scores.data_ptr(), int(rows), int(n), int(row_stride), _ptr(n_per_row), int(k), _ptr(k_per_row),
        idx_out.data_ptr(), _ptr(idx_indptr), _ptr(val_out), ws.ptr(), ws.nbytes, _stream()), "ld_topk_select")
    return idx_out
