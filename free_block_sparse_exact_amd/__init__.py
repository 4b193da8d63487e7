"""Python binding of liblosa.so: retained-mass block-sparse self-attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/losa.h``).  PyTorch provides device
memory (tensors) and the stream; there is no CPU or PyTorch fallback -- if
the library is missing, importing works but every call raises.

The functions carry the C names:

    losa_block_mass(q, k, tokens, q_block, k_block)            -> M
    losa_select(M, p, tokens, q_block, k_block, ...)          -> (row_ptr, col_idx, order)
    losa_sparse_attn(q, k, v, row_ptr, col_idx, order, ...)   -> O
    losa_dense_attn_mass(q, k, v, tokens, q_block, k_block)   -> (O, M)
    losa_sparse_attn_mass(q, k, v, row_ptr, col_idx, order, ...) -> (O, M within the lists)
    losa_pooled_mass(q, k, tokens, q_block, k_block)          -> P
    losa_retained_mass(M, row_ptr, col_idx, ...)              -> kept [rows, 2]

Workspaces are allocated per call unless a tensor is passed as ``ws`` (any
dtype; its size in bytes is what counts).

Tensors are [batch, heads, tokens_alloc, head_dim] CUDA tensors (bf16 or
fp32) whose last axis is contiguous.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple, Union

__all__ = [
    "LosaError",
    "LIB_PATH",
    "load_library",
    "Geometry",
    "losa_abi_version",
    "losa_block_mass_workspace",
    "losa_block_mass",
    "losa_select_workspace",
    "losa_select",
    "losa_select_noalloc",
    "SELECT_SCRATCH_BYTES",
    "losa_sparse_attn_workspace",
    "losa_sparse_attn",
    "losa_retained_mass",
    "losa_sparse_attn_threshold_workspace",
    "losa_sparse_attn_threshold",
    "losa_dense_attn_mass_workspace",
    "losa_dense_attn_mass",
    "losa_sparse_attn_mass_workspace",
    "losa_sparse_attn_mass",
    "losa_pooled_mass_workspace",
    "losa_pooled_mass",
    "losa_select_threshold_workspace",
    "losa_select_threshold",
    "losa_qk_drift_workspace",
    "losa_qk_drift",
    "losa_merge_lists_workspace",
    "losa_merge_lists",
    "LOSA_F32",
    "LOSA_BF16",
    "STATUS",
]

# The library built next to this file (free_block_sparse_exact_amd._build); no other is ever loaded.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblosa.so")

LOSA_F32 = 0
LOSA_BF16 = 1
SELECT_SCRATCH_BYTES = 32 << 20  # LOSA_SELECT_SCRATCH_BYTES
STATUS = {
    0: "LOSA_OK",
    1: "LOSA_ERR_NULL",
    2: "LOSA_ERR_INVALID_ARG",
    3: "LOSA_ERR_UNSUPPORTED",
    4: "LOSA_ERR_WORKSPACE",
    5: "LOSA_ERR_CAPACITY",
    6: "LOSA_ERR_HIP",
}


class LosaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class losa_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("tokens", ctypes.c_int32),
        ("tokens_alloc", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_block", ctypes.c_int32),
        ("k_block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load liblosa.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m free_block_sparse_exact_amd._build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.POINTER(losa_shape)
    sz = ctypes.POINTER(ctypes.c_size_t)
    i32 = ctypes.c_int32
    sig = {
        "losa_abi_version": ([], i32),
        "losa_status_string": ([i32], ctypes.c_char_p),
        "losa_block_mass_workspace": ([S, sz], i32),
        "losa_block_mass": ([S, P, P, P, P, ctypes.c_size_t, P], i32),
        "losa_select_workspace": ([S, sz], i32),
        "losa_select": ([S, P, ctypes.POINTER(ctypes.c_double), i32, P, P, ctypes.c_int64, P, P,
                         ctypes.c_size_t, P], i32),
        "losa_select_noalloc": ([S, P, ctypes.POINTER(ctypes.c_double), i32, P, P, ctypes.c_int64, P, P], i32),
        "losa_sparse_attn_workspace": ([S, sz], i32),
        "losa_sparse_attn": ([S, P, P, P, P, P, P, P, i32, P, ctypes.c_size_t, P], i32),
        "losa_retained_mass": ([S, P, P, P, P, P], i32),
        "losa_sparse_attn_threshold_workspace": ([S, sz], i32),
        "losa_sparse_attn_threshold": ([S, P, P, P, ctypes.POINTER(ctypes.c_double), i32, P, i32, P, P, P,
                                        ctypes.c_size_t, P], i32),
        "losa_dense_attn_mass_workspace": ([S, sz], i32),
        "losa_dense_attn_mass": ([S, P, P, P, P, P, i32, P, ctypes.c_size_t, P], i32),
        "losa_sparse_attn_mass_workspace": ([S, sz], i32),
        "losa_sparse_attn_mass": ([S, P, P, P, P, P, P, P, P, i32, P, ctypes.c_size_t, P], i32),
        "losa_pooled_mass_workspace": ([S, sz], i32),
        "losa_pooled_mass": ([S, P, P, P, P, ctypes.c_size_t, P], i32),
        "losa_select_threshold_workspace": ([S, sz], i32),
        "losa_select_threshold": ([S, P, ctypes.POINTER(ctypes.c_double), i32, P, P, ctypes.c_int64, P, P,
                                   ctypes.c_size_t, P], i32),
        "losa_qk_drift_workspace": ([S, sz], i32),
        "losa_qk_drift": ([S, P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_size_t, P], i32),
        "losa_merge_lists_workspace": ([S, sz], i32),
        "losa_merge_lists": ([S, P, P, P, P, P, P, P, ctypes.c_int64, P, P, ctypes.c_size_t, P], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _L() -> ctypes.CDLL:
    return load_library()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise LosaError(status, where)


@dataclass(frozen=True)
class Geometry:
    """Block geometry of one attention layer (mirrors losa_shape)."""
    batch: int
    heads: int
    tokens: int
    tokens_alloc: int
    head_dim: int
    q_block: int
    k_block: int
    dtype: int
    softmax_scale: float = 0.0

    @property
    def n_q(self) -> int:
        return -(-self.tokens // self.q_block)

    @property
    def n_k(self) -> int:
        return -(-self.tokens // self.k_block)

    @property
    def rows(self) -> int:
        return self.batch * self.heads * self.n_q

    @staticmethod
    def of(q, tokens: int, q_block: int, k_block: int, softmax_scale: Optional[float] = None) -> "Geometry":
        import torch
        B, H, Na, d = q.shape
        dt = {torch.bfloat16: LOSA_BF16, torch.float32: LOSA_F32}.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        return Geometry(B, H, int(tokens), Na, d, int(q_block), int(k_block), dt,
                        float(softmax_scale) if softmax_scale else 0.0)

    def shape(self, q=None, k=None, v=None, o=None) -> losa_shape:
        s = losa_shape()
        s.batch, s.heads, s.tokens, s.tokens_alloc = self.batch, self.heads, self.tokens, self.tokens_alloc
        s.head_dim, s.q_block, s.k_block, s.dtype = self.head_dim, self.q_block, self.k_block, self.dtype
        s.softmax_scale = self.softmax_scale
        s.reserved = 0
        for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
            arr = getattr(s, name)
            if t is not None:
                st = t.stride()
                if st[3] != 1:
                    raise ValueError(f"{name[0]}: head_dim axis must be contiguous")
                arr[0], arr[1], arr[2] = st[0], st[1], st[2]
            else:
                d = self.head_dim
                arr[0], arr[1], arr[2] = self.heads * self.tokens_alloc * d, self.tokens_alloc * d, d
        return s


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _tstream(stream):
    """The stream a call runs on, as a torch stream: torch's current stream
    by default, a torch stream as given, or a raw hipStream_t handle."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(st) -> int:
    return st.cuda_stream


def _empty(st, *args, **kw):
    """torch.empty on the call's stream: the caching allocator then ties the
    memory to that stream, so a buffer freed when the call returns is not
    handed to work on another stream while the kernels still use it."""
    import torch
    with torch.cuda.stream(st):
        return torch.empty(*args, **kw)


def _nbytes(ws) -> int:
    """Size in bytes of a workspace tensor (any dtype), 0 for none."""
    return 0 if ws is None else ws.numel() * ws.element_size()


def _workspace(nbytes: int, device, ws, st):
    import torch
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return _empty(st, nbytes, dtype=torch.uint8, device=device)


def losa_abi_version() -> int:
    return int(_L().losa_abi_version())


def losa_block_mass_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_block_mass_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)), "losa_block_mass_workspace")
    return n.value


def losa_block_mass(q, k, tokens: int, q_block: int, k_block: int, softmax_scale: Optional[float] = None,
                    out=None, ws=None, stream=None):
    """Exact block masses M [B, H, n_q, n_k] (fp32, row-mean form)."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    shp = g.shape(q=q, k=k)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_block_mass_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_block_mass_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    if out is None:
        out = _empty(st, (g.batch, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=q.device)
    _check(_L().losa_block_mass(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(out), _ptr(ws),
                                _nbytes(ws), _stream(st)), "losa_block_mass")
    return out


def losa_select_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_select_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)), "losa_select_workspace")
    return n.value


def losa_select(M, p: Union[float, Sequence[float]], tokens: int, q_block: int, k_block: int,
                tokens_alloc: Optional[int] = None, head_dim: int = 128, dtype: int = LOSA_BF16,
                want_order: bool = True, row_ptr=None, col_idx=None, order=None, ws=None, stream=None):
    """Retained-mass lists: (row_ptr int32 [rows+1], col_idx int32 [capacity], order int32 [rows] or None).

    col_idx has capacity rows*n_k; its used length is row_ptr[-1].
    """
    import torch
    st = _tstream(stream)
    B, H, nq, nk = M.shape
    Na = tokens_alloc if tokens_alloc is not None else max(nq * q_block, nk * k_block)
    g = Geometry(B, H, int(tokens), Na, head_dim, int(q_block), int(k_block), dtype)
    if g.n_q != nq or g.n_k != nk:
        raise ValueError("M does not match tokens/q_block/k_block")
    shp = g.shape()
    pv = [float(p)] if isinstance(p, (int, float)) else [float(x) for x in p]
    parr = (ctypes.c_double * len(pv))(*pv)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_select_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_select_workspace")
    ws = _workspace(nbytes.value, M.device, ws, st)
    rows = g.rows
    dev = M.device
    if row_ptr is None:
        row_ptr = _empty(st, rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = _empty(st, rows * nk, dtype=torch.int32, device=dev)
    if want_order and order is None:
        order = _empty(st, rows, dtype=torch.int32, device=dev)
    if not want_order:
        order = None
    _check(_L().losa_select(ctypes.byref(shp), _ptr(M), parr, len(pv), _ptr(row_ptr), _ptr(col_idx),
                            col_idx.numel(), _ptr(order), _ptr(ws), _nbytes(ws),
                            _stream(st)), "losa_select")
    return row_ptr, col_idx, order


def losa_select_noalloc(M, p: Union[float, Sequence[float]], tokens: int, q_block: int, k_block: int,
                        row_ptr, col_idx, order=None, tokens_alloc: Optional[int] = None, head_dim: int = 128,
                        dtype: int = LOSA_BF16, stream=None):
    """losa_select without a workspace: the library's own device scratch array
    holds the selector's scratch.  The caller passes every output (row_ptr,
    col_idx, and order or None); nothing is allocated.  Returns them."""
    st = _tstream(stream)
    B, H, nq, nk = M.shape
    Na = tokens_alloc if tokens_alloc is not None else max(nq * q_block, nk * k_block)
    g = Geometry(B, H, int(tokens), Na, head_dim, int(q_block), int(k_block), dtype)
    if g.n_q != nq or g.n_k != nk:
        raise ValueError("M does not match tokens/q_block/k_block")
    pv = [float(p)] if isinstance(p, (int, float)) else [float(x) for x in p]
    parr = (ctypes.c_double * len(pv))(*pv)
    _check(_L().losa_select_noalloc(ctypes.byref(g.shape()), _ptr(M), parr, len(pv), _ptr(row_ptr), _ptr(col_idx),
                                    col_idx.numel(), _ptr(order), _stream(st)), "losa_select_noalloc")
    return row_ptr, col_idx, order


def losa_sparse_attn_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_sparse_attn_workspace")
    return n.value


def losa_sparse_attn(q, k, v, row_ptr, col_idx, order, tokens: int, q_block: int, k_block: int,
                     softmax_scale: Optional[float] = None, out=None, out_dtype=None, ws=None, stream=None):
    """Frozen-pattern sparse attention -> O [B, H, tokens_alloc, d] (bf16 by default for bf16 inputs)."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    if out is None:
        out = _empty(st, q.shape, dtype=out_dtype or q.dtype, device=q.device)
    odt = {torch.bfloat16: LOSA_BF16, torch.float32: LOSA_F32}[out.dtype]
    shp = g.shape(q=q, k=k, v=v, o=out)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_sparse_attn_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    _check(_L().losa_sparse_attn(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                 _ptr(order), _ptr(out), odt, _ptr(ws), _nbytes(ws),
                                 _stream(st)), "losa_sparse_attn")
    return out


def losa_sparse_attn_threshold_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_threshold_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_sparse_attn_threshold_workspace")
    return n.value


def losa_sparse_attn_threshold(q, k, v, theta: Union[float, Sequence[float]], tokens: int, q_block: int,
                               k_block: int, softmax_scale: Optional[float] = None, out=None, out_dtype=None,
                               kept_count=None, kept_mask=None, want_kept: bool = True, ws=None, stream=None):
    """Sparse attention with on-the-fly block thresholding against the pooled
    proxy (blocks chosen inside the attention kernel, no proxy matrix) ->
    (O, kept_count int32 [rows] or None, kept_mask int32 [rows, ceil(n_k/32)] or None)."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    if out is None:
        out = _empty(st, q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if want_kept and kept_count is None:
        kept_count = _empty(st, g.rows, dtype=torch.int32, device=q.device)
    if want_kept and kept_mask is None:
        kept_mask = _empty(st, (g.rows, (g.n_k + 31) // 32), dtype=torch.int32, device=q.device)
    odt = {torch.bfloat16: LOSA_BF16, torch.float32: LOSA_F32}[out.dtype]
    shp = g.shape(q=q, k=k, v=v, o=out)
    tv = [float(theta)] if isinstance(theta, (int, float)) else [float(x) for x in theta]
    tarr = (ctypes.c_double * len(tv))(*tv)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_threshold_workspace(ctypes.byref(shp), ctypes.byref(nbytes)),
           "losa_sparse_attn_threshold_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    _check(_L().losa_sparse_attn_threshold(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), tarr, len(tv), _ptr(out),
                                           odt, _ptr(kept_count), _ptr(kept_mask), _ptr(ws), _nbytes(ws),
                                           _stream(st)), "losa_sparse_attn_threshold")
    return out, kept_count, kept_mask


def losa_dense_attn_mass_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_dense_attn_mass_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_dense_attn_mass_workspace")
    return n.value


def losa_dense_attn_mass(q, k, v, tokens: int, q_block: int, k_block: int, softmax_scale: Optional[float] = None,
                         out=None, out_dtype=None, M=None, ws=None, stream=None):
    """Dense attention and exact block masses in one pass -> (O [B, H, tokens_alloc, d], M [B, H, n_q, n_k])."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    if out is None:
        out = _empty(st, q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if M is None:
        M = _empty(st, (g.batch, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=q.device)
    odt = {torch.bfloat16: LOSA_BF16, torch.float32: LOSA_F32}[out.dtype]
    shp = g.shape(q=q, k=k, v=v, o=out)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_dense_attn_mass_workspace(ctypes.byref(shp), ctypes.byref(nbytes)),
           "losa_dense_attn_mass_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    _check(_L().losa_dense_attn_mass(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(M), _ptr(out), odt,
                                     _ptr(ws), _nbytes(ws), _stream(st)),
           "losa_dense_attn_mass")
    return out, M


def losa_sparse_attn_mass_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_mass_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_sparse_attn_mass_workspace")
    return n.value


def losa_sparse_attn_mass(q, k, v, row_ptr, col_idx, order, tokens: int, q_block: int, k_block: int,
                          softmax_scale: Optional[float] = None, out=None, out_dtype=None, M=None, ws=None,
                          stream=None):
    """Sparse attention over the lists and the exact masses within them ->
    (O [B, H, tokens_alloc, d], M [B, H, n_q, n_k], 0 outside the lists)."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    if out is None:
        out = _empty(st, q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if M is None:
        M = _empty(st, (g.batch, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=q.device)
    odt = {torch.bfloat16: LOSA_BF16, torch.float32: LOSA_F32}[out.dtype]
    shp = g.shape(q=q, k=k, v=v, o=out)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_sparse_attn_mass_workspace(ctypes.byref(shp), ctypes.byref(nbytes)),
           "losa_sparse_attn_mass_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    _check(_L().losa_sparse_attn_mass(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                      _ptr(order), _ptr(M), _ptr(out), odt, _ptr(ws), _nbytes(ws),
                                      _stream(st)), "losa_sparse_attn_mass")
    return out, M


def losa_pooled_mass_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_pooled_mass_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)), "losa_pooled_mass_workspace")
    return n.value


def losa_pooled_mass(q, k, tokens: int, q_block: int, k_block: int, softmax_scale: Optional[float] = None,
                     out=None, ws=None, stream=None):
    """Pooled proxy masses P [B, H, n_q, n_k] (fp32): block-mean Q against block-mean K,
    block-weighted softmax over key blocks."""
    import torch
    st = _tstream(stream)
    g = Geometry.of(q, tokens, q_block, k_block, softmax_scale)
    if out is None:
        out = _empty(st, (g.batch, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=q.device)
    shp = g.shape(q=q, k=k)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_pooled_mass_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_pooled_mass_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    _check(_L().losa_pooled_mass(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(out), _ptr(ws),
                                 _nbytes(ws), _stream(st)), "losa_pooled_mass")
    return out


def losa_retained_mass(M, row_ptr, col_idx, tokens: int, q_block: int, k_block: int, out=None, stream=None):
    """Per-row (kept mass, total mass) of M under the lists -> fp32 [rows, 2]."""
    import torch
    st = _tstream(stream)
    B, H, nq, nk = M.shape
    g = Geometry(B, H, int(tokens), max(nq * q_block, nk * k_block), 128, int(q_block), int(k_block), LOSA_BF16)
    if out is None:
        out = _empty(st, (g.rows, 2), dtype=torch.float32, device=M.device)
    _check(_L().losa_retained_mass(ctypes.byref(g.shape()), _ptr(M), _ptr(row_ptr), _ptr(col_idx), _ptr(out),
                                   _stream(st)), "losa_retained_mass")
    return out


def losa_select_threshold_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_select_threshold_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_select_threshold_workspace")
    return n.value


def losa_select_threshold(M, theta: Union[float, Sequence[float]], tokens: int, q_block: int, k_block: int,
                          tokens_alloc: Optional[int] = None, want_order: bool = True, row_ptr=None, col_idx=None,
                          order=None, ws=None, stream=None):
    """Online block thresholding lists (block j kept when its mass is at least
    theta times the running maximum): (row_ptr, col_idx, order or None), as
    losa_select returns them."""
    import torch
    st = _tstream(stream)
    B, H, nq, nk = M.shape
    Na = tokens_alloc if tokens_alloc is not None else max(nq * q_block, nk * k_block)
    g = Geometry(B, H, int(tokens), Na, 128, int(q_block), int(k_block), LOSA_BF16)
    if g.n_q != nq or g.n_k != nk:
        raise ValueError("M does not match tokens/q_block/k_block")
    shp = g.shape()
    tv = [float(theta)] if isinstance(theta, (int, float)) else [float(x) for x in theta]
    tarr = (ctypes.c_double * len(tv))(*tv)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_select_threshold_workspace(ctypes.byref(shp), ctypes.byref(nbytes)),
           "losa_select_threshold_workspace")
    dev = M.device
    ws = _workspace(nbytes.value, dev, ws, st)
    rows = g.rows
    if row_ptr is None:
        row_ptr = _empty(st, rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = _empty(st, rows * nk, dtype=torch.int32, device=dev)
    if want_order and order is None:
        order = _empty(st, rows, dtype=torch.int32, device=dev)
    if not want_order:
        order = None
    _check(_L().losa_select_threshold(ctypes.byref(shp), _ptr(M), tarr, len(tv), _ptr(row_ptr), _ptr(col_idx),
                                      col_idx.numel(), _ptr(order), _ptr(ws), _nbytes(ws), _stream(st)),
           "losa_select_threshold")
    return row_ptr, col_idx, order


def losa_qk_drift_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_qk_drift_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)), "losa_qk_drift_workspace")
    return n.value


def losa_qk_drift(q, k, q_ref, k_ref, tokens: int, tau: float, q_block: int = 64, k_block: int = 64,
                  drift=None, refresh=None, ws=None, stream=None):
    """Drift of Q and K per (batch, head) since the reference step and the heads
    to refresh: (drift fp64 [B, H, 2], refresh int32 [B, H])."""
    import torch
    st = _tstream(stream)
    if q_ref.shape != q.shape or k_ref.shape != k.shape or q_ref.stride() != q.stride() \
            or k_ref.stride() != k.stride() or {q_ref.dtype, k_ref.dtype, k.dtype} != {q.dtype}:
        raise ValueError("q_ref/k_ref must match q/k in shape, strides and dtype")
    g = Geometry.of(q, tokens, q_block, k_block)
    shp = g.shape(q=q, k=k)
    nbytes = ctypes.c_size_t()
    _check(_L().losa_qk_drift_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_qk_drift_workspace")
    ws = _workspace(nbytes.value, q.device, ws, st)
    if drift is None:
        drift = _empty(st, (g.batch, g.heads, 2), dtype=torch.float64, device=q.device)
    if refresh is None:
        refresh = _empty(st, (g.batch, g.heads), dtype=torch.int32, device=q.device)
    _check(_L().losa_qk_drift(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(q_ref), _ptr(k_ref), float(tau),
                              _ptr(drift), _ptr(refresh), _ptr(ws), _nbytes(ws), _stream(st)), "losa_qk_drift")
    return drift, refresh


def losa_merge_lists_workspace(geom: Geometry) -> int:
    n = ctypes.c_size_t()
    _check(_L().losa_merge_lists_workspace(ctypes.byref(geom.shape()), ctypes.byref(n)),
           "losa_merge_lists_workspace")
    return n.value


def losa_merge_lists(take_b, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, tokens: int, q_block: int, k_block: int,
                     tokens_alloc: Optional[int] = None, want_order: bool = True, row_ptr=None, col_idx=None,
                     order=None, ws=None, stream=None):
    """Lists of the heads flagged in take_b [B, H] from set b, the others from
    set a: (row_ptr, col_idx, order or None), as losa_select returns them."""
    import torch
    st = _tstream(stream)
    B, H = take_b.shape
    n_q, n_k = -(-int(tokens) // q_block), -(-int(tokens) // k_block)
    Na = tokens_alloc if tokens_alloc is not None else max(n_q * q_block, n_k * k_block)
    g = Geometry(B, H, int(tokens), Na, 128, int(q_block), int(k_block), LOSA_BF16)
    shp = g.shape()
    nbytes = ctypes.c_size_t()
    _check(_L().losa_merge_lists_workspace(ctypes.byref(shp), ctypes.byref(nbytes)), "losa_merge_lists_workspace")
    dev = take_b.device
    ws = _workspace(nbytes.value, dev, ws, st)
    rows = g.rows
    if row_ptr is None:
        row_ptr = _empty(st, rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = _empty(st, rows * n_k, dtype=torch.int32, device=dev)
    if want_order and order is None:
        order = _empty(st, rows, dtype=torch.int32, device=dev)
    if not want_order:
        order = None
    _check(_L().losa_merge_lists(ctypes.byref(shp), _ptr(take_b), _ptr(row_ptr_a), _ptr(col_idx_a),
                                 _ptr(row_ptr_b), _ptr(col_idx_b), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                 _ptr(order), _ptr(ws), _nbytes(ws), _stream(st)), "losa_merge_lists")
    return row_ptr, col_idx, order
