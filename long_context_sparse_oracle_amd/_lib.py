"""ctypes binding of libctxsparse.so (C ABI declared in include/ctxsparse.h).

Argument marshalling only: shapes and pointers are read from torch tensors, outputs and
workspaces are allocated with torch when the caller passes none, and every step of the
computation runs in the library's HIP kernels on the current torch stream.  There is no CPU
fallback: importing this module without the built library raises ImportError.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple, Union

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libctxsparse.so")

CS_OK = 0
CS_KV_CONTIGUOUS = 0
CS_KV_PAGED = 1
STATUS_NAMES = {
    0: "CS_OK",
    1: "CS_ERR_INVALID_ARG",
    2: "CS_ERR_UNSUPPORTED",
    3: "CS_ERR_WORKSPACE_TOO_SMALL",
    4: "CS_ERR_HIP",
    5: "CS_ERR_SCRATCH_LIMIT",
}
EXPORTS = (
    "cs_status_str",
    "cs_version",
    "topk_index_workspace_size",
    "topk_index",
    "sparse_decode_attn_workspace_size",
    "sparse_decode_attn",
    "sparse_decode_attn_noalloc",
    "dense_decode_attn_workspace_size",
    "dense_decode_attn",
    "sparse_decode_step_workspace_size",
    "sparse_decode_step",
    "key_sketch_build",
    "topk_index_sketch_workspace_size",
    "topk_index_sketch",
    "sparse_decode_step_sketch_workspace_size",
    "sparse_decode_step_sketch",
)


class DecodeShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class KVDesc(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("layout", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


class KeySketchDesc(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_oracle_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sz = ctypes.c_size_t
    i32 = ctypes.c_int32
    f32 = ctypes.c_float
    shp = ctypes.POINTER(DecodeShape)
    kvp = ctypes.POINTER(KVDesc)
    lib.cs_status_str.argtypes = [ctypes.c_int]
    lib.cs_status_str.restype = ctypes.c_char_p
    lib.cs_version.argtypes = []
    lib.cs_version.restype = i32
    lib.topk_index_workspace_size.argtypes = [shp, kvp, i32]
    lib.topk_index_workspace_size.restype = sz
    lib.topk_index.argtypes = [shp, P, kvp, f32, P, i32, P, P, sz, P]
    lib.topk_index.restype = ctypes.c_int
    lib.sparse_decode_attn_workspace_size.argtypes = [shp, i32, i32]
    lib.sparse_decode_attn_workspace_size.restype = sz
    lib.sparse_decode_attn.argtypes = [shp, P, kvp, P, i32, f32, i32, P, P, P, sz, P]
    lib.sparse_decode_attn.restype = ctypes.c_int
    lib.sparse_decode_attn_noalloc.argtypes = [shp, P, kvp, P, i32, f32, i32, P, P, P]
    lib.sparse_decode_attn_noalloc.restype = ctypes.c_int
    lib.dense_decode_attn_workspace_size.argtypes = [shp, kvp, i32]
    lib.dense_decode_attn_workspace_size.restype = sz
    lib.dense_decode_attn.argtypes = [shp, P, kvp, f32, i32, P, P, P, sz, P]
    lib.dense_decode_attn.restype = ctypes.c_int
    lib.sparse_decode_step_workspace_size.argtypes = [shp, kvp, i32]
    lib.sparse_decode_step_workspace_size.restype = sz
    lib.sparse_decode_step.argtypes = [shp, P, kvp, f32, P, i32, P, P, P, P, sz, P]
    lib.sparse_decode_step.restype = ctypes.c_int
    skp = ctypes.POINTER(KeySketchDesc)
    lib.key_sketch_build.argtypes = [shp, kvp, i32, skp, P]
    lib.key_sketch_build.restype = ctypes.c_int
    lib.topk_index_sketch_workspace_size.argtypes = [shp, kvp, i32, i32]
    lib.topk_index_sketch_workspace_size.restype = sz
    lib.topk_index_sketch.argtypes = [shp, P, kvp, skp, f32, P, i32, i32, P, P, sz, P]
    lib.topk_index_sketch.restype = ctypes.c_int
    lib.sparse_decode_step_sketch_workspace_size.argtypes = [shp, kvp, i32, i32]
    lib.sparse_decode_step_sketch_workspace_size.restype = sz
    lib.sparse_decode_step_sketch.argtypes = [shp, P, kvp, skp, f32, P, i32, i32, P, P, P, P, sz, P]
    lib.sparse_decode_step_sketch.restype = ctypes.c_int
    return lib


LIB = _load()


class CtxSparseError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")


def _check(fn: str, status: int) -> None:
    if status != CS_OK:
        raise CtxSparseError(fn, status)


class KVCache:
    """A bf16 KV cache resident on the GPU (tensors stay owned by the caller).

    contiguous: k, v [B, Hkv, max_len, d]
    paged:      k, v [num_pages, Hkv, page_size, d] with page_table int32 [B, max_pages]
    seq_lens:   int32 [B] on the same device (L_b, counting the new tokens)
    max_len:    host-side bound on every L_b (defaults to the buffer capacity)
    """

    def __init__(
        self,
        k: torch.Tensor,
        v: torch.Tensor,
        seq_lens: torch.Tensor,
        *,
        page_table: Optional[torch.Tensor] = None,
        max_len: Optional[int] = None,
    ):
        if k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
            raise TypeError("K and V must be bfloat16")
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("K and V must share a 4-d shape")
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("K and V must be contiguous")
        if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
            raise TypeError("seq_lens must be a contiguous int32 tensor")
        self.k, self.v, self.seq_lens = k, v, seq_lens
        self.page_table = page_table
        self.num_kv_heads = int(k.shape[1])
        self.head_dim = int(k.shape[3])
        if page_table is None:
            self.layout = CS_KV_CONTIGUOUS
            self.page_size = 0
            self.max_pages = 0
            self.num_pages = 0
            self.max_len = int(k.shape[2]) if max_len is None else int(max_len)
        else:
            if page_table.dtype != torch.int32 or not page_table.is_contiguous():
                raise TypeError("page_table must be a contiguous int32 tensor")
            self.layout = CS_KV_PAGED
            self.page_size = int(k.shape[2])
            self.max_pages = int(page_table.shape[1])
            self.num_pages = int(k.shape[0])
            self.max_len = self.max_pages * self.page_size if max_len is None else int(max_len)

    def desc(self) -> KVDesc:
        return KVDesc(
            self.k.data_ptr(),
            self.v.data_ptr(),
            self.layout,
            self.max_len,
            self.page_size,
            self.max_pages,
            self.num_pages,
            0 if self.page_table is None else self.page_table.data_ptr(),
            self.seq_lens.data_ptr(),
        )


def _shape(q: torch.Tensor, cache: KVCache) -> DecodeShape:
    if q.dtype != torch.bfloat16 or q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous bfloat16 tensor [B, T, Hq, d]")
    B, T, Hq, d = (int(x) for x in q.shape)
    if d != cache.head_dim:
        raise ValueError("q and the cache disagree on head_dim")
    return DecodeShape(B, T, Hq, cache.num_kv_heads, d)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _scale(d: int, sm_scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Tuple[int, int]:
    if nbytes == 0:
        return 0, 0
    if ws is None:
        # freed on return; torch's caching allocator reuses it only in stream order
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _k_arg(k, k_max, shp, device):
    """(k tensor kept alive, device pointer or 0, k_max) from an int or an int32 tensor [B]."""
    if isinstance(k, torch.Tensor):
        if k.dtype != torch.int32 or not k.is_contiguous():
            raise TypeError("k per request must be a contiguous int32 tensor")
        if k_max is None:
            raise ValueError("k_max is required with a per-request k tensor")
        return k, k.data_ptr(), int(k_max)
    k_max = int(k) if k_max is None else int(k_max)
    if int(k) == k_max:
        return k, 0, k_max
    kt = torch.full((shp.batch,), int(k), dtype=torch.int32, device=device)
    return kt, kt.data_ptr(), k_max


def topk_index_workspace_size(q: torch.Tensor, cache: KVCache, k_max: int) -> int:
    shp = _shape(q, cache)
    desc = cache.desc()
    return int(LIB.topk_index_workspace_size(ctypes.byref(shp), ctypes.byref(desc), int(k_max)))


def topk_index(
    q: torch.Tensor,
    cache: KVCache,
    k: Union[int, torch.Tensor],
    *,
    k_max: Optional[int] = None,
    sm_scale: Optional[float] = None,
    indices: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Oracle top-k indexer: int32 [B, T, Hq, k_max] of selected positions per row (ascending,
    -1 padded).  `k` is one int for every request or an int32 device tensor [B]."""
    shp = _shape(q, cache)
    k, kptr, k_max = _k_arg(k, k_max, shp, q.device)
    if indices is None:
        indices = torch.empty((shp.batch, shp.q_len, shp.num_q_heads, k_max), dtype=torch.int32,
                              device=q.device)
    desc = cache.desc()
    need = int(LIB.topk_index_workspace_size(ctypes.byref(shp), ctypes.byref(desc), k_max))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.topk_index(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc),
                        _scale(shp.head_dim, sm_scale), kptr, k_max, indices.data_ptr(), wptr,
                        wbytes, _stream(q))
    _check("topk_index", st)
    return indices


def sparse_decode_attn_workspace_size(q: torch.Tensor, cache: KVCache, k_max: int,
                                      num_splits: int = 0) -> int:
    shp = _shape(q, cache)
    return int(LIB.sparse_decode_attn_workspace_size(ctypes.byref(shp), int(k_max), int(num_splits)))


def _outputs(shp: DecodeShape, device, out, lse):
    if out is None:
        out = torch.empty((shp.batch, shp.q_len, shp.num_q_heads, shp.head_dim), dtype=torch.float32,
                          device=device)
    if lse is None:
        lse = torch.empty((shp.batch, shp.q_len, shp.num_q_heads), dtype=torch.float32, device=device)
    return out, lse


def sparse_decode_attn(
    q: torch.Tensor,
    cache: KVCache,
    indices: torch.Tensor,
    *,
    sm_scale: Optional[float] = None,
    num_splits: int = 0,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention over index lists int32 [B, T, Hq, k_max]: returns (out fp32 [B, T, Hq, d],
    lse fp32 [B, T, Hq])."""
    shp = _shape(q, cache)
    if indices.dtype != torch.int32 or indices.dim() != 4 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 tensor [B, T, Hq, k_max]")
    k_max = int(indices.shape[3])
    out, lse = _outputs(shp, q.device, out, lse)
    desc = cache.desc()
    need = int(LIB.sparse_decode_attn_workspace_size(ctypes.byref(shp), k_max, int(num_splits)))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.sparse_decode_attn(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc),
                                indices.data_ptr(), k_max, _scale(shp.head_dim, sm_scale),
                                int(num_splits), out.data_ptr(), lse.data_ptr(), wptr, wbytes,
                                _stream(q))
    _check("sparse_decode_attn", st)
    return out, lse


def sparse_decode_attn_noalloc(
    q: torch.Tensor,
    cache: KVCache,
    indices: torch.Tensor,
    *,
    sm_scale: Optional[float] = None,
    num_splits: int = 0,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """sparse_decode_attn without a workspace: the split partials go to the library's fixed
    per-GPU scratch buffer.  Pass `out` and `lse` to allocate nothing at all."""
    shp = _shape(q, cache)
    if indices.dtype != torch.int32 or indices.dim() != 4 or not indices.is_contiguous():
        raise ValueError("indices must be a contiguous int32 tensor [B, T, Hq, k_max]")
    k_max = int(indices.shape[3])
    out, lse = _outputs(shp, q.device, out, lse)
    desc = cache.desc()
    st = LIB.sparse_decode_attn_noalloc(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc),
                                        indices.data_ptr(), k_max, _scale(shp.head_dim, sm_scale),
                                        int(num_splits), out.data_ptr(), lse.data_ptr(), _stream(q))
    _check("sparse_decode_attn_noalloc", st)
    return out, lse


def dense_decode_attn_workspace_size(q: torch.Tensor, cache: KVCache, num_splits: int = 0) -> int:
    shp = _shape(q, cache)
    desc = cache.desc()
    return int(LIB.dense_decode_attn_workspace_size(ctypes.byref(shp), ctypes.byref(desc),
                                                    int(num_splits)))


def dense_decode_attn(
    q: torch.Tensor,
    cache: KVCache,
    *,
    sm_scale: Optional[float] = None,
    num_splits: int = 0,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
) -> Tuple[torch.Tensor, torch.Tensor]:
    """Dense decode attention over every visible position: (out, lse) as sparse_decode_attn."""
    shp = _shape(q, cache)
    out, lse = _outputs(shp, q.device, out, lse)
    desc = cache.desc()
    need = int(LIB.dense_decode_attn_workspace_size(ctypes.byref(shp), ctypes.byref(desc),
                                                    int(num_splits)))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.dense_decode_attn(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc),
                               _scale(shp.head_dim, sm_scale), int(num_splits), out.data_ptr(),
                               lse.data_ptr(), wptr, wbytes, _stream(q))
    _check("dense_decode_attn", st)
    return out, lse


def sparse_decode_step_workspace_size(q: torch.Tensor, cache: KVCache, k_max: int) -> int:
    shp = _shape(q, cache)
    desc = cache.desc()
    return int(LIB.sparse_decode_step_workspace_size(ctypes.byref(shp), ctypes.byref(desc), int(k_max)))


def sparse_decode_step(
    q: torch.Tensor,
    cache: KVCache,
    k: Union[int, torch.Tensor],
    *,
    k_max: Optional[int] = None,
    sm_scale: Optional[float] = None,
    indices: Optional[torch.Tensor] = None,
    return_indices: bool = False,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
):
    """The oracle-indexed decode step in one call (the results of topk_index and of
    sparse_decode_attn over its lists, the attention computed on the indexer's scores): returns
    (out, lse), or (out, lse, indices) with return_indices or an `indices` tensor given."""
    shp = _shape(q, cache)
    k, kptr, k_max = _k_arg(k, k_max, shp, q.device)
    if indices is None and return_indices:
        indices = torch.empty((shp.batch, shp.q_len, shp.num_q_heads, k_max), dtype=torch.int32,
                              device=q.device)
    out, lse = _outputs(shp, q.device, out, lse)
    desc = cache.desc()
    need = int(LIB.sparse_decode_step_workspace_size(ctypes.byref(shp), ctypes.byref(desc), k_max))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.sparse_decode_step(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc),
                                _scale(shp.head_dim, sm_scale), kptr, k_max,
                                indices.data_ptr() if indices is not None else 0, out.data_ptr(),
                                lse.data_ptr(), wptr, wbytes, _stream(q))
    _check("sparse_decode_step", st)
    if indices is not None:
        return out, lse, indices
    return out, lse


# ---------------------------------------------------------------------------- reduced-byte indexer
class KeySketch:
    """int8 sketch of a KVCache's keys: codes int8 with K's shape, scales float32 with K's shape
    without the last axis (tensors owned by the caller).  Fill it with key_sketch_build."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        if codes.dtype != torch.int8 or not codes.is_contiguous() or codes.dim() != 4:
            raise TypeError("codes must be a contiguous 4-d int8 tensor")
        if scales.dtype != torch.float32 or not scales.is_contiguous() or tuple(scales.shape) != tuple(codes.shape[:3]):
            raise TypeError("scales must be a contiguous float32 tensor of codes.shape[:3]")
        self.codes, self.scales = codes, scales

    @classmethod
    def empty_for(cls, cache: KVCache) -> "KeySketch":
        codes = torch.zeros(cache.k.shape, dtype=torch.int8, device=cache.k.device)
        scales = torch.zeros(cache.k.shape[:3], dtype=torch.float32, device=cache.k.device)
        return cls(codes, scales)

    def check(self, cache: KVCache) -> None:
        if tuple(self.codes.shape) != tuple(cache.k.shape):
            raise ValueError("the sketch's shape differs from the cache's K")

    def desc(self) -> KeySketchDesc:
        return KeySketchDesc(self.codes.data_ptr(), self.scales.data_ptr())


def key_sketch_build(cache: KVCache, sketch: Optional[KeySketch] = None, *, last_n: int = 0) -> KeySketch:
    """Sketch key positions [max(0, L_b - last_n), L_b) of every request and KV head (last_n = 0:
    all of [0, L_b)) into `sketch` (allocated when None); returns the sketch."""
    if sketch is None:
        sketch = KeySketch.empty_for(cache)
    sketch.check(cache)
    B = int(cache.seq_lens.numel())
    shp = DecodeShape(B, 1, cache.num_kv_heads, cache.num_kv_heads, cache.head_dim)
    desc = cache.desc()
    sd = sketch.desc()
    st = LIB.key_sketch_build(ctypes.byref(shp), ctypes.byref(desc), int(last_n), ctypes.byref(sd),
                              _stream(cache.k))
    _check("key_sketch_build", st)
    return sketch


def topk_index_sketch_workspace_size(q: torch.Tensor, cache: KVCache, k_max: int, cand_mult: int = 2) -> int:
    shp = _shape(q, cache)
    desc = cache.desc()
    return int(LIB.topk_index_sketch_workspace_size(ctypes.byref(shp), ctypes.byref(desc), int(k_max),
                                                    int(cand_mult)))


def topk_index_sketch(
    q: torch.Tensor,
    cache: KVCache,
    sketch: KeySketch,
    k: Union[int, torch.Tensor],
    *,
    k_max: Optional[int] = None,
    cand_mult: int = 2,
    sm_scale: Optional[float] = None,
    indices: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Reduced-byte indexer: cand_mult * k candidates per row ranked on the int8 key sketch, the
    k best of them on exact scores; int32 [B, T, Hq, k_max] as topk_index."""
    shp = _shape(q, cache)
    sketch.check(cache)
    k, kptr, k_max = _k_arg(k, k_max, shp, q.device)
    if indices is None:
        indices = torch.empty((shp.batch, shp.q_len, shp.num_q_heads, k_max), dtype=torch.int32,
                              device=q.device)
    desc = cache.desc()
    sd = sketch.desc()
    need = int(LIB.topk_index_sketch_workspace_size(ctypes.byref(shp), ctypes.byref(desc), k_max,
                                                    int(cand_mult)))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.topk_index_sketch(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc), ctypes.byref(sd),
                               _scale(shp.head_dim, sm_scale), kptr, k_max, int(cand_mult),
                               indices.data_ptr(), wptr, wbytes, _stream(q))
    _check("topk_index_sketch", st)
    return indices


def sparse_decode_step_sketch_workspace_size(q: torch.Tensor, cache: KVCache, k_max: int,
                                             cand_mult: int = 2) -> int:
    shp = _shape(q, cache)
    desc = cache.desc()
    return int(LIB.sparse_decode_step_sketch_workspace_size(ctypes.byref(shp), ctypes.byref(desc),
                                                            int(k_max), int(cand_mult)))


def sparse_decode_step_sketch(
    q: torch.Tensor,
    cache: KVCache,
    sketch: KeySketch,
    k: Union[int, torch.Tensor],
    *,
    k_max: Optional[int] = None,
    cand_mult: int = 2,
    sm_scale: Optional[float] = None,
    indices: Optional[torch.Tensor] = None,
    return_indices: bool = False,
    out: Optional[torch.Tensor] = None,
    lse: Optional[torch.Tensor] = None,
    workspace: Optional[torch.Tensor] = None,
):
    """The decode step with the reduced-byte indexer: (out, lse), or (out, lse, indices)."""
    shp = _shape(q, cache)
    sketch.check(cache)
    k, kptr, k_max = _k_arg(k, k_max, shp, q.device)
    if indices is None and return_indices:
        indices = torch.empty((shp.batch, shp.q_len, shp.num_q_heads, k_max), dtype=torch.int32,
                              device=q.device)
    out, lse = _outputs(shp, q.device, out, lse)
    desc = cache.desc()
    sd = sketch.desc()
    need = int(LIB.sparse_decode_step_sketch_workspace_size(ctypes.byref(shp), ctypes.byref(desc), k_max,
                                                            int(cand_mult)))
    wptr, wbytes = _workspace(need, q.device, workspace)
    st = LIB.sparse_decode_step_sketch(ctypes.byref(shp), q.data_ptr(), ctypes.byref(desc), ctypes.byref(sd),
                                       _scale(shp.head_dim, sm_scale), kptr, k_max, int(cand_mult),
                                       indices.data_ptr() if indices is not None else 0, out.data_ptr(),
                                       lse.data_ptr(), wptr, wbytes, _stream(q))
    _check("sparse_decode_step_sketch", st)
    if indices is not None:
        return out, lse, indices
    return out, lse
