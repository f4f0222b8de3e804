"""Oracle top-k context-sparse decode attention on AMD Instinct MI355X (gfx950).

The computation lives in libctxsparse.so (hand-written HIP kernels behind the C ABI of
include/ctxsparse.h); this package is a thin ctypes binding with the same entry-point names:

    topk_index(q, cache, k)                 -> int32 [B, T, Hq, k] selected positions
    sparse_decode_attn(q, cache, indices)   -> (out fp32 [B, T, Hq, d], lse fp32 [B, T, Hq])
    dense_decode_attn(q, cache)             -> (out, lse) over every visible position
    sparse_decode_step(q, cache, k)         -> (out, lse): the indexer and the sparse attention
                                               in one call, the attention on the indexer's own
                                               scores (V rows gathered only)
    key_sketch_build(cache)                 -> KeySketch: int8 codes + float32 scale per key row
    topk_index_sketch(q, cache, sketch, k)  -> the reduced-byte indexer: cand_mult * k candidates
                                               ranked on the sketch, re-ranked on exact scores
    sparse_decode_step_sketch(q, cache, sketch, k) -> (out, lse) with that indexer, fused
    KVCache(k, v, seq_lens, page_table=...) -> contiguous or paged bf16 cache description

Build the library with `python -m long_context_sparse_oracle_amd.build`.  Accessing any of the
names above without the built library raises ImportError: there is no CPU fallback.
"""

_BINDING_NAMES = (
    "KVCache",
    "CtxSparseError",
    "topk_index",
    "topk_index_workspace_size",
    "sparse_decode_attn",
    "sparse_decode_attn_workspace_size",
    "sparse_decode_attn_noalloc",
    "dense_decode_attn",
    "dense_decode_attn_workspace_size",
    "sparse_decode_step",
    "sparse_decode_step_workspace_size",
    "KeySketch",
    "key_sketch_build",
    "topk_index_sketch",
    "topk_index_sketch_workspace_size",
    "sparse_decode_step_sketch",
    "sparse_decode_step_sketch_workspace_size",
    "LIB",
    "LIB_PATH",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _lib

        return getattr(_lib, name)
    raise AttributeError(name)
