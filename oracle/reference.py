"""CPU oracle for oracle-top-k context-sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the benchmark's CPU
baseline leg may import this module.  The HIP library never calls it, and it shares no code,
constants or helpers with the library: it is plain NumPy written from the pages' definitions, in
float64 unless a step below states otherwise.

Sources (the pages are summaries of one paper, "Inference Time Context Sparsity: Illusion or
Opportunity?", plus the FlashSFA summary "Scaling Attention via Feature Sparsity"):

* Oracle top-k: exact selection of the k tokens with the highest scores, chosen separately for
  every decode token, query and head (technical summary, section 2 "Methodology", sparsity
  mechanisms: Oracle Top-K and the hardware implementation bullet).
* Sparse decode attention: softmax attention restricted to the selected tokens; the traffic per
  decode step drops from O(N d) to O(k d) (technical summary, section 3.C "Systems and hardware
  efficiency", bandwidth-efficiency bullet).
* Sparsity level: 50x sparsity keeps about 2% of the tokens (section 3.A, hybrid-models bullet).
* Dense decode: every decode step reads the whole cache (section 1 "Problem statement": the
  linear memory-bandwidth cost of decoding in dense attention).
* Split evaluation with a log-sum-exp merge: tiling with online softmax (FlashSFA summary,
  "Systeemimplementatie: FlashSFA", tiling and online-softmax bullet).

Readings where the pages are silent (each is listed with its reason in the design notes):
  score          s_n = (q . K_n) / sqrt(d), natural-log units; ranking by the signed score.
  ties           equal scores: the lower position is selected first.
  precision      scores and attention in float64; the top-k decision is taken on the scores
                 rounded to float32, the precision the GPU kernel ranks in.
  causality      with T new tokens per request of cached length L (T included), token t sees
                 positions 0 .. L - T + t.
  k              a row keeps min(k_b, visible) positions.
  GQA            query head hq reads KV head floor(hq / (Hq / Hkv)).
  index lists    order is irrelevant, -1 is padding, a repeated entry counts once per repeat.
  empty list     output 0, log-sum-exp -inf.
  paged cache    logical position n of request b lives in page page_table[b, n // page_size],
                 slot n % page_size.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "Cache",
    "visible_length",
    "scaled_scores",
    "topk_positions",
    "attention_weights",
    "attend",
    "lse_merge",
    "row_topk",
    "row_sparse",
    "row_dense",
    "decode_topk",
    "decode_sparse",
    "decode_dense",
]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers given as their raw 16-bit patterns: a bf16 is the upper half of
    an IEEE binary32, so the float32 with those bits in its top half is the same number."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def visible_length(seq_len: int, q_len: int, t: int) -> int:
    """Number of positions token t may attend to: positions 0 .. L - T + t (causal decode of T new
    tokens appended at the end of a cache of length L)."""
    return int(seq_len) - int(q_len) + int(t) + 1


class Cache:
    """Logical view of a bf16 KV cache held as raw bit patterns.

    contiguous: k_bits, v_bits uint16 [B, Hkv, max_len, d]
    paged:      k_bits, v_bits uint16 [num_pages, Hkv, page_size, d], page_table int [B, max_pages]
    """

    def __init__(self, k_bits, v_bits, seq_lens, layout="contiguous", page_table=None, page_size=0):
        self.k_bits = np.asarray(k_bits)
        self.v_bits = np.asarray(v_bits)
        self.seq_lens = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
        self.layout = layout
        self.page_table = None if page_table is None else np.asarray(page_table)
        self.page_size = int(page_size)
        if layout not in ("contiguous", "paged"):
            raise ValueError(layout)

    def _rows(self, bits, b: int, h: int) -> np.ndarray:
        L = self.seq_lens[b]
        if self.layout == "contiguous":
            return bf16_bits_to_f64(bits[b, h, :L])
        n = np.arange(L)
        pages = self.page_table[b, n // self.page_size]
        return bf16_bits_to_f64(bits[pages, h, n % self.page_size])

    def keys(self, b: int, h: int) -> np.ndarray:
        """K[b, h, 0:L_b, :] as float64 [L_b, d]."""
        return self._rows(self.k_bits, b, h)

    def values(self, b: int, h: int) -> np.ndarray:
        """V[b, h, 0:L_b, :] as float64 [L_b, d]."""
        return self._rows(self.v_bits, b, h)


def scaled_scores(q_row: np.ndarray, keys: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """s_n = (q . K_n) * scale for every row n of `keys`, in float64; scale defaults to
    1/sqrt(d).  This is the q.K^T scoring the oracle indexer ranks by."""
    q_row = np.asarray(q_row, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q_row.shape[-1])
    return (keys @ q_row) * scale


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k selection: the positions of the k largest scores, ranked on the scores rounded
    to float32, larger first and lower position first among equal values.  Returns min(k, n)
    positions in ascending order."""
    s32 = np.asarray(scores, dtype=np.float64).astype(np.float32)
    k = max(0, min(int(k), s32.shape[0]))
    order = np.argsort(-s32, kind="stable")
    return np.sort(order[:k])


def attention_weights(scores: np.ndarray) -> np.ndarray:
    """Softmax weights e^{s_i - m} / sum_j e^{s_j - m} over a list of scores (m = max)."""
    s = np.asarray(scores, dtype=np.float64)
    if s.size == 0:
        return s.copy()
    w = np.exp(s - s.max())
    return w / w.sum()


def attend(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """Softmax-weighted sum of `values` rows under `scores`, and the log-sum-exp of the scores.

    o = sum_i w_i v_i with w = softmax(s); lse = m + ln sum_i e^{s_i - m}.  An empty list gives
    o = 0 and lse = -inf."""
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    if s.size == 0:
        return np.zeros(v.shape[-1], dtype=np.float64), -math.inf
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ v) / l, float(m + math.log(l))


def lse_merge(parts: Sequence[Tuple[np.ndarray, float]]) -> Tuple[np.ndarray, float]:
    """Merge attention results computed over disjoint pieces of one index list.

    Piece j contributes (o_j, lse_j); with M = max lse_j the merged result is
    o = sum_j e^{lse_j - M} o_j / sum_j e^{lse_j - M} and lse = M + ln sum_j e^{lse_j - M}.
    Empty pieces (lse = -inf) contribute nothing."""
    parts = [(np.asarray(o, dtype=np.float64), float(l)) for o, l in parts]
    live = [(o, l) for o, l in parts if l != -math.inf]
    if not live:
        return np.zeros_like(parts[0][0]), -math.inf
    M = max(l for _, l in live)
    w = np.array([math.exp(l - M) for _, l in live])
    o = sum(wi * oi for wi, (oi, _) in zip(w, live)) / w.sum()
    return o, M + math.log(w.sum())


def row_topk(q_row, keys, visible: int, k: int, scale=None) -> np.ndarray:
    """Oracle top-k for one (request, token, query head) row over its visible positions."""
    visible = max(0, min(int(visible), keys.shape[0]))
    return topk_positions(scaled_scores(q_row, keys[:visible], scale), k)


def row_sparse(q_row, keys, values, positions, visible: int, scale=None) -> Tuple[np.ndarray, float]:
    """Sparse decode attention for one row over an index list (-1 entries skipped, repeats
    counted).  Every other entry must lie in [0, visible)."""
    pos = np.asarray(positions, dtype=np.int64).reshape(-1)
    pos = pos[pos != -1]
    if pos.size and (pos.min() < 0 or pos.max() >= visible):
        raise ValueError("index outside the visible range")
    s = scaled_scores(q_row, keys[pos], scale)
    return attend(s, values[pos])


def row_dense(q_row, keys, values, visible: int, scale=None) -> Tuple[np.ndarray, float]:
    """Dense decode attention for one row: every visible position."""
    visible = max(0, min(int(visible), keys.shape[0]))
    s = scaled_scores(q_row, keys[:visible], scale)
    return attend(s, values[:visible])


def _rows(B: int, T: int, Hq: int, rows: Optional[Iterable[Tuple[int, int, int]]]):
    if rows is None:
        return [(b, t, h) for b in range(B) for t in range(T) for h in range(Hq)]
    return [tuple(int(x) for x in r) for r in rows]


def decode_topk(q_bits, cache: Cache, k_per_req, k_max: int, scale=None, rows=None) -> np.ndarray:
    """Oracle indexer for a decode step: int32 [B, T, Hq, k_max], each row's selected positions in
    ascending order followed by -1 padding.  `rows` restricts the work to listed (b, t, hq) rows;
    other rows stay -1."""
    q = bf16_bits_to_f64(q_bits)
    B, T, Hq, _ = q.shape
    Hkv = cache.k_bits.shape[1]
    G = Hq // Hkv
    k_req = [int(x) for x in np.asarray(k_per_req).reshape(-1)]
    out = np.full((B, T, Hq, k_max), -1, dtype=np.int32)
    keys_cache = {}
    for b, t, hq in _rows(B, T, Hq, rows):
        h = hq // G
        if (b, h) not in keys_cache:
            keys_cache = {(b, h): cache.keys(b, h)}
        vis = visible_length(cache.seq_lens[b], T, t)
        sel = row_topk(q[b, t, hq], keys_cache[(b, h)], vis, min(k_req[b], k_max), scale)
        out[b, t, hq, : sel.size] = sel
    return out


def decode_sparse(q_bits, cache: Cache, indices, scale=None, rows=None):
    """Sparse decode attention for a decode step given index lists [B, T, Hq, k]: returns
    (o float64 [B, T, Hq, d], lse float64 [B, T, Hq]).  Unlisted rows stay NaN."""
    q = bf16_bits_to_f64(q_bits)
    B, T, Hq, d = q.shape
    Hkv = cache.k_bits.shape[1]
    G = Hq // Hkv
    idx = np.asarray(indices)
    o = np.full((B, T, Hq, d), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    kv = {}
    for b, t, hq in _rows(B, T, Hq, rows):
        h = hq // G
        if (b, h) not in kv:
            kv = {(b, h): (cache.keys(b, h), cache.values(b, h))}
        K, V = kv[(b, h)]
        vis = visible_length(cache.seq_lens[b], T, t)
        o[b, t, hq], lse[b, t, hq] = row_sparse(q[b, t, hq], K, V, idx[b, t, hq], vis, scale)
    return o, lse


def decode_dense(q_bits, cache: Cache, scale=None, rows=None):
    """Dense decode attention for a decode step: (o [B, T, Hq, d], lse [B, T, Hq]) in float64.
    Unlisted rows stay NaN."""
    q = bf16_bits_to_f64(q_bits)
    B, T, Hq, d = q.shape
    Hkv = cache.k_bits.shape[1]
    G = Hq // Hkv
    o = np.full((B, T, Hq, d), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    kv = {}
    for b, t, hq in _rows(B, T, Hq, rows):
        h = hq // G
        if (b, h) not in kv:
            kv = {(b, h): (cache.keys(b, h), cache.values(b, h))}
        K, V = kv[(b, h)]
        vis = visible_length(cache.seq_lens[b], T, t)
        o[b, t, hq], lse[b, t, hq] = row_dense(q[b, t, hq], K, V, vis, scale)
    return o, lse


def kth_score(q_row, keys, visible: int, k: int, scale=None) -> float:
    """The k-th largest float64 score among the visible positions (k >= 1): the reference value
    of the band rule for comparing selected sets."""
    visible = max(0, min(int(visible), keys.shape[0]))
    s = scaled_scores(q_row, keys[:visible], scale)
    k = min(int(k), s.shape[0])
    return float(np.sort(s)[::-1][k - 1])


__all__.append("kth_score")
