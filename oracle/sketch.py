"""CPU oracle for the reduced-byte indexer (int8 key sketch + exact re-rank).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite, the package smoke
check and the benchmark's CPU baseline leg may import it; the HIP library never calls it and
shares no code with it.

The pages count an indexer's cost against the sparse kernel's gain -- they simulate one with
Double Sparsity, a method that scores a reduced part of each key, and report break-even points
between 2x and 10x sparsity with 2.8x-4.17x gains at 100x (technical summary, section 3.C,
indexing-overhead bullet).  This module defines this project's own reduced-byte indexer so that
its break-even can be measured; it is not a method from the pages:

  sketch    every key row K_n (bf16, d values) is stored as int8 codes with one float32 scale:
                m_n = max_i |K_n,i|, scale_n = m_n / 127, c_n,i = rint(K_n,i / scale_n)
            in float32 arithmetic (the division correctly rounded, rint = round half to even),
            codes clamped to [-127, 127]; an all-zero row has scale 0 and codes 0.  The query
            row is quantised the same way (scale_q, c_q).
  approx    a_n = (scale_q * scale_n) * (c_q . c_n): the integer dot product is exact, the two
            float32 products are rounded in that order.  Every step is exact or a single
            float32 rounding, so the approximate ranking is reproducible bit for bit.
  select    the candidates are the min(m * k', visible) positions with the largest a_n (lower
            position first among equal values), m >= 1 the candidate multiplier; the result is
            the k' candidates with the largest exact scores, ranked as the oracle indexer ranks
            (scores rounded to float32, lower position first among equal values), in ascending
            order.  With m * k' >= visible it is the oracle top-k itself.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .reference import Cache, bf16_bits_to_f64, scaled_scores, visible_length

__all__ = ["int8_sketch", "sketch_scores", "sketch_candidates", "row_topk_sketch", "decode_topk_sketch"]


def int8_sketch(rows) -> Tuple[np.ndarray, np.ndarray]:
    """int8 codes [n, d] and float32 scales [n] of float rows [n, d] (values exact in float32)."""
    x = np.asarray(rows, dtype=np.float64).astype(np.float32)
    x = np.atleast_2d(x)
    m = np.abs(x).max(axis=1)
    scale = (m / np.float32(127.0)).astype(np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    live = scale > 0
    if live.any():
        q = np.rint(x[live] / scale[live][:, None]).astype(np.float32)
        codes[live] = np.clip(q, -127, 127).astype(np.int8)
    return codes, scale


def sketch_scores(q_row, codes, scales) -> np.ndarray:
    """Approximate scores a_n (float32) of one query row against sketched keys."""
    qc, qs = int8_sketch(np.asarray(q_row)[None, :])
    dot = np.asarray(codes, dtype=np.int64) @ qc[0].astype(np.int64)
    prod = (np.float32(qs[0]) * np.asarray(scales, dtype=np.float32)).astype(np.float32)
    return (prod * dot.astype(np.float32)).astype(np.float32)


def sketch_candidates(q_row, keys, visible: int, k: int, cand_mult: int) -> np.ndarray:
    """Ascending positions of the min(m * k', visible) visible keys with the largest sketch
    scores (lower position first among equal values), k' = min(k, visible)."""
    visible = max(0, min(int(visible), keys.shape[0]))
    kk = max(0, min(int(k), visible))
    nc = min(int(cand_mult) * kk, visible)
    if nc == 0:
        return np.zeros(0, dtype=np.int64)
    codes, scales = int8_sketch(keys[:visible])
    approx = sketch_scores(q_row, codes, scales)
    return np.sort(np.argsort(-approx, kind="stable")[:nc])


def row_topk_sketch(q_row, keys, visible: int, k: int, cand_mult: int, scale=None) -> np.ndarray:
    """Reduced-byte indexer for one row: ascending positions of the selection described above."""
    visible = max(0, min(int(visible), keys.shape[0]))
    kk = max(0, min(int(k), visible))
    cand = sketch_candidates(q_row, keys, visible, kk, cand_mult)
    if kk == 0:
        return cand
    s32 = scaled_scores(q_row, keys[cand], scale).astype(np.float32)
    keep = np.argsort(-s32, kind="stable")[:kk]
    return np.sort(cand[keep])


def decode_topk_sketch(q_bits, cache: Cache, k_per_req, k_max: int, cand_mult: int, scale=None,
                       rows=None) -> np.ndarray:
    """The reduced-byte indexer for a decode step: int32 [B, T, Hq, k_max], each row's selection
    (row_topk_sketch) in ascending order followed by -1 padding, for all rows or the listed
    (b, t, hq) `rows` (others stay -1)."""
    q = bf16_bits_to_f64(q_bits)
    B, T, Hq, _ = q.shape
    G = Hq // cache.k_bits.shape[1]
    k_req = [int(x) for x in np.asarray(k_per_req).reshape(-1)]
    out = np.full((B, T, Hq, k_max), -1, dtype=np.int32)
    todo = rows if rows is not None else [(b, t, h) for b in range(B) for t in range(T) for h in range(Hq)]
    for b, t, hq in todo:
        K = cache.keys(b, hq // G)
        vis = visible_length(cache.seq_lens[b], T, t)
        sel = row_topk_sketch(q[b, t, hq], K, vis, min(k_req[b], k_max), cand_mult, scale)
        out[b, t, hq, : sel.size] = sel
    return out
