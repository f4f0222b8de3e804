"""Helpers for GPU parity tests: run the HIP library on a workload and compare with the oracle.

Comparison rules (tolerances fixed for this method: 2e-3 absolute on outputs, 1e-3 on the
log-sum-exp, and a 1e-3 band around the k-th score for selected sets):
  indexer    every position in (GPU set) xor (oracle set) has an oracle score within 1e-3 of the
             oracle's k-th largest score; the GPU row holds exactly min(k_b, visible) distinct
             visible positions in ascending order, then -1.
  attention  max |out - out_oracle| <= 2e-3 and |lse - lse_oracle| <= 1e-3 per row.
  sketch     (reduced-byte indexer) every selected position lies in the oracle's candidate set,
             which the GPU reproduces exactly, and the selection differs from the oracle's only at
             positions within 1e-3 of the k-th largest exact score among the candidates.
"""

import math

import numpy as np
import torch

import oracle
from tests._util import bits

OUT_TOL = 2e-3
LSE_TOL = 1e-3
BAND = 1e-3


def cache_of(wl):
    from long_context_sparse_oracle_amd import KVCache

    return KVCache(wl.k_cache, wl.v_cache, wl.seq_lens, page_table=wl.page_table,
                   max_len=wl.max_len)


def logical_kv(wl, b, h):
    """float64 logical K, V [L_b, d] of (request b, KV head h), copied from wherever they live."""
    L = int(wl.seq_lens[b])
    if wl.layout == "contiguous":
        kb = bits(wl.k_cache[b, h, :L])
        vb = bits(wl.v_cache[b, h, :L])
    else:
        n = torch.arange(L, device=wl.page_table.device)
        pages = wl.page_table[b, n // wl.page_size].long()
        kb = bits(wl.k_cache[pages, h, n % wl.page_size])
        vb = bits(wl.v_cache[pages, h, n % wl.page_size])
    return oracle.bf16_bits_to_f64(kb), oracle.bf16_bits_to_f64(vb)


def check_topk_row(gpu_row, q_row, K, vis, k, where=""):
    """Band-rule comparison of one GPU index row against the oracle."""
    kk = min(k, vis)
    row = np.asarray(gpu_row)
    sel = row[:kk]
    assert (row[kk:] == -1).all(), f"{where}: padding"
    assert (sel >= 0).all() and (sel < vis).all(), f"{where}: out of range"
    assert (np.diff(sel) > 0).all(), f"{where}: not strictly ascending"
    if kk == 0:
        return 0
    want = oracle.row_topk(q_row, K, vis, kk)
    diff = np.setxor1d(sel, want)
    if diff.size:
        s = oracle.scaled_scores(q_row, K[:vis])
        sk = float(np.sort(s)[::-1][kk - 1])
        bad = diff[np.abs(s[diff] - sk) > BAND]
        assert bad.size == 0, f"{where}: {bad.size} positions outside the band, e.g. {bad[:5]}"
    return int(diff.size)


def check_sketch_row(gpu_row, q_row, K, vis, k, m, where=""):
    """Comparison of one GPU row of the reduced-byte indexer (cand_mult m) with its oracle."""
    kk = min(k, vis)
    row = np.asarray(gpu_row)
    sel = row[:kk]
    assert (row[kk:] == -1).all(), f"{where}: padding"
    assert (sel >= 0).all() and (sel < vis).all(), f"{where}: out of range"
    assert (np.diff(sel) > 0).all(), f"{where}: not strictly ascending"
    if kk == 0:
        return 0
    cand = oracle.sketch_candidates(q_row, K, vis, kk, m)
    outside = np.setdiff1d(sel, cand)
    assert outside.size == 0, f"{where}: {outside.size} positions outside the sketch candidates, e.g. {outside[:5]}"
    want = oracle.row_topk_sketch(q_row, K, vis, kk, m)
    diff = np.setxor1d(sel, want)
    if diff.size:
        s = oracle.scaled_scores(q_row, K[:vis])
        sk = float(np.sort(s[cand])[::-1][kk - 1])
        bad = diff[np.abs(s[diff] - sk) > BAND]
        assert bad.size == 0, f"{where}: {bad.size} positions outside the band, e.g. {bad[:5]}"
    return int(diff.size)


def check_attn_row(o, lse, want_o, want_lse, where=""):
    if want_lse == -math.inf:
        assert lse == -math.inf, f"{where}: lse {lse} for an empty row"
        assert np.abs(o).max() == 0.0, f"{where}: nonzero output for an empty row"
        return
    err = float(np.abs(np.asarray(o, np.float64) - want_o).max())
    assert err <= OUT_TOL, f"{where}: max |out err| {err}"
    assert abs(float(lse) - want_lse) <= LSE_TOL, f"{where}: lse {lse} vs {want_lse}"


def all_rows(wl):
    return [(b, t, h) for b in range(wl.batch) for t in range(wl.q_len) for h in range(wl.num_q_heads)]


def threshold_regimes_workload():
    # k_max = 4096 = max_len / 16 keeps every row on the filtered path.  Expected samples among a
    # row's top k, mu = k * samples / visible: about 0.06, 10 and 64 for the three full rows
    # (threshold ranks 11, 36 and 112 of 1024); about 400 for the 8000-position row, whose
    # threshold keeps about half its positions so that slots overflow and it is recomputed in
    # full; and past the sample count for the two short rows (every position a candidate).
    from workloads import make_workload

    return make_workload(batch=6, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         seq_lens=[65536, 65536, 65536, 8000, 3000, 1500],
                         k=[4, 655, 4096, 3200, 2900, 1499], max_len=65536, needles_per_head=2, seed=49)
