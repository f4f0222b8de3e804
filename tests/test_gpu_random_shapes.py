"""Seeded random decode shapes through every entry point, each row against the CPU oracle.

Shapes cover 1-3 requests with ragged lengths (some shorter than the tile sizes), 1-4 query
tokens, GQA ratios 1-8, head_dim 64 and 128, contiguous and paged caches (page sizes 16-256),
per-request k from 0 to more than the visible length, and candidate multipliers 1-3, so both
indexer paths (candidates and full scores), the fallbacks and the sketch's list modes are hit at
sizes the oracle checks row by row."""

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits, oracle_cache
from tests.gpu_util import all_rows, cache_of, check_attn_row, check_sketch_row, check_topk_row
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    max_len = int(rng.choice([257, 1000, 3000, 6144]))
    lens = [int(rng.integers(T, max_len + 1)) for _ in range(B)]
    layout = str(rng.choice(["contiguous", "paged"]))
    page = int(rng.choice([16, 64, 256]))
    if layout == "paged":
        max_len = -(-max_len // page) * page
    frac = float(rng.choice([0.005, 0.02, 0.1, 0.5]))
    ks = [int(rng.choice([0, max(1, int(frac * L)), L + 5])) if rng.random() < 0.3 else max(1, int(frac * L))
          for L in lens]
    m = int(rng.integers(1, 4))
    wl = make_workload(batch=B, q_len=T, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d, seq_lens=lens,
                       k=ks, layout=layout, page_size=page, max_len=max_len, needles_per_head=1, seed=seed)
    return wl, m


@pytest.mark.parametrize("seed", range(64))
def test_random_shape_every_entry_point(seed):
    import long_context_sparse_oracle_amd as lib

    wl_cpu, m = _case(9000 + seed)
    wl = wl_cpu.to("cuda")
    cache = cache_of(wl)
    k_max = wl.k_max
    idx = lib.topk_index(wl.q, cache, wl.k_per_req, k_max=k_max)
    o_s, l_s = lib.sparse_decode_attn(wl.q, cache, idx)
    o_d, l_d = lib.dense_decode_attn(wl.q, cache)
    o_st, l_st, idx_st = lib.sparse_decode_step(wl.q, cache, wl.k_per_req, k_max=k_max, return_indices=True)
    sk = lib.key_sketch_build(cache)
    o_sk, l_sk, idx_sk = lib.sparse_decode_step_sketch(wl.q, cache, sk, wl.k_per_req, k_max=k_max, cand_mult=m,
                                                       return_indices=True)
    idx_sk2 = lib.topk_index_sketch(wl.q, cache, sk, wl.k_per_req, k_max=k_max, cand_mult=m)
    torch.cuda.synchronize()
    idx, idx_st, idx_sk, idx_sk2 = (t.cpu().numpy() for t in (idx, idx_st, idx_sk, idx_sk2))
    o_s, l_s, o_d, l_d, o_st, l_st, o_sk, l_sk = (t.cpu().numpy() for t in (o_s, l_s, o_d, l_d, o_st, l_st, o_sk, l_sk))
    # the index-only sketch call and the fused one select the same lists
    np.testing.assert_array_equal(idx_sk, idx_sk2)
    q = oracle.bf16_bits_to_f64(bits(wl_cpu.q))
    oc = oracle_cache(wl_cpu)
    kreq = wl_cpu.k_per_req.numpy()
    for b, t, hq in all_rows(wl_cpu):
        K = oc.keys(b, hq // wl.group)
        V = oc.values(b, hq // wl.group)
        vis = oracle.visible_length(oc.seq_lens[b], wl.q_len, t)
        kk = min(int(kreq[b]), k_max)
        where = f"seed {seed} row {(b, t, hq)}"
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, kk, "topk " + where)
        check_topk_row(idx_st[b, t, hq], q[b, t, hq], K, vis, kk, "step topk " + where)
        check_sketch_row(idx_sk[b, t, hq], q[b, t, hq], K, vis, kk, m, "sketch " + where)
        for out, lse, lst, name in ((o_s, l_s, idx, "sparse"), (o_st, l_st, idx_st, "step"),
                                    (o_sk, l_sk, idx_sk, "sketch step")):
            want = oracle.row_sparse(q[b, t, hq], K, V, lst[b, t, hq], vis)
            check_attn_row(out[b, t, hq], lse[b, t, hq], want[0], want[1], f"{name} {where}")
        want = oracle.row_dense(q[b, t, hq], K, V, vis)
        check_attn_row(o_d[b, t, hq], l_d[b, t, hq], want[0], want[1], "dense " + where)
