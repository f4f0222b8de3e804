"""GPU parity: the HIP library through its C ABI against the CPU oracle, element by element, on
seeded inputs that span several tiles, chunks and splits with ragged tails, plus the method's
edge cases (k = 1, k = visible, exact ties, empty rows, causal multi-token decode, paged caches,
GQA groups spanning two MFMA row tiles)."""

import math

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits, oracle_cache
from tests.gpu_util import all_rows, cache_of, check_attn_row, check_topk_row
from workloads import make_named, make_workload, random_index_sets

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


def _run_and_check(wl_cpu, k=None, splits=(0,), check_dense=True):
    """Upload a CPU workload, run the three entry points, compare every row with the oracle."""
    m = _lib()
    wl = wl_cpu.to("cuda")
    cache = cache_of(wl)
    qb = bits(wl_cpu.q)
    ocache = oracle_cache(wl_cpu)
    kreq = wl_cpu.k_per_req.numpy()
    idx_gpu = m.topk_index(wl.q, cache, wl.k_per_req, k_max=wl.k_max)
    torch.cuda.synchronize()
    idx_gpu = idx_gpu.cpu().numpy()
    q = oracle.bf16_bits_to_f64(qb)
    G = wl.group
    for b, t, hq in all_rows(wl_cpu):
        K = ocache.keys(b, hq // G)
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx_gpu[b, t, hq], q[b, t, hq], K, vis, int(kreq[b]), f"row {(b, t, hq)}")
    # sparse attention fed the oracle's own index lists
    idx_ref = oracle.decode_topk(qb, ocache, kreq, wl.k_max)
    o_ref, l_ref = oracle.decode_sparse(qb, ocache, idx_ref)
    idx_dev = torch.from_numpy(idx_ref).to("cuda")
    for S in splits:
        o, l = m.sparse_decode_attn(wl.q, cache, idx_dev, num_splits=S)
        torch.cuda.synchronize()
        o, l = o.cpu().numpy(), l.cpu().numpy()
        for b, t, hq in all_rows(wl_cpu):
            check_attn_row(o[b, t, hq], l[b, t, hq], o_ref[b, t, hq], l_ref[b, t, hq],
                           f"sparse S={S} row {(b, t, hq)}")
    if check_dense:
        od_ref, ld_ref = oracle.decode_dense(qb, ocache)
        for S in splits:
            o, l = m.dense_decode_attn(wl.q, cache, num_splits=S)
            torch.cuda.synchronize()
            o, l = o.cpu().numpy(), l.cpu().numpy()
            for b, t, hq in all_rows(wl_cpu):
                check_attn_row(o[b, t, hq], l[b, t, hq], od_ref[b, t, hq], ld_ref[b, t, hq],
                               f"dense S={S} row {(b, t, hq)}")
    return idx_gpu


def test_tiny_named_matches_golden():
    """The tiny seeded decode step (d=64, N=1024, k=32, needles) against the stored oracle output."""
    import json
    import os

    wl = make_named("tiny_d64_n1024", device="cpu")
    idx = _run_and_check(wl, splits=(0, 1, 3))
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_d64_n1024.json")) as f:
        rec = json.load(f)
    for b, t, hq, p in rec["needles"]:
        assert p in idx[b, t, hq].tolist()


def test_contiguous_d128_ragged_tail():
    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[5000, 3333], k=100, max_len=5003, needles_per_head=3, seed=21)
    _run_and_check(wl, splits=(0, 1, 2, 7))


def test_contiguous_d64_gqa4():
    wl = make_workload(batch=3, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       seq_lens=[2049, 17, 4096], k=64, seed=22)
    _run_and_check(wl, splits=(0, 5))


def test_multitoken_causal_ragged():
    # T=4: token t sees L - 4 + t + 1 positions; one request is exactly T long (visible 1..4)
    wl = make_workload(batch=4, q_len=4, num_q_heads=4, num_kv_heads=1, head_dim=128,
                       seq_lens=[3001, 4, 64, 1500], k=50, needles_per_head=1, seed=23)
    _run_and_check(wl, splits=(0, 3))


@pytest.mark.parametrize("page_size,d", [(16, 128), (64, 64), (16, 64)])
def test_paged(page_size, d):
    wl = make_workload(batch=3, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=d,
                       seq_lens=[2500, 777, 40], k=0.05, layout="paged", page_size=page_size,
                       max_len=2560, needles_per_head=2, seed=24 + page_size)
    _run_and_check(wl, splits=(0, 2))


def test_gqa_two_row_tiles():
    # G = 8, T = 4 -> 32 query rows per KV head: two 16-row MFMA tiles
    wl = make_workload(batch=1, q_len=4, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       seq_lens=[2000], k=40, seed=25)
    _run_and_check(wl, splits=(0,))


def test_lowrank_heavy_tailed():
    wl = make_workload(batch=1, q_len=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       seq_lens=[8192], k=164, structure="lowrank", seed=26)
    _run_and_check(wl, splits=(0, 4))


def test_k_edges():
    # k = 1 and k = visible (every position)
    wl = make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=128,
                       seq_lens=[300, 129], k=[1, 129], max_len=300, seed=27)
    idx = _run_and_check(wl, splits=(0,))
    # request 1 keeps everything visible: positions 0..vis-1 exactly
    for t in range(2):
        vis = 129 - 2 + t + 1
        for hq in range(4):
            assert idx[1, t, hq, :vis].tolist() == list(range(vis))


@pytest.mark.parametrize("n", [3000, 20000])
def test_exact_ties_lowest_positions_first(n):
    """All keys equal -> all scores tie -> the k lowest positions.  n=20000 puts more than the
    LDS candidate capacity into the threshold bin (the global refinement path)."""
    m = _lib()
    wl = make_workload(batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                       seq_lens=[n], k=777, seed=28)
    wl.k_cache[:] = wl.k_cache[0, 0, 0]
    # query head 3 gets a few larger keys so its set mixes strict winners and ties
    wl.k_cache[0, 0, [5, n - 1, 1234]] = (wl.q[0, 0, 3].float() * 4).to(torch.bfloat16)
    g = wl.to("cuda")
    idx = m.topk_index(g.q, cache_of(g), 777).cpu().numpy()
    ocache = oracle_cache(wl)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    for hq in range(4):
        want = oracle.row_topk(q[0, 0, hq], ocache.keys(0, 0), n, 777)
        np.testing.assert_array_equal(idx[0, 0, hq], want)


def test_sparse_padding_duplicates_invalid_and_empty():
    m = _lib()
    wl = make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=128,
                       seq_lens=[500, 200], k=64, max_len=500, seed=29)
    rs = np.random.default_rng(5)
    idx = rs.integers(0, 200, size=(2, 2, 4, 64)).astype(np.int32)  # duplicates likely
    idx[:, :, :, ::7] = -1
    idx[0, 0, 1, :] = -1  # empty row
    idx[1, 1, 2, 3] = 10_000  # beyond the cache: skipped
    idx[1, 0, 0, 9] = 199  # L=200, T=2: token 0 sees 0..198 -> 199 skipped for it
    idx[1, 0, 0, 10] = -5  # negative: skipped
    g = wl.to("cuda")
    o, l = m.sparse_decode_attn(g.q, cache_of(g), torch.from_numpy(idx).cuda(), num_splits=3)
    o, l = o.cpu().numpy(), l.cpu().numpy()
    # the oracle takes only valid entries: drop everything outside each row's visible range
    clean = idx.copy()
    for b, t, hq in all_rows(wl):
        vis = oracle.visible_length(int(wl.seq_lens[b]), wl.q_len, t)
        r = clean[b, t, hq]
        r[(r < 0) | (r >= vis)] = -1
    assert clean[1, 1, 2, 3] == -1 and clean[1, 0, 0, 9] == -1 and clean[1, 0, 0, 10] == -1
    o_ref, l_ref = oracle.decode_sparse(bits(wl.q), oracle_cache(wl), clean)
    for r in all_rows(wl):
        check_attn_row(o[r], l[r], o_ref[r], l_ref[r], f"row {r}")
    assert l[0, 0, 1] == -math.inf and not o[0, 0, 1].any()


def test_random_index_sets_match_oracle():
    m = _lib()
    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[4096, 2500], k=300, max_len=4096, seed=30)
    idx = random_index_sets(wl, seed=3)
    g = wl.to("cuda")
    for S in (0, 1, 4):
        o, l = m.sparse_decode_attn(g.q, cache_of(g), idx.cuda(), num_splits=S)
        o, l = o.cpu().numpy(), l.cpu().numpy()
        o_ref, l_ref = oracle.decode_sparse(bits(wl.q), oracle_cache(wl), idx.numpy())
        for r in all_rows(wl):
            check_attn_row(o[r], l[r], o_ref[r], l_ref[r], f"S={S} row {r}")


def test_sparse_with_all_positions_equals_dense():
    m = _lib()
    wl = make_workload(batch=1, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[1000], k=1000, seed=31)
    g = wl.to("cuda")
    c = cache_of(g)
    idx = torch.arange(1000, dtype=torch.int32, device="cuda").flip(0).expand(1, 1, 8, 1000).contiguous()
    o1, l1 = m.sparse_decode_attn(g.q, c, idx)
    o2, l2 = m.dense_decode_attn(g.q, c)
    assert (o1 - o2).abs().max().item() <= 2e-3
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_deterministic():
    m = _lib()
    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[6000, 6000], k=120, seed=32).to("cuda")
    c = cache_of(wl)
    i1 = m.topk_index(wl.q, c, 120)
    i2 = m.topk_index(wl.q, c, 120)
    assert torch.equal(i1, i2)
    a = m.sparse_decode_attn(wl.q, c, i1, num_splits=4)
    b = m.sparse_decode_attn(wl.q, c, i1, num_splits=4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    a = m.dense_decode_attn(wl.q, c)
    b = m.dense_decode_attn(wl.q, c)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_error_status_raises():
    m = _lib()
    wl = make_workload(batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                       seq_lens=[100], k=10, seed=33).to("cuda")
    with pytest.raises(m.CtxSparseError):
        m.topk_index(wl.q, cache_of(wl), 101)  # k_max above max_len


def test_paged_equals_contiguous_every_entry_point():
    """The same logical cache stored paged (permuted pages) and contiguously gives the same index
    lists (the scores are bit-identical) and the same outputs, on every entry point."""
    m = _lib()
    wl = make_workload(batch=3, q_len=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[5000, 1234, 3000], k=0.02, layout="paged", page_size=16, max_len=5008,
                       needles_per_head=2, seed=33).to("cuda")
    B, Hkv, d, L = wl.batch, wl.num_kv_heads, wl.head_dim, wl.max_len
    kc = torch.zeros((B, Hkv, L, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b in range(B):
        n = torch.arange(int(wl.seq_lens[b]), device="cuda")
        pages = wl.page_table[b, n // 16].long()
        kc[b, :, : n.numel()] = wl.k_cache[pages, :, n % 16].transpose(0, 1)
        vc[b, :, : n.numel()] = wl.v_cache[pages, :, n % 16].transpose(0, 1)
    paged = cache_of(wl)
    contig = m.KVCache(kc, vc, wl.seq_lens, max_len=L)
    res = {}
    for name, cache in (("paged", paged), ("contiguous", contig)):
        idx = m.topk_index(wl.q, cache, wl.k_per_req, k_max=wl.k_max)
        o, l = m.sparse_decode_attn(wl.q, cache, idx)
        od, ld = m.dense_decode_attn(wl.q, cache)
        os_, ls_, is_ = m.sparse_decode_step(wl.q, cache, wl.k_per_req, k_max=wl.k_max, return_indices=True)
        sk = m.key_sketch_build(cache)
        ok, lk, ik = m.sparse_decode_step_sketch(wl.q, cache, sk, wl.k_per_req, k_max=wl.k_max, cand_mult=2,
                                                 return_indices=True)
        torch.cuda.synchronize()
        res[name] = (idx, o, l, od, ld, os_, ls_, is_, ok, lk, ik)
    names = ("idx", "sparse o", "sparse lse", "dense o", "dense lse", "step o", "step lse", "step idx",
             "sketch o", "sketch lse", "sketch idx")
    for n, a, c in zip(names, res["paged"], res["contiguous"]):
        if a.dtype == torch.int32:
            assert torch.equal(a, c), n
        else:
            fin = torch.isfinite(c)
            assert torch.equal(torch.isfinite(a), fin), n
            assert float((a[fin] - c[fin]).abs().max()) <= 1e-5, n
