"""GPU parity of the indexer's paths against the CPU oracle.

For k <= max_len / 8 the indexer first estimates a per-row score threshold from a strided sample
of at most 1024 positions per (request, KV head), keeps only the positions scoring at or above it
as candidates and selects among those; when fewer than k candidates survive (or a candidate slot
overflows) the row is recomputed in full.  Larger k use the full-score path directly, and caches
of at most 1024 positions are scored whole and selected in one kernel.  These tests drive each
branch, the boundaries between the paths and per-request k including 0 and k >= visible.
"""

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits, oracle_cache
from tests.gpu_util import all_rows, cache_of, check_attn_row, check_topk_row, threshold_regimes_workload
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


def _check_indexer(wl_cpu, k_max=None):
    m = _lib()
    wl = wl_cpu.to("cuda")
    kmax = wl.k_max if k_max is None else k_max
    idx = m.topk_index(wl.q, cache_of(wl), wl.k_per_req, k_max=kmax)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    q = oracle.bf16_bits_to_f64(bits(wl_cpu.q))
    ocache = oracle_cache(wl_cpu)
    kreq = wl_cpu.k_per_req.numpy()
    for b, t, hq in all_rows(wl_cpu):
        K = ocache.keys(b, hq // wl.group)
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, min(int(kreq[b]), kmax), f"row {(b, t, hq)}")
    return idx


def test_threshold_from_unrepresentative_sample_falls_back():
    """The sampled positions (every 32nd of 32768) hold 100 planted keys that score about 3, far
    above everything else, so the sampled threshold leaves fewer than k = 655 candidates: the
    rows must be recomputed in full and still give the exact top-k."""
    L, k = 32768, 655
    wl = make_workload(batch=1, q_len=1, num_q_heads=2, num_kv_heads=2, head_dim=128,
                       seq_lens=[L], k=k, seed=41)
    for h in range(2):
        qh = wl.q[0, 0, h].float()
        key = (3.0 * qh / qh.norm()).to(torch.bfloat16)
        wl.k_cache[0, h, torch.arange(100) * (L // 1024)] = key
    idx = _check_indexer(wl)
    for h in range(2):
        planted = set((np.arange(100) * (L // 1024)).tolist())
        assert planted <= set(idx[0, 0, h].tolist())


def test_threshold_path_many_rows_gqa():
    """Filtered path with GQA 8, several chunks per row and a ragged tail."""
    wl = make_workload(batch=2, q_len=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       seq_lens=[40000, 23457], k=0.02, max_len=40003, needles_per_head=4, seed=42)
    _check_indexer(wl)


def test_threshold_rule_regimes():
    """The candidate threshold's rank across its regimes, on the index-only indexer."""
    _check_indexer(threshold_regimes_workload())


@pytest.mark.parametrize("k,label", [(512, "filtered at k = N/8"), (513, "full-score path")])
def test_path_boundary(k, label):
    wl = make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       seq_lens=[4096, 3000], k=k, max_len=4096, seed=43)
    _check_indexer(wl)


def test_per_request_k_zero_small_and_all():
    # k_max 256 of max_len 4096 (filtered); request 0 asks for none, request 3 for more than it has
    wl = make_workload(batch=4, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                       seq_lens=[4096, 1000, 3000, 200], k=[0, 5, 256, 256], max_len=4096, seed=44)
    idx = _check_indexer(wl, k_max=256)
    assert (idx[0] == -1).all()
    assert idx[3, 0, :, :200].tolist() == [list(range(200))] * 4


def test_paged_filtered_causal():
    wl = make_workload(batch=3, q_len=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[20000, 5000, 900], k=0.02, layout="paged", page_size=16,
                       max_len=20480, needles_per_head=2, seed=45)
    _check_indexer(wl)


def test_filtered_long_lists_large_capacity_select():
    # k = 8000 of 65536 on 8 rows: about 12100 candidates per row expected (some rows past 12288),
    # so the selection runs in the workgroup variant that holds up to 24576 of them in LDS
    wl = make_workload(batch=1, q_len=1, num_q_heads=8, num_kv_heads=1, head_dim=128,
                       seq_lens=[65536], k=8000, seed=46)
    _check_indexer(wl)


def test_k_equals_max_len():
    wl = make_workload(batch=2, q_len=2, num_q_heads=2, num_kv_heads=1, head_dim=128,
                       seq_lens=[512, 300], k=512, max_len=512, seed=47)
    idx = _check_indexer(wl)
    assert idx[0, 1, :, :512].tolist() == [list(range(512))] * 2


# ---- caches of at most 1024 positions: every position is scored and selected in one kernel

@pytest.mark.parametrize("max_len", [1024, 1025])
def test_small_cache_boundary(max_len):
    """1024 positions take the whole-row kernel, 1025 the regular paths: both exact, causal T = 4,
    GQA 8 over two KV heads (two row tiles per KV head), paged and contiguous requests."""
    for layout in ("contiguous", "paged"):
        wl = make_workload(batch=2, q_len=4, num_q_heads=16, num_kv_heads=2, head_dim=128,
                           seq_lens=[max_len, 700], k=[40, 700], layout=layout, page_size=64, max_len=max_len,
                           needles_per_head=2, seed=48)
        idx = _check_indexer(wl, k_max=700)
        # request 1 asks for more than it has: every visible position, ascending
        for t in range(4):
            assert idx[1, t, :, : 697 + t].tolist() == [list(range(697 + t))] * 16


def test_small_cache_exact_ties_and_edges():
    """All-equal keys (every score ties: the lowest positions win), a few strict winners mixed in,
    k = 1, and k = 0 for one request, on a 1000-position cache, head_dim 64."""
    m = _lib()
    n = 1000
    wl = make_workload(batch=2, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64, seq_lens=[n, 600],
                       k=[37, 0], max_len=n, seed=49)
    wl.k_cache[0] = wl.k_cache[0, 0, 0]
    wl.k_cache[0, 0, [5, n - 1, 321]] = (wl.q[0, 0, 3].float() * 4).to(torch.bfloat16)
    g = wl.to("cuda")
    idx = m.topk_index(g.q, cache_of(g), g.k_per_req, k_max=37).cpu().numpy()
    idx1 = m.topk_index(g.q, cache_of(g), 1).cpu().numpy()
    ocache = oracle_cache(wl)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    for hq in range(4):
        np.testing.assert_array_equal(idx[0, 0, hq], oracle.row_topk(q[0, 0, hq], ocache.keys(0, 0), n, 37))
        np.testing.assert_array_equal(idx1[0, 0, hq], oracle.row_topk(q[0, 0, hq], ocache.keys(0, 0), n, 1))
        assert (idx[1, 0, hq] == -1).all()


def test_small_cache_step_matches_oracle():
    """The one-call step on a short cache (whole-row selection, then attention on the kept
    scores): its lists by the band rule, its outputs against the oracle over those lists."""
    m = _lib()
    wl = make_workload(batch=3, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_lens=[900, 513, 64],
                       k=[50, 20, 64], layout="paged", page_size=16, max_len=912, needles_per_head=1, seed=50)
    g = wl.to("cuda")
    o, l, idx = m.sparse_decode_step(g.q, cache_of(g), g.k_per_req, k_max=64, return_indices=True)
    torch.cuda.synchronize()
    o, l, idx = o.cpu().numpy(), l.cpu().numpy(), idx.cpu().numpy()
    ocache = oracle_cache(wl)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    kreq = wl.k_per_req.numpy()
    for b, t, hq in all_rows(wl):
        K = ocache.keys(b, hq // wl.group)
        V = ocache.values(b, hq // wl.group)
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, min(int(kreq[b]), 64), f"row {(b, t, hq)}")
        want = oracle.row_sparse(q[b, t, hq], K, V, idx[b, t, hq], vis)
        check_attn_row(o[b, t, hq], l[b, t, hq], want[0], want[1], f"step row {(b, t, hq)}")


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_sample_pass_one_workgroup_per_tile(layout):
    """With at least half as many (request, KV head, 16-row tile) groups as compute units, one
    workgroup samples each tile and sets its thresholds; with fewer (the other tests here), four
    workgroups share a tile's samples and the candidate pass sets the thresholds.  160 groups,
    ragged lengths, q_len 2; the indexer and the one-call step's lists."""
    m = _lib()
    rng = np.random.default_rng(51)
    lens = rng.integers(1100, 2049, size=40).tolist()
    wl = make_workload(batch=40, q_len=2, num_q_heads=8, num_kv_heads=4, head_dim=64, seq_lens=lens,
                       k=0.05, layout=layout, page_size=16, max_len=2048, needles_per_head=1, seed=51)
    assert int(wl.k_per_req.max()) <= 2048 // 16  # the candidate path
    _check_indexer(wl)
    g = wl.to("cuda")
    o, l, idx = m.sparse_decode_step(g.q, cache_of(g), g.k_per_req, k_max=wl.k_max, return_indices=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    ocache = oracle_cache(wl)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    kreq = wl.k_per_req.numpy()
    for b, t, hq in all_rows(wl):
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx[b, t, hq], q[b, t, hq], ocache.keys(b, hq // wl.group), vis,
                       min(int(kreq[b]), wl.k_max), f"step row {(b, t, hq)}")


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_small_cache_one_workgroup_per_tile(layout):
    """Caches of at most 1024 positions with at least half as many tiles as compute units: one
    workgroup per tile scores the whole row and selects (with fewer tiles, four workgroups score a
    quarter each and a second kernel selects: the other small-cache tests).  160 groups, ragged
    lengths, q_len 2; the indexer and the one-call step's lists and outputs."""
    m = _lib()
    rng = np.random.default_rng(52)
    lens = rng.integers(300, 1001, size=40).tolist()
    wl = make_workload(batch=40, q_len=2, num_q_heads=8, num_kv_heads=4, head_dim=64, seq_lens=lens,
                       k=0.05, layout=layout, page_size=16, max_len=1008, needles_per_head=1, seed=52)
    _check_indexer(wl)
    g = wl.to("cuda")
    o, l, idx = m.sparse_decode_step(g.q, cache_of(g), g.k_per_req, k_max=wl.k_max, return_indices=True)
    torch.cuda.synchronize()
    o, l, idx = o.cpu().numpy(), l.cpu().numpy(), idx.cpu().numpy()
    ocache = oracle_cache(wl)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    kreq = wl.k_per_req.numpy()
    for b, t, hq in all_rows(wl):
        K = ocache.keys(b, hq // wl.group)
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, min(int(kreq[b]), wl.k_max), f"step row {(b, t, hq)}")
        if b % 8 == 0:
            want = oracle.row_sparse(q[b, t, hq], K, ocache.values(b, hq // wl.group), idx[b, t, hq], vis)
            check_attn_row(o[b, t, hq], l[b, t, hq], want[0], want[1], f"step row {(b, t, hq)}")


def test_fallback_paged_multitoken_ragged():
    """Planted high keys at the sampled positions of two requests of a ragged, paged, two-token
    batch push their rows' sampled thresholds above all but the planted keys, so those rows fall
    short of k candidates and are rescored in full through the page table; every row still gives
    the exact top-k, and the one-call step selects the same lists and attends to them."""
    m = _lib()
    lens = [9000, 40000, 2050, 17777]
    wl = make_workload(batch=4, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_lens=lens,
                       k=0.02, layout="paged", page_size=16, max_len=40000, seed=47)
    for b in (1, 3):  # requests whose rows fall back
        L = lens[b]
        stride = -(-L // 1024)  # the sample's stride for a request of length L
        n = torch.arange(0, L - 2, stride)  # every sampled position: ~250 per query head, far more
        for hq in range(8):                    # than the ~60 samples the threshold's rank asks for
            qh = wl.q[b, 1, hq].float()
            key = (3.0 * qh / qh.norm()).to(torch.bfloat16)
            sel = n[hq % 4::4]  # a quarter of the sampled positions per query head of the group
            wl.k_cache[wl.page_table[b, sel // 16].long(), hq // 4, sel % 16] = key
    idx = _check_indexer(wl)
    g = wl.to("cuda")
    o, l, idx_st = m.sparse_decode_step(g.q, cache_of(g), g.k_per_req, k_max=g.k_max, return_indices=True)
    torch.cuda.synchronize()
    idx_st = idx_st.cpu().numpy()
    np.testing.assert_array_equal(idx_st, idx)  # the same selection rule on the same scores
    o_ref, l_ref = oracle.decode_sparse(bits(wl.q), oracle_cache(wl), idx_st)
    o, l = o.cpu().numpy(), l.cpu().numpy()
    for r in all_rows(wl):
        check_attn_row(o[r], l[r], o_ref[r], l_ref[r], f"step row {r}")
