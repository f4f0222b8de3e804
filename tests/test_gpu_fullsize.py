"""GPU parity at the named workloads' full sizes, in the launch configuration bench.py times
(automatic splits and chunking), including the sweep's 500x point and its 64-request batch, and
at the library's documented limits (262144 positions on both indexer paths, 64 query rows per KV
head, 4096-position pages, head_dim 64 at a long context).

* Sampled rows (first, last and seeded random ones) are compared with the CPU oracle one by one:
  indexer by the band rule, sparse attention fed the oracle's own index lists, dense attention;
  the one-call step and the reduced-byte indexer's step (cand_mult 2, as bench.py runs them):
  their lists by the band rules, their outputs against the oracle's attention over those lists.
* Every row is checked for properties that hold at any size: each index row holds min(k_b,
  visible) distinct visible positions in ascending order then -1; every planted needle is
  selected; and against float32 scores computed independently with torch on the GPU, every
  selected position scores >= the row's k-th score - 1e-3 and every unselected one <= it + 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits
from tests.gpu_util import check_attn_row, check_sketch_row, check_topk_row, logical_kv
from workloads import make_named, random_index_sets
from workloads.synth import SWEEP_K

pytestmark = pytest.mark.gpu

N_SAMPLES = 6


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


def _cache(wl):
    m = _lib()
    return m.KVCache(wl.k_cache, wl.v_cache, wl.seq_lens, page_table=wl.page_table, max_len=wl.max_len)


def _sample_rows(wl, seed):
    rng = np.random.default_rng(seed)
    rows = [(0, 0, 0), (wl.batch - 1, wl.q_len - 1, wl.num_q_heads - 1)]
    while len(rows) < N_SAMPLES:
        rows.append((int(rng.integers(wl.batch)), int(rng.integers(wl.q_len)), int(rng.integers(wl.num_q_heads))))
    return rows


def _torch_scores_group(wl, b, h):
    """float32 scores [T*G, L] of one (request, KV head) group, with torch (independent of the
    library): logical K gathered through the page table when paged."""
    L = int(wl.seq_lens[b])
    G = wl.group
    if wl.layout == "contiguous":
        K = wl.k_cache[b, h, :L].float()
    else:
        n = torch.arange(L, device=wl.q.device)
        K = wl.k_cache[wl.page_table[b, n // wl.page_size].long(), h, n % wl.page_size].float()
    Q = wl.q[b, :, h * G:(h + 1) * G].float().reshape(-1, wl.head_dim)  # [T*G, d]
    return (Q @ K.t().contiguous()) / float(np.sqrt(wl.head_dim)), L


def _check_all_rows(wl, idx, kreq):
    """Properties of the GPU indexer output on every row."""
    B, T, Hq, G = wl.batch, wl.q_len, wl.num_q_heads, wl.group
    k_max = idx.shape[-1]
    pos = torch.arange(k_max, device=idx.device)
    for b in range(B):
        L = int(wl.seq_lens[b])
        for h in range(wl.num_kv_heads):
            S, _ = _torch_scores_group(wl, b, h)
            for t in range(T):
                vis = L - T + t + 1
                kk = min(int(kreq[b]), vis)
                rows = idx[b, t, h * G:(h + 1) * G]  # [G, k_max]
                sel = rows[:, :kk].long()
                assert bool((rows[:, kk:] == -1).all()), f"padding b{b} t{t} h{h}"
                assert bool(((sel >= 0) & (sel < vis)).all()), f"range b{b} t{t} h{h}"
                if kk > 1:
                    assert bool((sel[:, 1:] > sel[:, :-1]).all()), f"ascending b{b} t{t} h{h}"
                if kk == 0:
                    continue
                s = S[t * G:(t + 1) * G, :vis]
                kth = torch.topk(s, kk, dim=1).values[:, -1:]
                ss = torch.gather(s, 1, sel)
                assert bool((ss >= kth - 1e-3).all()), f"selected below the band b{b} t{t} h{h}"
                mask = torch.ones_like(s, dtype=torch.bool)
                mask.scatter_(1, sel, False)
                unsel_max = torch.where(mask, s, torch.full_like(s, -float("inf"))).max(dim=1, keepdim=True).values
                assert bool((unsel_max <= kth + 1e-3).all()), f"unselected above the band b{b} t{t} h{h}"
            del S
    del pos
    for b, t, hq, p in wl.needles.tolist():
        assert p in idx[b, t, hq].tolist(), f"needle {(b, t, hq, p)} not selected"


def _check_structure(wl, idx, kreq):
    """Padding, range and order of every row of an index tensor."""
    B, T = wl.batch, wl.q_len
    for b in range(B):
        L = int(wl.seq_lens[b])
        for t in range(T):
            vis = L - T + t + 1
            kk = min(int(kreq[b]), vis)
            rows = idx[b, t]
            sel = rows[:, :kk].long()
            assert bool((rows[:, kk:] == -1).all()), f"padding b{b} t{t}"
            assert bool(((sel >= 0) & (sel < vis)).all()), f"range b{b} t{t}"
            if kk > 1:
                assert bool((sel[:, 1:] > sel[:, :-1]).all()), f"ascending b{b} t{t}"


def _check_steps(wl, cache, kt, k_max, kreq, rows, q):
    """The one-call step and the reduced-byte indexer's step at full size, on sampled rows."""
    m = _lib()
    o, l, idx = m.sparse_decode_step(wl.q, cache, kt, k_max=k_max, return_indices=True)
    sketch = m.key_sketch_build(cache)
    o2, l2, idx2 = m.sparse_decode_step_sketch(wl.q, cache, sketch, kt, k_max=k_max, cand_mult=2,
                                               return_indices=True)
    torch.cuda.synchronize()
    _check_structure(wl, idx, kreq)
    _check_structure(wl, idx2, kreq)
    o, l, idx = o.cpu().numpy(), l.cpu().numpy(), idx.cpu().numpy()
    o2, l2, idx2 = o2.cpu().numpy(), l2.cpu().numpy(), idx2.cpu().numpy()
    del sketch
    G = wl.group
    for b, t, hq in rows:
        K, V = logical_kv(wl, b, hq // G)
        vis = oracle.visible_length(int(wl.seq_lens[b]), wl.q_len, t)
        kk = int(kreq[b])
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, kk, f"step topk {(b, t, hq)}")
        want = oracle.row_sparse(q[b, t, hq], K, V, idx[b, t, hq], vis)
        check_attn_row(o[b, t, hq], l[b, t, hq], want[0], want[1], f"step {(b, t, hq)}")
        check_sketch_row(idx2[b, t, hq], q[b, t, hq], K, vis, kk, 2, f"sketch topk {(b, t, hq)}")
        want = oracle.row_sparse(q[b, t, hq], K, V, idx2[b, t, hq], vis)
        check_attn_row(o2[b, t, hq], l2[b, t, hq], want[0], want[1], f"sketch step {(b, t, hq)}")


def _run(wl, k=None, seed=0, check_dense=True):
    m = _lib()
    cache = _cache(wl)
    kreq = wl.k_per_req.cpu().numpy() if k is None else np.full(wl.batch, k)
    k_max = wl.k_max if k is None else int(k)
    kt = wl.k_per_req if k is None else torch.full((wl.batch,), k, dtype=torch.int32, device="cuda")
    idx = m.topk_index(wl.q, cache, kt, k_max=k_max)
    torch.cuda.synchronize()
    _check_all_rows(wl, idx, kreq)
    idx_cpu = idx.cpu().numpy()

    rows = _sample_rows(wl, seed)
    qb = bits(wl.q)
    q = oracle.bf16_bits_to_f64(qb)
    G = wl.group
    # sparse attention: uniform random sets everywhere, the oracle's own top-k on sampled rows
    sets = random_index_sets(wl, k=k_max if k is not None else None, seed=seed + 1)
    ref = {}
    for b, t, hq in rows:
        K, V = logical_kv(wl, b, hq // G)
        L = int(wl.seq_lens[b])
        vis = oracle.visible_length(L, wl.q_len, t)
        kk = int(kreq[b])
        check_topk_row(idx_cpu[b, t, hq], q[b, t, hq], K, vis, kk, f"topk {(b, t, hq)}")
        osel = oracle.row_topk(q[b, t, hq], K, vis, kk)
        sets[b, t, hq] = -1
        sets[b, t, hq, : osel.size] = torch.from_numpy(osel.astype(np.int32))
        ref[(b, t, hq)] = (oracle.row_sparse(q[b, t, hq], K, V, osel, vis),
                           oracle.row_dense(q[b, t, hq], K, V, vis) if check_dense else None)
    # a few random-set rows are checked too
    rnd_rows = _sample_rows(wl, seed + 7)[2:4]
    sets_cpu = sets.cpu().numpy()
    for b, t, hq in rnd_rows:
        if (b, t, hq) in ref:
            continue
        K, V = logical_kv(wl, b, hq // G)
        vis = oracle.visible_length(int(wl.seq_lens[b]), wl.q_len, t)
        ref[(b, t, hq)] = (oracle.row_sparse(q[b, t, hq], K, V, sets_cpu[b, t, hq], vis), None)
    o, l = m.sparse_decode_attn(wl.q, cache, sets.contiguous())
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    for r, (sp, _) in ref.items():
        check_attn_row(o[r], l[r], sp[0], sp[1], f"sparse {r}")
    if check_dense:
        od, ld = m.dense_decode_attn(wl.q, cache)
        torch.cuda.synchronize()
        od, ld = od.cpu().numpy(), ld.cpu().numpy()
        for r, (_, dn) in ref.items():
            if dn is not None:
                check_attn_row(od[r], ld[r], dn[0], dn[1], f"dense {r}")
    _check_steps(wl, cache, kt, k_max, kreq, rows, q)


def test_llama3_8b_n32k_k655():
    wl = make_named("llama3_8b_n32k_k655", device="cuda")
    _run(wl, seed=11)


def test_qwen25_72b_n128k_k2621():
    wl = make_named("qwen25_72b_n128k_k2621", device="cuda")
    _run(wl, seed=12)


@pytest.fixture(scope="module")
def sweep_wl():
    wl = make_named("sweep_b16_n128k", device="cuda")
    yield wl
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("level", ["s2", "s5", "s10", "s20", "s50", "s100", "s500", "s1000"])
def test_sweep_b16_n128k(sweep_wl, level):
    _run(sweep_wl, k=SWEEP_K[level], seed=13, check_dense=(level == "s50"))


def test_sweep_b64_n128k_500x():
    """The large-batch sweep point: 64 requests of 131072 positions, k = N/500."""
    wl = make_named("sweep_b64_n128k", device="cuda")
    _run(wl, seed=15)
    del wl
    torch.cuda.empty_cache()


def test_ragged_paged_b32_t4():
    wl = make_named("ragged_paged_b32_t4", device="cuda")
    _run(wl, seed=14)


# ---- the documented limits: max_len = 262144 (the exact indexer's bound) on both indexer paths,
# 64 query rows per KV head, the largest page size, head_dim 64 at a long context

def test_max_len_limit_filtered():
    """262144 positions, k = N/50: the candidate path (k * 8 <= N)."""
    from workloads import make_workload

    wl = make_workload(batch=1, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128, seq_lens=[262144],
                       k=5242, needles_per_head=4, seed=41, device="cuda")
    _run(wl, seed=41)


def test_max_len_limit_full_score():
    """262144 positions, k > N/8: the full-score path (every score, histogram select)."""
    from workloads import make_workload

    wl = make_workload(batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128, seq_lens=[262144],
                       k=40000, needles_per_head=2, seed=42, device="cuda")
    _run(wl, seed=42)


def test_64_query_rows_per_kv_head_paged():
    """G * T = 64 (G = 16, T = 4): four 16-row tiles per KV head, ragged paged requests."""
    from workloads import make_workload

    wl = make_workload(batch=2, q_len=4, num_q_heads=16, num_kv_heads=1, head_dim=128,
                       seq_lens=[20000, 9001], k=0.02, layout="paged", page_size=16, max_len=20000,
                       needles_per_head=2, seed=43, device="cuda")
    _run(wl, seed=43)


def test_64_query_heads_on_one_kv_head_page_4096():
    """G = 64 at T = 1, pages of 4096 positions (the largest page size)."""
    from workloads import make_workload

    wl = make_workload(batch=2, q_len=1, num_q_heads=64, num_kv_heads=1, head_dim=128,
                       seq_lens=[40000, 12289], k=0.02, layout="paged", page_size=4096, max_len=40960,
                       needles_per_head=2, seed=44, device="cuda")
    _run(wl, seed=44)


def test_head_dim_64_long_context():
    """d = 64 at 65536 positions, G = 1, k = N/100."""
    from workloads import make_workload

    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=8, head_dim=64, seq_lens=[65536, 50000],
                       k=655, needles_per_head=2, seed=45, device="cuda")
    _run(wl, seed=45)


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_attention_one_million_positions(layout):
    """sparse_decode_attn and dense_decode_attn (no length bound of their own) at 2**20 positions,
    two query tokens (causal), uniform random index sets of 2% of the row: sampled rows against
    the oracle."""
    from workloads import make_workload

    m = _lib()
    L = 1 << 20
    wl = make_workload(batch=1, q_len=2, num_q_heads=4, num_kv_heads=1, head_dim=128, seq_lens=[L],
                       k=L // 50, layout=layout, page_size=64, seed=46, device="cuda")
    cache = _cache(wl)
    sets = random_index_sets(wl, seed=47)
    o, l = m.sparse_decode_attn(wl.q, cache, sets)
    od, ld = m.dense_decode_attn(wl.q, cache)
    torch.cuda.synchronize()
    o, l, od, ld = o.cpu().numpy(), l.cpu().numpy(), od.cpu().numpy(), ld.cpu().numpy()
    sets_cpu = sets.cpu().numpy()
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    K, V = logical_kv(wl, 0, 0)
    for t, hq in ((0, 0), (1, 3), (1, 1)):
        vis = oracle.visible_length(L, wl.q_len, t)
        want = oracle.row_sparse(q[0, t, hq], K, V, sets_cpu[0, t, hq], vis)
        check_attn_row(o[0, t, hq], l[0, t, hq], want[0], want[1], f"sparse {(t, hq)}")
        want = oracle.row_dense(q[0, t, hq], K, V, vis)
        check_attn_row(od[0, t, hq], ld[0, t, hq], want[0], want[1], f"dense {(t, hq)}")
