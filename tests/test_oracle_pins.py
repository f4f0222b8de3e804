"""Pins for the CPU oracle: each check compares it with something other than itself (exact
rational arithmetic, brute force over all subsets, closed forms, SciPy routines, invariants), so a
dropped term, a wrong sign, a wrong index or a transposed operand fails at least one of them."""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests._util import bf16_from_float, bits, oracle_cache
from workloads import make_workload

RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------------------- bf16 decoding
def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, math.inf, 2.0 ** -133, 3.140625]
    got = oracle.bf16_bits_to_f64(pats)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_bf16_decode_matches_torch():
    x = torch.randn(4096, generator=torch.Generator().manual_seed(1)) * 100
    b = x.to(torch.bfloat16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits(b)), b.float().double().numpy())


# ----------------------------------------------------------------------------- scores
def _exact_dot(q, k):
    return sum(Fraction(float(a)) * Fraction(float(c)) for a, c in zip(q, k))


def test_scores_exact_rational_bruteforce():
    # d = 4 so the default scale 1/sqrt(4) = 1/2 is exact; keys are a non-square 7 x 4 block so a
    # transposed operand cannot produce the right shape or values.
    q = oracle.bf16_bits_to_f64(bf16_from_float(RNG.normal(size=4)))
    K = oracle.bf16_bits_to_f64(bf16_from_float(RNG.normal(size=(7, 4))))
    got = oracle.scaled_scores(q, K)
    assert got.shape == (7,)
    for n in range(7):
        want = _exact_dot(q, K[n]) / 2
        assert got[n] == float(want)


def test_scores_default_scale_closed_form():
    d = 128
    q = oracle.bf16_bits_to_f64(bf16_from_float(RNG.normal(size=d)))
    K = np.stack([c * q for c in (3.0, -2.0, 0.5)])
    got = oracle.scaled_scores(q, K)
    nq2 = float(np.sum(q * q))
    np.testing.assert_allclose(got, [c * nq2 / math.sqrt(d) for c in (3.0, -2.0, 0.5)], rtol=1e-13)


def test_scores_orthogonal_is_zero_and_sign():
    q = np.array([1.0, 0.0, 0.0, 0.0])
    K = np.array([[0.0, 5.0, 0.0, 0.0], [-2.0, 0.0, 0.0, 0.0]])
    np.testing.assert_array_equal(oracle.scaled_scores(q, K), [0.0, -1.0])


# ----------------------------------------------------------------------------- top-k
def _dominance_sets(s, k):
    """All subsets S of size k with: for i in S, j not in S, s_i > s_j or (s_i == s_j and i < j)."""
    n = len(s)
    found = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        ok = all(
            (s[i] > s[j]) or (s[i] == s[j] and i < j)
            for i in Sset
            for j in range(n)
            if j not in Sset
        )
        if ok:
            found.append(S)
    return found


@pytest.mark.parametrize("trial", range(40))
def test_topk_bruteforce_with_ties(trial):
    rng = np.random.default_rng(trial)
    n = int(rng.integers(1, 9))
    s = rng.integers(-3, 4, size=n).astype(np.float64)  # small integers: many exact ties
    for k in range(0, n + 1):
        sets = _dominance_sets(list(s), k)
        assert len(sets) == 1
        np.testing.assert_array_equal(oracle.topk_positions(s, k), np.array(sets[0], dtype=np.int64))


def test_topk_float32_decision():
    # differ only below float32 resolution -> a tie -> lower position wins
    assert oracle.topk_positions(np.array([1.0, 1.0 + 1e-12]), 1).tolist() == [0]
    # differ by one float32 ulp -> the larger one wins
    assert oracle.topk_positions(np.array([1.0, 1.0 + 2.0 ** -23]), 1).tolist() == [1]


def test_topk_signed_not_magnitude_and_zero_ties():
    assert oracle.topk_positions(np.array([-5.0, 1.0, -0.5]), 1).tolist() == [1]
    assert oracle.topk_positions(np.array([-5.0, 1.0, -0.5]), 2).tolist() == [1, 2]
    assert oracle.topk_positions(np.array([-0.0, 0.0]), 1).tolist() == [0]
    assert oracle.topk_positions(np.array([0.0, -0.0]), 1).tolist() == [0]


def test_topk_clamps_and_empty():
    assert oracle.topk_positions(np.array([2.0, 1.0]), 5).tolist() == [0, 1]
    assert oracle.topk_positions(np.array([2.0, 1.0]), 0).tolist() == []
    assert oracle.topk_positions(np.array([]), 3).tolist() == []


def test_topk_random_vs_full_sort_of_pairs():
    # larger n: compare with Python's sort of (-s, n) pairs on float32-rounded scores
    for trial in range(10):
        rng = np.random.default_rng(100 + trial)
        n = int(rng.integers(10, 300))
        s = np.round(rng.normal(size=n), 2)  # 2 decimals: plenty of exact ties
        k = int(rng.integers(0, n + 1))
        pairs = sorted((-float(np.float32(x)), i) for i, x in enumerate(s))
        want = sorted(i for _, i in pairs[:k])
        assert oracle.topk_positions(s, k).tolist() == want


# ----------------------------------------------------------------------------- attention
def test_attend_single_token():
    v = RNG.normal(size=(1, 8))
    o, lse = oracle.attend(np.array([0.7]), v)
    np.testing.assert_array_equal(o, v[0])
    assert lse == 0.7


def test_attend_all_equal_scores_is_mean():
    v = RNG.normal(size=(9, 16))
    o, lse = oracle.attend(np.full(9, -1.25), v)
    np.testing.assert_allclose(o, v.mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse - (-1.25 + math.log(9))) < 1e-14


def test_attend_two_tokens_logistic():
    v = RNG.normal(size=(2, 5))
    for s1, s2 in [(0.3, -1.1), (1000.0, 999.0), (-40.0, 3.0)]:
        o, lse = oracle.attend(np.array([s1, s2]), v)
        want = scipy.special.expit(s1 - s2) * v[0] + scipy.special.expit(s2 - s1) * v[1]
        np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-15)
        assert abs(lse - np.logaddexp(s1, s2)) < 1e-12


def test_attend_matches_scipy_softmax():
    s = RNG.normal(size=200) * 4
    v = RNG.normal(size=(200, 32))
    o, lse = oracle.attend(s, v)
    np.testing.assert_allclose(o, scipy.special.softmax(s) @ v, rtol=1e-12, atol=1e-14)
    assert abs(lse - scipy.special.logsumexp(s)) < 1e-12


def test_attend_empty():
    o, lse = oracle.attend(np.array([]), np.zeros((0, 4)))
    np.testing.assert_array_equal(o, np.zeros(4))
    assert lse == -math.inf


def test_weights_sum_to_one():
    for n in (1, 2, 17, 1000):
        w = oracle.attention_weights(RNG.normal(size=n) * 10)
        assert abs(w.sum() - 1.0) < 1e-12 and (w >= 0).all()


def _tiny_case(n=40, d=16, seed=0):
    rng = np.random.default_rng(seed)
    q = oracle.bf16_bits_to_f64(bf16_from_float(rng.normal(size=d)))
    K = oracle.bf16_bits_to_f64(bf16_from_float(rng.normal(size=(n, d))))
    V = oracle.bf16_bits_to_f64(bf16_from_float(rng.normal(size=(n, d))))
    return q, K, V


def test_sparse_order_invariant():
    q, K, V = _tiny_case()
    pos = np.array([3, 17, 5, 39, 0, 22])
    o1, l1 = oracle.row_sparse(q, K, V, pos, 40)
    for perm in itertools.islice(itertools.permutations(range(6)), 1, 30):
        o2, l2 = oracle.row_sparse(q, K, V, pos[list(perm)], 40)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
        assert abs(l2 - l1) < 1e-14


def test_sparse_padding_and_duplicates():
    q, K, V = _tiny_case()
    s = oracle.scaled_scores(q, K)
    o, lse = oracle.row_sparse(q, K, V, np.array([4, -1, 4, 9, -1]), 40)
    # a repeated entry counts twice: the same as one entry with weight doubled (score + ln 2)
    want_o, want_l = oracle.attend(np.array([s[4] + math.log(2), s[9]]), V[[4, 9]])
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-14)
    assert abs(lse - want_l) < 1e-13
    o, lse = oracle.row_sparse(q, K, V, np.array([-1, -1]), 40)
    assert lse == -math.inf and not o.any()


def test_sparse_rejects_out_of_range():
    q, K, V = _tiny_case()
    with pytest.raises(ValueError):
        oracle.row_sparse(q, K, V, np.array([3, 40]), 40)
    with pytest.raises(ValueError):
        oracle.row_sparse(q, K, V, np.array([3, 30]), 30)


def test_sparse_k_equals_n_is_dense():
    q, K, V = _tiny_case()
    o1, l1 = oracle.row_sparse(q, K, V, np.arange(40)[::-1], 40)
    o2, l2 = oracle.row_dense(q, K, V, 40)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    assert abs(l1 - l2) < 1e-13
    # dense equals the textbook formula via SciPy
    s = oracle.scaled_scores(q, K)
    np.testing.assert_allclose(o2, scipy.special.softmax(s) @ V, rtol=1e-12, atol=1e-14)


def test_lse_merge_partition_invariance():
    q, K, V = _tiny_case(n=120, seed=3)
    rng = np.random.default_rng(7)
    pos = rng.permutation(120)[:77]
    whole = oracle.row_sparse(q, K, V, pos, 120)
    for trial in range(20):
        cuts = np.sort(rng.integers(0, 78, size=int(rng.integers(1, 9))))
        pieces = np.split(pos, cuts)  # may include empty pieces
        parts = [oracle.row_sparse(q, K, V, p, 120) for p in pieces]
        o, lse = oracle.lse_merge(parts)
        np.testing.assert_allclose(o, whole[0], rtol=0, atol=1e-13)
        assert abs(lse - whole[1]) < 1e-12


def test_topk_set_maximises_attention_mass():
    # the top-k set is the size-k subset with the largest total softmax weight (softmax is monotone
    # in the score); brute force over all subsets of a tiny row
    q, K, V = _tiny_case(n=9, d=8, seed=11)
    s = oracle.scaled_scores(q, K)
    w = oracle.attention_weights(s)
    for k in range(1, 9):
        best = max(itertools.combinations(range(9), k), key=lambda S: sum(w[list(S)]))
        assert oracle.row_topk(q, K, 9, k).tolist() == sorted(best)


# ----------------------------------------------------------------------------- step level
def _small(layout="contiguous", T=1, seed=5, lens=(300, 257), k=20, Hq=4, Hkv=2, needles=0):
    return make_workload(
        batch=len(lens), q_len=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=64,
        seq_lens=list(lens), k=k, layout=layout, page_size=16, max_len=320,
        needles_per_head=needles, seed=seed,
    )


def test_paged_cache_matches_contiguous_gather():
    wl = _small(layout="paged", lens=(300, 97))
    cache = oracle_cache(wl)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        for h in range(wl.num_kv_heads):
            # independent gather: walk pages one by one with torch
            rows = []
            for p in range(-(-L // 16)):
                rows.append(wl.k_cache[int(wl.page_table[b, p]), h].float())
            want = torch.cat(rows)[:L].double().numpy()
            np.testing.assert_array_equal(cache.keys(b, h), want)


def test_page_permutation_invariance():
    # the same logical cache stored contiguously and paged gives identical oracle results
    wl = _small(layout="paged", lens=(300, 97), T=2)
    cache_p = oracle_cache(wl)
    B, Hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    kc = np.zeros((B, Hkv, 320, d), np.uint16)
    vc = np.zeros((B, Hkv, 320, d), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            L = cache_p.seq_lens[b]
            for n in range(L):
                page = int(wl.page_table[b, n // 16])
                kc[b, h, n] = bits(wl.k_cache[page, h, n % 16])
                vc[b, h, n] = bits(wl.v_cache[page, h, n % 16])
    cache_c = oracle.Cache(kc, vc, wl.seq_lens.numpy())
    qb = bits(wl.q)
    i_p = oracle.decode_topk(qb, cache_p, wl.k_per_req.numpy(), wl.k_max)
    i_c = oracle.decode_topk(qb, cache_c, wl.k_per_req.numpy(), wl.k_max)
    np.testing.assert_array_equal(i_p, i_c)
    o_p, l_p = oracle.decode_dense(qb, cache_p)
    o_c, l_c = oracle.decode_dense(qb, cache_c)
    np.testing.assert_array_equal(o_p, o_c)
    np.testing.assert_array_equal(l_p, l_c)


def test_causality_last_position_only_for_last_token():
    T, L, d = 4, 64, 64
    wl = make_workload(batch=1, q_len=T, num_q_heads=2, num_kv_heads=1, head_dim=d,
                       seq_lens=[L], k=3, seed=9)
    # plant a dominant key for every token at the last position
    q = wl.q.float()
    wl.k_cache[0, 0, L - 1] = (10.0 * q[0, :, 0].sum(0) / q[0, :, 0].sum(0).norm()).to(torch.bfloat16)
    cache = oracle_cache(wl)
    idx = oracle.decode_topk(bits(wl.q), cache, [3], 3)
    for t in range(T - 1):
        assert (L - 1) not in idx[0, t].tolist()
        assert idx[0, t].max() <= L - T + t
    assert oracle.visible_length(L, T, T - 1) == L
    # dense: changing V at the last position moves only the last token's outputs
    o1, _ = oracle.decode_dense(bits(wl.q), cache)
    wl.v_cache[0, 0, L - 1] += 5.0
    o2, _ = oracle.decode_dense(bits(wl.q), oracle_cache(wl))
    np.testing.assert_array_equal(o1[0, : T - 1], o2[0, : T - 1])
    assert np.abs(o1[0, T - 1] - o2[0, T - 1]).max() > 1e-3


def test_gqa_head_mapping():
    # Hq = 4 on Hkv = 2: query heads 0,1 read KV head 0, heads 2,3 read KV head 1
    wl = _small(lens=(100, 100), k=5)
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    o1, _ = oracle.decode_dense(qb, cache)
    wl.v_cache[:, 1] = (wl.v_cache[:, 1].float() + 1.0).to(torch.bfloat16)
    o2, _ = oracle.decode_dense(qb, oracle_cache(wl))
    np.testing.assert_array_equal(o1[:, :, :2], o2[:, :, :2])
    assert np.abs(o1[:, :, 2:] - o2[:, :, 2:]).min() > 0


def test_needles_are_selected():
    wl = make_workload(batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                       seq_lens=[1024], k=32, needles_per_head=1, seed=1001)
    idx = oracle.decode_topk(bits(wl.q), oracle_cache(wl), wl.k_per_req.numpy(), wl.k_max)
    for b, t, hq, p in wl.needles.tolist():
        assert p in idx[b, t, hq].tolist()


def test_decode_topk_matches_rowwise_and_padding():
    wl = _small(T=2, lens=(300, 30), k=40)
    cache = oracle_cache(wl)
    idx = oracle.decode_topk(bits(wl.q), cache, wl.k_per_req.numpy(), wl.k_max)
    q = oracle.bf16_bits_to_f64(bits(wl.q))
    for b in range(2):
        for t in range(2):
            vis = oracle.visible_length(int(wl.seq_lens[b]), 2, t)
            for hq in range(4):
                sel = oracle.row_topk(q[b, t, hq], cache.keys(b, hq // 2), vis, 40)
                assert sel.size == min(40, vis)
                np.testing.assert_array_equal(idx[b, t, hq, : sel.size], sel)
                assert (idx[b, t, hq, sel.size:] == -1).all()
                s = oracle.scaled_scores(q[b, t, hq], cache.keys(b, hq // 2)[:vis])
                # every selected score is >= every unselected score (up to float32 rounding)
                unsel = np.setdiff1d(np.arange(vis), sel)
                if unsel.size and sel.size:
                    assert np.float32(s[sel].min()) >= np.float32(s[unsel].max())


def test_kth_score():
    q, K, V = _tiny_case(n=50)
    s = oracle.scaled_scores(q, K)
    assert oracle.kth_score(q, K, 50, 1) == s.max()
    assert oracle.kth_score(q, K, 50, 50) == s.min()


def test_golden_fixture_reproduced():
    """The oracle still reproduces its stored output for the tiny seeded decode step."""
    import json
    import os

    from workloads import make_named

    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_d64_n1024.json")
    with open(path) as f:
        rec = json.load(f)
    wl = make_named("tiny_d64_n1024", device="cpu")
    assert wl.needles.tolist() == rec["needles"]
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    idx = oracle.decode_topk(qb, cache, wl.k_per_req.numpy(), wl.k_max)
    np.testing.assert_array_equal(idx, np.array(rec["topk_indices"]))
    o, lse = oracle.decode_sparse(qb, cache, idx)
    np.testing.assert_allclose(o, rec["sparse_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rec["sparse_lse"], rtol=0, atol=1e-12)
    o, lse = oracle.decode_dense(qb, cache)
    np.testing.assert_allclose(o, rec["dense_out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rec["dense_lse"], rtol=0, atol=1e-12)
    # every needle is in its head's selection
    for b, t, hq, p in rec["needles"]:
        assert p in rec["topk_indices"][b][t][hq]


# ----------------------------------------------------------------------------- decode_sparse
def _gqa_ragged_paged(seed=21):
    # GQA 8:2 (four query heads per KV head), three new tokens per request, ragged lengths,
    # paged cache with a permuted page table
    return make_workload(
        batch=3, q_len=3, num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=[70, 33, 129],
        k=9, layout="paged", page_size=16, max_len=144, needles_per_head=0, seed=seed,
    )


def test_decode_sparse_all_visible_equals_dense():
    """Sparse attention over every visible position, listed shuffled and -1 padded, is dense
    attention (the method's k = N case), row by row; a wrong KV-head map or a causal window that
    ignores the token index gives a different row or an out-of-range entry."""
    wl = _gqa_ragged_paged()
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    B, T, Hq = wl.batch, wl.q_len, wl.num_q_heads
    lens = wl.seq_lens.tolist()
    kpad = max(lens) + 5
    idx = np.full((B, T, Hq, kpad), -1, dtype=np.int32)
    rng = np.random.default_rng(7)
    for b in range(B):
        for t in range(T):
            vis = lens[b] - T + t + 1  # token t of the T appended tokens sees 0 .. L - T + t
            for hq in range(Hq):
                slots = rng.permutation(kpad)[:vis]  # padding interleaved, not only at the end
                idx[b, t, hq, slots] = rng.permutation(vis)
    o_s, l_s = oracle.decode_sparse(qb, cache, idx)
    o_d, l_d = oracle.decode_dense(qb, cache)
    np.testing.assert_allclose(o_s, o_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_s, l_d, rtol=0, atol=1e-12)


def test_decode_sparse_against_independent_page_walk():
    """Sampled rows of `decode_sparse` against a row computed here without the oracle's cache
    view, head map or causal window: K and V gathered by walking the page table with torch, the
    KV head written out per query head, softmax by SciPy."""
    wl = _gqa_ragged_paged(seed=22)
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    B, T, Hq, d = wl.batch, wl.q_len, wl.num_q_heads, wl.head_dim
    lens = wl.seq_lens.tolist()
    kv_head_of = [0, 0, 0, 0, 1, 1, 1, 1]  # Hq = 8 on Hkv = 2, contiguous groups of four
    rng = np.random.default_rng(8)
    kmax = 12
    idx = np.full((B, T, Hq, kmax), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            last = lens[b] - T + t  # last position token t may see
            for hq in range(Hq):
                n = int(rng.integers(1, kmax + 1))
                idx[b, t, hq, :n] = rng.integers(0, last + 1, size=n)  # repeats allowed
                if t == T - 1:
                    idx[b, t, hq, 0] = last  # the last token reaches the newest position
    o, lse = oracle.decode_sparse(qb, cache, idx)
    q = wl.q.double()
    for b, t, hq in [(0, 0, 0), (0, 2, 7), (1, 1, 3), (1, 2, 4), (2, 0, 5), (2, 2, 1), (2, 1, 6)]:
        h = kv_head_of[hq]
        pos = [int(p) for p in idx[b, t, hq] if p != -1]
        krows = torch.stack([wl.k_cache[int(wl.page_table[b, p // 16]), h, p % 16] for p in pos])
        vrows = torch.stack([wl.v_cache[int(wl.page_table[b, p // 16]), h, p % 16] for p in pos])
        s = (krows.double() @ q[b, t, hq]).numpy() / math.sqrt(d)
        w = scipy.special.softmax(s)
        np.testing.assert_allclose(o[b, t, hq], w @ vrows.double().numpy(), rtol=0, atol=1e-12)
        assert abs(lse[b, t, hq] - scipy.special.logsumexp(s)) <= 1e-12


def test_decode_sparse_rejects_positions_past_each_tokens_window():
    """Token t of T sees positions 0 .. L - T + t: one entry past that window is an error for
    every token, and the same entry is accepted by the next token."""
    wl = _gqa_ragged_paged(seed=23)
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    B, T, Hq = wl.batch, wl.q_len, wl.num_q_heads
    lens = wl.seq_lens.tolist()
    for b in range(B):
        for t in range(T):
            idx = np.full((B, T, Hq, 2), -1, dtype=np.int32)
            idx[b, t, 5, 0] = lens[b] - T + t + 1
            with pytest.raises(ValueError):
                oracle.decode_sparse(qb, cache, idx, rows=[(b, t, 5)])
            if t + 1 < T:
                idx2 = np.full((B, T, Hq, 2), -1, dtype=np.int32)
                idx2[b, t + 1, 5, 0] = lens[b] - T + t + 1
                oracle.decode_sparse(qb, cache, idx2, rows=[(b, t + 1, 5)])
