"""Pins for the reduced-byte indexer's CPU oracle (oracle/sketch.py): an int8 sketch of every key
row, candidates ranked on the sketch, the final selection re-ranked on exact scores.

Each check compares the oracle with something other than itself: closed forms of rows whose
scale is a power of two, a hand-worked two-key case, the quantisation error bound, brute force by
rank counting over tiny rows, and the reduction to the pinned exact indexer when every visible
position is a candidate."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._util import bf16_from_float, bits, oracle_cache
from workloads import make_workload

RNG = np.random.default_rng(777)


def _bf16(x):
    return oracle.bf16_bits_to_f64(bf16_from_float(x))


# ----------------------------------------------------------------------------- quantisation
def test_power_of_two_scale_closed_form():
    # max |x| = 127 * 2^j makes the scale exactly 2^j; integer multiples of 2^j quantise exactly
    for j in (-8, -3, 0, 2):
        c = RNG.integers(-127, 128, size=(5, 64))
        c[:, 7] = np.where(RNG.random(5) < 0.5, 127, -127)  # the row maxima
        x = c.astype(np.float64) * 2.0 ** j
        assert np.array_equal(_bf16(x), x)
        codes, scale = oracle.int8_sketch(x)
        assert codes.dtype == np.int8 and scale.dtype == np.float32
        assert (scale == np.float32(2.0 ** j)).all()
        np.testing.assert_array_equal(codes, c)


def test_round_half_to_even():
    # scale 1/64: 64 x lands exactly halfway for these values
    x = np.array([[127 / 64, 1 + 1 / 128, 1 + 3 / 128, -(1 + 1 / 128), 0.5 + 1 / 128, 0.0]])
    assert np.array_equal(_bf16(x), x)
    codes, scale = oracle.int8_sketch(x)
    assert scale[0] == np.float32(1 / 64)
    assert codes[0].tolist() == [127, 64, 66, -64, 32, 0]


def test_zero_row_and_sign_symmetry():
    codes, scale = oracle.int8_sketch(np.zeros((1, 16)))
    assert scale[0] == 0 and (codes == 0).all()
    x = _bf16(RNG.normal(size=(20, 128)))
    c1, s1 = oracle.int8_sketch(x)
    c2, s2 = oracle.int8_sketch(-x)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, -c2)


def test_quantisation_error_bound_and_range():
    x = _bf16(RNG.normal(size=(200, 128)) * np.exp(RNG.normal(size=(200, 1))))
    codes, scale = oracle.int8_sketch(x)
    assert np.abs(codes.astype(int)).max() <= 127
    # the largest magnitude of each row quantises to +-127
    am = np.abs(x).argmax(axis=1)
    assert (np.abs(codes[np.arange(200), am].astype(int)) == 127).all()
    # |x - c * scale| <= scale / 2, up to the float32 rounding of the scale and of x / scale
    err = np.abs(x - codes.astype(np.float64) * scale.astype(np.float64)[:, None])
    assert (err <= scale.astype(np.float64)[:, None] * (0.5 + 1e-5)).all()
    # scale is m / 127 rounded once to float32
    m = np.abs(x).max(axis=1)
    for i in range(200):
        exact = Fraction(float(m[i])) / 127
        s = Fraction(float(scale[i]))
        ulp = Fraction(2) ** (math.frexp(float(scale[i]))[1] - 24)
        assert abs(s - exact) <= ulp / 2


# ----------------------------------------------------------------------------- approximate scores
def test_integer_dot_is_exact_bruteforce():
    q = _bf16(RNG.normal(size=32))
    K = _bf16(RNG.normal(size=(9, 32)))
    qc, qs = oracle.int8_sketch(q[None, :])
    kc, ks = oracle.int8_sketch(K)
    got = oracle.sketch_scores(q, kc, ks)
    for n in range(9):
        dot = 0
        for i in range(32):
            dot += int(qc[0, i]) * int(kc[n, i])
        want = np.float32(np.float32(qs[0]) * np.float32(ks[n])) * np.float32(dot)
        assert got[n] == want


def test_representable_rows_give_exact_scores():
    # q and keys with power-of-two scales and integer codes: the sketch score is the exact dot
    q = RNG.integers(-127, 128, size=64).astype(np.float64)
    q[3] = 127
    K = RNG.integers(-127, 128, size=(30, 64)).astype(np.float64) / 8
    K[:, 5] = 127 / 8
    kc, ks = oracle.int8_sketch(K)
    got = oracle.sketch_scores(q, kc, ks)
    np.testing.assert_array_equal(got.astype(np.float64), K @ q)


def test_sketch_score_error_bound():
    # q = qs (cq + eq), K = ks (ck + ek) with |e| <= 1/2 per element, so
    # |q.K - qs ks cq.ck| <= qs ks (sum |cq| / 2 + sum |ck| / 2 + d / 4), plus float32 rounding
    d = 128
    q = _bf16(RNG.normal(size=d))
    K = _bf16(RNG.normal(size=(500, d)))
    qc, qs = oracle.int8_sketch(q[None, :])
    kc, ks = oracle.int8_sketch(K)
    a = oracle.sketch_scores(q, kc, ks).astype(np.float64)
    exact = K @ q
    bound = (float(qs[0]) * ks.astype(np.float64) *
             (np.abs(qc[0]).sum() / 2 + np.abs(kc.astype(int)).sum(axis=1) / 2 + d / 4))
    assert (np.abs(a - exact) <= bound * (1 + 1e-4) + 1e-6 * np.abs(exact)).all()
    # and the error is far below the spread of the scores on random rows
    assert np.abs(a - exact).max() < 0.05 * exact.std()


# ----------------------------------------------------------------------------- selection
def test_hand_worked_two_keys():
    """d = 2, q = (127/64, 0), so q's scale is 1/64 and its codes are (127, 0).
    K0 = (1, 127/64):      codes (64, 127), sketch score (1/64)(1/64)(127 * 64) = 127/64
    K1 = (1 + 1/128, 127/64): 64 * K1[0] = 64.5 rounds to even 64, so the same sketch score,
    and K1 ranks second on the sketch (equal value, higher position) but first exactly.
    K2 = (-1, 127/64):     codes (-64, 127), sketch score -127/64."""
    q = np.array([127 / 64, 0.0])
    K = np.array([[1.0, 127 / 64], [1 + 1 / 128, 127 / 64], [-1.0, 127 / 64]])
    assert np.array_equal(_bf16(K), K)
    kc, ks = oracle.int8_sketch(K)
    assert kc.tolist() == [[64, 127], [64, 127], [-64, 127]]
    a = oracle.sketch_scores(q, kc, ks)
    assert a.tolist() == [127 / 64, 127 / 64, -127 / 64]
    # one candidate: the sketch tie goes to the lower position
    assert oracle.row_topk_sketch(q, K, 3, 1, cand_mult=1).tolist() == [0]
    # two candidates {0, 1}: the exact re-rank picks position 1
    assert oracle.row_topk_sketch(q, K, 3, 1, cand_mult=2).tolist() == [1]
    assert oracle.row_topk(q, K, 3, 1).tolist() == [1]
    # position 2 is never among the top 2
    assert oracle.row_topk_sketch(q, K, 3, 2, cand_mult=1).tolist() == [0, 1]
    # visibility: with only position 0 visible it is the only answer
    assert oracle.row_topk_sketch(q, K, 1, 1, cand_mult=4).tolist() == [0]


def _rank_count_select(vals, n_take, among):
    """Brute force: the members of `among` with fewer than n_take members of `among` ranked
    above them, where j ranks above i if vals[j] > vals[i], or equal and j < i."""
    out = []
    for i in among:
        above = 0
        for j in among:
            if vals[j] > vals[i] or (vals[j] == vals[i] and j < i):
                above += 1
        if above < n_take:
            out.append(i)
    return sorted(out)


@pytest.mark.parametrize("trial", range(30))
def test_selection_bruteforce_rank_counting(trial):
    rng = np.random.default_rng(1000 + trial)
    n, d = int(rng.integers(5, 14)), 8
    # coarse values make ties on both the sketch and the exact scores common
    q = rng.integers(-3, 4, size=d).astype(np.float64) / 2
    K = rng.integers(-3, 4, size=(n, d)).astype(np.float64) / 2
    vis = int(rng.integers(1, n + 1))
    k = int(rng.integers(0, vis + 2))
    m = int(rng.integers(1, 4))
    got = oracle.row_topk_sketch(q, K, vis, k, cand_mult=m).tolist()
    kk = min(k, vis)
    if kk == 0:
        assert got == []
        return
    qc, qs = oracle.int8_sketch(q[None, :])
    kc, ks = oracle.int8_sketch(K[:vis])
    approx = [float(np.float32(np.float32(qs[0]) * ks[i]) * np.float32(int(np.dot(qc[0].astype(int), kc[i].astype(int)))))
              for i in range(vis)]
    cand = _rank_count_select(approx, min(m * kk, vis), list(range(vis)))
    assert oracle.sketch_candidates(q, K, vis, k, m).tolist() == cand
    exact = [float(np.float32(float(np.dot(q, K[i])) / math.sqrt(d))) for i in range(vis)]
    want = _rank_count_select(exact, kk, cand)
    assert got == want


def test_all_candidates_reduces_to_exact_oracle():
    for seed in range(5):
        rng = np.random.default_rng(seed)
        q = _bf16(rng.normal(size=64))
        K = _bf16(rng.normal(size=(200, 64)))
        for vis, k, m in ((200, 10, 20), (150, 7, 1000), (200, 200, 1), (37, 5, 8)):
            np.testing.assert_array_equal(oracle.row_topk_sketch(q, K, vis, k, m),
                                          oracle.row_topk(q, K, vis, k))


def test_recall_high_with_two_fold_candidates():
    # random rows: the exact top-k is recovered (nearly) whole with m = 2
    q = _bf16(RNG.normal(size=128))
    K = _bf16(RNG.normal(size=(4000, 128)))
    want = set(oracle.row_topk(q, K, 4000, 80).tolist())
    got = set(oracle.row_topk_sketch(q, K, 4000, 80, cand_mult=2).tolist())
    assert len(got) == 80 and len(got & want) >= 78


def test_decode_level_layout_gqa_causal():
    wl = make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                       seq_lens=[300, 97], k=20, layout="paged", page_size=16, max_len=320, seed=8)
    cache = oracle_cache(wl)
    qb = bits(wl.q)
    kreq = wl.k_per_req.numpy()
    # every visible position a candidate: the exact oracle indexer
    np.testing.assert_array_equal(oracle.decode_topk_sketch(qb, cache, kreq, wl.k_max, cand_mult=1000),
                                  oracle.decode_topk(qb, cache, kreq, wl.k_max))
    got = oracle.decode_topk_sketch(qb, cache, kreq, wl.k_max, cand_mult=2)
    q = oracle.bf16_bits_to_f64(qb)
    for b in range(2):
        for t in range(2):
            vis = oracle.visible_length(int(wl.seq_lens[b]), 2, t)
            for hq in range(4):
                sel = oracle.row_topk_sketch(q[b, t, hq], cache.keys(b, hq // 2), vis, 20, 2)
                np.testing.assert_array_equal(got[b, t, hq, : sel.size], sel)
                assert (got[b, t, hq, sel.size:] == -1).all()
                assert sel.max() < vis
