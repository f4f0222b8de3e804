"""GPU parity of the one-call decode step (sparse_decode_step): the indexer and the sparse
attention together, fused per row when k <= max_len / 8.

Each row is checked against the CPU oracle twice: its index list by the indexer's band rule, and
(out, lse) against the oracle's sparse attention over that same list -- a set that differs from
the oracle's only inside the 1e-3 band can still move out by more than 2e-3 when many weights are
alike, so the attention is compared on the list the step actually used.
"""

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits, oracle_cache
from tests.gpu_util import all_rows, cache_of, check_attn_row, check_topk_row, threshold_regimes_workload
from workloads import make_named, make_workload

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


def _check_step(wl_cpu, k_max=None, rows=None):
    m = _lib()
    wl = wl_cpu.to("cuda")
    kmax = wl.k_max if k_max is None else k_max
    out, lse, idx = m.sparse_decode_step(wl.q, cache_of(wl), wl.k_per_req, k_max=kmax,
                                         return_indices=True)
    # the same step without asking for the lists gives the same outputs
    out2, lse2 = m.sparse_decode_step(wl.q, cache_of(wl), wl.k_per_req, k_max=kmax)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    out, lse, idx = out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()
    q = oracle.bf16_bits_to_f64(bits(wl_cpu.q))
    ocache = oracle_cache(wl_cpu)
    kreq = wl_cpu.k_per_req.numpy()
    for b, t, hq in rows if rows is not None else all_rows(wl_cpu):
        K = ocache.keys(b, hq // wl.group)
        V = ocache.values(b, hq // wl.group)
        vis = oracle.visible_length(ocache.seq_lens[b], wl.q_len, t)
        check_topk_row(idx[b, t, hq], q[b, t, hq], K, vis, min(int(kreq[b]), kmax), f"row {(b, t, hq)}")
        want = oracle.row_sparse(q[b, t, hq], K, V, idx[b, t, hq], vis)
        check_attn_row(out[b, t, hq], lse[b, t, hq], want[0], want[1], f"step row {(b, t, hq)}")


def test_step_threshold_rule_regimes():
    """The one-call step over the same rows as the indexer's threshold-regime test: very sparse
    rows, a row recomputed in full after its slots overflow, rows where every position is a
    candidate."""
    _check_step(threshold_regimes_workload())


def test_step_fused_gqa_ragged_tail():
    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[20000, 7777], k=0.02, max_len=20003, needles_per_head=3, seed=51)
    _check_step(wl)


def test_step_fused_paged_causal_d64():
    wl = make_workload(batch=3, q_len=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       seq_lens=[9000, 2500, 300], k=0.02, layout="paged", page_size=16,
                       max_len=9216, needles_per_head=2, seed=52)
    _check_step(wl)


def test_step_fused_gqa_two_row_tiles():
    wl = make_workload(batch=1, q_len=4, num_q_heads=16, num_kv_heads=2, head_dim=128,
                       seq_lens=[6000], k=100, seed=53)
    _check_step(wl)


def test_step_per_request_k_zero_and_all():
    # k_max 256 of 4096 (fused); request 0 asks for none, request 3 for more than it has
    wl = make_workload(batch=4, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
                       seq_lens=[4096, 1000, 3000, 200], k=[0, 5, 256, 256], max_len=4096, seed=54)
    _check_step(wl, k_max=256)


def test_step_full_score_path():
    # k > max_len / 8: indexer and attention run back to back
    wl = make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=128,
                       seq_lens=[4096, 3000], k=600, max_len=4096, seed=55)
    _check_step(wl)


def test_step_fallback_rows():
    # the sampled positions carry planted high keys, so the rows are recomputed in full
    L, k = 32768, 655
    wl = make_workload(batch=1, q_len=1, num_q_heads=2, num_kv_heads=2, head_dim=128,
                       seq_lens=[L], k=k, seed=56)
    for h in range(2):
        qh = wl.q[0, 0, h].float()
        wl.k_cache[0, h, torch.arange(100) * (L // 1024)] = (3.0 * qh / qh.norm()).to(torch.bfloat16)
    _check_step(wl)


def test_step_llama3_8b_n32k_k655_sampled_rows():
    wl = make_named("llama3_8b_n32k_k655", device="cpu")
    rng = np.random.default_rng(57)
    rows = [(0, 0, 0), (7, 0, 31)] + [(int(rng.integers(8)), 0, int(rng.integers(32))) for _ in range(6)]
    _check_step(wl, rows=rows)
