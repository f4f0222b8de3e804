"""The allocation-free sparse attention entry point (split partials in the library's fixed
per-GPU scratch) against sparse_decode_attn with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller problem, each bit-identical to the workspace entry point (same
kernels, same split plan) and within the oracle tolerances of the CPU oracle on the same lists."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from tests._util import bits, oracle_cache
from tests.gpu_util import all_rows, cache_of, check_attn_row
from workloads import make_workload, random_index_sets

pytestmark = pytest.mark.gpu


def _case(wl_cpu, num_splits, seed):
    import long_context_sparse_oracle_amd as m
    from long_context_sparse_oracle_amd import _lib

    wl = wl_cpu.to("cuda")
    cache = cache_of(wl)
    idx = random_index_sets(wl_cpu, seed=seed)
    idx[..., ::7] = -1  # padding inside the lists
    idx_dev = idx.to("cuda")
    shp = _lib._shape(wl.q, cache)
    k_max = int(idx.shape[3])
    # the split plan must use the scratch (more than one split per row)
    need = int(_lib.LIB.sparse_decode_attn_workspace_size(ctypes.byref(shp), k_max, num_splits))
    assert 0 < need <= 4 << 20
    out_n = torch.full((wl.batch, wl.q_len, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
    lse_n = torch.full((wl.batch, wl.q_len, wl.num_q_heads), float("nan"), device="cuda")
    desc = cache.desc()
    print(f"[no_alloc] B{wl.batch} T{wl.q_len} Hq{wl.num_q_heads} Hkv{wl.num_kv_heads} d{wl.head_dim} "
          f"k_max {k_max} splits {num_splits} scratch {need} B", flush=True)
    st = _lib.LIB.sparse_decode_attn_noalloc(
        ctypes.byref(shp), wl.q.data_ptr(), ctypes.byref(desc), idx_dev.data_ptr(), k_max,
        _lib._scale(wl.head_dim, None), num_splits, out_n.data_ptr(), lse_n.data_ptr(), _lib._stream(wl.q))
    assert st == 0, _lib.STATUS_NAMES.get(st, st)
    out_w, lse_w = m.sparse_decode_attn(wl.q, cache, idx_dev, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_w), float((out_n - out_w).abs().max())
    assert torch.equal(lse_n, lse_w)
    # and against the oracle on the same lists
    qb = bits(wl_cpu.q)
    o_ref, l_ref = oracle.decode_sparse(qb, oracle_cache(wl_cpu), idx.numpy())
    o, l = out_n.cpu().numpy(), lse_n.cpu().numpy()
    for b, t, hq in all_rows(wl_cpu):
        check_attn_row(o[b, t, hq], l[b, t, hq], o_ref[b, t, hq], l_ref[b, t, hq], f"row {(b, t, hq)}")
    return need


def test_noalloc_matches_workspace_entry_point_twice_second_smaller():
    big = make_workload(batch=2, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        seq_lens=[4096, 3001], k=600, layout="paged", page_size=16, max_len=4096, seed=71)
    small = make_workload(batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                          seq_lens=[1000], k=300, max_len=1024, seed=72)
    need_big = _case(big, 0, 1)
    need_small = _case(small, 0, 2)
    assert need_small < need_big
    # an explicit split count, again on the smaller problem after the larger one
    _case(big, 5, 3)
    _case(small, 3, 4)


def test_noalloc_refuses_plans_beyond_the_scratch():
    import long_context_sparse_oracle_amd as m

    wl = make_workload(batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[2048, 2048], k=1000, seed=73).to("cuda")
    cache = cache_of(wl)
    idx = random_index_sets(wl, seed=5)
    with pytest.raises(m.CtxSparseError) as ei:
        m.sparse_decode_attn_noalloc(wl.q, cache, idx, num_splits=1000)
    assert ei.value.status == 5
