"""The decode step under HIP graph capture: every library call queues only kernels on the caller's
stream (no allocation, synchronisation or memset inside the library), so a serving loop can
capture a step once and replay it.  Each replay, with eager work and synchronisations between
replays, must reproduce the eagerly computed outputs bit for bit (the kernels are deterministic)."""

import pytest
import torch

from tests.gpu_util import cache_of
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_step_graph_replays_match_eager(layout):
    m = _lib()
    wl = make_workload(batch=2, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[9000, 4000], k=0.02, layout=layout, page_size=16, max_len=9216,
                       needles_per_head=2, seed=81).to("cuda")
    cache = cache_of(wl)
    k_max = wl.k_max
    sketch = m.key_sketch_build(cache)
    shapes = (wl.batch, wl.q_len, wl.num_q_heads)
    out = torch.empty(*shapes, wl.head_dim, device="cuda")
    lse = torch.empty(*shapes, device="cuda")
    idx = torch.empty(*shapes, k_max, dtype=torch.int32, device="cuda")
    out_s = torch.empty_like(out)
    lse_s = torch.empty_like(lse)
    idx_s = torch.empty_like(idx)
    ws = torch.empty(m.sparse_decode_step_workspace_size(wl.q, cache, k_max), dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(m.sparse_decode_step_sketch_workspace_size(wl.q, cache, k_max, 2), dtype=torch.uint8,
                       device="cuda")

    def step():
        m.sparse_decode_step(wl.q, cache, wl.k_per_req, k_max=k_max, indices=idx, out=out, lse=lse, workspace=ws)
        m.key_sketch_build(cache, sketch, last_n=wl.q_len)
        m.sparse_decode_step_sketch(wl.q, cache, sketch, wl.k_per_req, k_max=k_max, cand_mult=2, indices=idx_s,
                                    out=out_s, lse=lse_s, workspace=ws_s)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (out, lse, idx, out_s, lse_s, idx_s)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on a side stream, as graph capture requires
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (out, lse, idx, out_s, lse_s, idx_s):
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for name, got, w in zip(("out", "lse", "idx", "out_s", "lse_s", "idx_s"),
                                (out, lse, idx, out_s, lse_s, idx_s), want):
            assert torch.equal(got, w), f"replay {rep}: {name} differs from the eager step"


def test_every_entry_point_graph_replays_match_eager():
    """topk_index on both paths (k <= N/8 and larger), sparse attention with splits (partials and
    the combine pass), dense attention, both sketch indexers and the full-score one-call step,
    captured together and replayed with eager work between replays."""
    m = _lib()
    wl = make_workload(batch=2, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[9000, 4000], k=200, layout="paged", page_size=32, max_len=9216,
                       needles_per_head=2, seed=82).to("cuda")
    cache = cache_of(wl)
    k_small, k_big = 200, 1500  # 200 * 8 <= 9216 < 1500 * 8
    kt_small = torch.full((wl.batch,), k_small, dtype=torch.int32, device="cuda")
    kt_big = torch.full((wl.batch,), k_big, dtype=torch.int32, device="cuda")
    sketch = m.key_sketch_build(cache)
    shapes = (wl.batch, wl.q_len, wl.num_q_heads)
    bufs = {
        "idx_small": torch.empty(*shapes, k_small, dtype=torch.int32, device="cuda"),
        "idx_big": torch.empty(*shapes, k_big, dtype=torch.int32, device="cuda"),
        "idx_sk1": torch.empty(*shapes, k_small, dtype=torch.int32, device="cuda"),
        "idx_sk4": torch.empty(*shapes, k_small, dtype=torch.int32, device="cuda"),
        "o_sp": torch.empty(*shapes, wl.head_dim, device="cuda"), "l_sp": torch.empty(*shapes, device="cuda"),
        "o_dn": torch.empty(*shapes, wl.head_dim, device="cuda"), "l_dn": torch.empty(*shapes, device="cuda"),
        "o_st": torch.empty(*shapes, wl.head_dim, device="cuda"), "l_st": torch.empty(*shapes, device="cuda"),
        "idx_st": torch.empty(*shapes, k_big, dtype=torch.int32, device="cuda"),
    }
    ws = {
        "t_small": m.topk_index_workspace_size(wl.q, cache, k_small),
        "t_big": m.topk_index_workspace_size(wl.q, cache, k_big),
        "sp": m.sparse_decode_attn_workspace_size(wl.q, cache, k_small, 4),
        "dn": m.dense_decode_attn_workspace_size(wl.q, cache),
        "sk1": m.topk_index_sketch_workspace_size(wl.q, cache, k_small, 1),
        "sk4": m.topk_index_sketch_workspace_size(wl.q, cache, k_small, 4),
        "st": m.sparse_decode_step_workspace_size(wl.q, cache, k_big),
    }
    ws = {n: torch.empty(max(1, v), dtype=torch.uint8, device="cuda") for n, v in ws.items()}
    b = bufs

    def step():
        m.topk_index(wl.q, cache, kt_small, k_max=k_small, indices=b["idx_small"], workspace=ws["t_small"])
        m.topk_index(wl.q, cache, kt_big, k_max=k_big, indices=b["idx_big"], workspace=ws["t_big"])
        m.sparse_decode_attn(wl.q, cache, b["idx_small"], num_splits=4, out=b["o_sp"], lse=b["l_sp"],
                             workspace=ws["sp"])
        m.dense_decode_attn(wl.q, cache, out=b["o_dn"], lse=b["l_dn"], workspace=ws["dn"])
        m.topk_index_sketch(wl.q, cache, sketch, kt_small, k_max=k_small, cand_mult=1, indices=b["idx_sk1"],
                            workspace=ws["sk1"])
        m.topk_index_sketch(wl.q, cache, sketch, kt_small, k_max=k_small, cand_mult=4, indices=b["idx_sk4"],
                            workspace=ws["sk4"])
        m.sparse_decode_step(wl.q, cache, kt_big, k_max=k_big, indices=b["idx_st"], out=b["o_st"], lse=b["l_st"],
                             workspace=ws["st"])

    step()
    torch.cuda.synchronize()
    want = {n: t.clone() for n, t in bufs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in bufs.values():
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for n, t in bufs.items():
            assert torch.equal(t, want[n]), f"replay {rep}: {n} differs from the eager calls"
