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
