"""Calls from two host threads, each on its own stream (default priority) with its own buffers and
workspaces, run concurrently and give the same results, bit for bit, as the same calls run one
after the other: the library keeps no mutable state between calls."""

import threading

import pytest
import torch

from tests.gpu_util import cache_of
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_sparse_oracle_amd as m

    return m


def _setup(seed, layout):
    m = _lib()
    wl = make_workload(batch=2, q_len=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                       seq_lens=[12000, 7000], k=0.02, layout=layout, page_size=16, max_len=12288,
                       needles_per_head=2, seed=seed).to("cuda")
    cache = cache_of(wl)
    k = wl.k_max
    shapes = (wl.batch, wl.q_len, wl.num_q_heads)
    bufs = {"idx": torch.empty(*shapes, k, dtype=torch.int32, device="cuda"),
            "o": torch.empty(*shapes, wl.head_dim, device="cuda"), "l": torch.empty(*shapes, device="cuda"),
            "od": torch.empty(*shapes, wl.head_dim, device="cuda"), "ld": torch.empty(*shapes, device="cuda"),
            "os": torch.empty(*shapes, wl.head_dim, device="cuda"), "ls": torch.empty(*shapes, device="cuda")}
    ws = [torch.empty(max(1, n), dtype=torch.uint8, device="cuda") for n in (
        m.topk_index_workspace_size(wl.q, cache, k), m.sparse_decode_attn_workspace_size(wl.q, cache, k),
        m.dense_decode_attn_workspace_size(wl.q, cache), m.sparse_decode_step_workspace_size(wl.q, cache, k))]

    def calls():
        m.topk_index(wl.q, cache, wl.k_per_req, k_max=k, indices=bufs["idx"], workspace=ws[0])
        m.sparse_decode_attn(wl.q, cache, bufs["idx"], out=bufs["o"], lse=bufs["l"], workspace=ws[1])
        m.dense_decode_attn(wl.q, cache, out=bufs["od"], lse=bufs["ld"], workspace=ws[2])
        m.sparse_decode_step(wl.q, cache, wl.k_per_req, k_max=k, out=bufs["os"], lse=bufs["ls"], workspace=ws[3])

    return calls, bufs


def test_two_threads_two_streams_match_sequential():
    jobs = [_setup(91, "contiguous"), _setup(92, "paged")]
    for calls, _ in jobs:
        calls()
    torch.cuda.synchronize()
    want = [{n: t.clone() for n, t in bufs.items()} for _, bufs in jobs]
    for _, bufs in jobs:
        for t in bufs.values():
            t.zero_()
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    jobs[i][0]()
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (_, bufs) in enumerate(jobs):
        for n, t in bufs.items():
            assert torch.equal(t, want[i][n]), f"job {i}: {n} differs from the sequential run"
