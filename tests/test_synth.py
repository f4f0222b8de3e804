"""CPU checks of the seeded input generator: a paged pool is drawn in a few large generator calls
(not one per page), the draws stay i.i.d. N(0, 1) rounded to bf16, and a workload is
reproducible from its seed."""

import torch

import workloads.synth as synth
from workloads import make_named, make_workload


def _count_randn(monkeypatch):
    calls = []
    real = torch.randn

    def counting(*a, **kw):
        calls.append(1)
        return real(*a, **kw)

    monkeypatch.setattr(torch, "randn", counting)
    return calls


def test_paged_pool_draw_uses_few_generator_calls(monkeypatch):
    # ~12k pages of 16 positions x 2 KV heads x d = 64; slabs of 2^20 values for the test
    monkeypatch.setattr(synth, "_SLAB_VALUES", 1 << 20)
    calls = _count_randn(monkeypatch)
    lens = [50_000, 70_001, 77_777]
    wl = make_workload(batch=3, q_len=4, num_q_heads=8, num_kv_heads=2, head_dim=64,
                       seq_lens=lens, k=0.02, layout="paged", page_size=16, max_len=80_000,
                       seed=5)
    pages = sum(-(-L // 16) for L in lens)
    assert wl.num_pages == pages
    per_pool = -(-pages * 2 * 16 * 64 // (1 << 20))  # slabs per pool
    # q in one call, K and V in per_pool calls each (one page per call would be 2 * pages)
    assert len(calls) <= 1 + 2 * (per_pool + 1)
    assert len(calls) < pages // 100


def test_named_ragged_batch_draw_call_count(monkeypatch):
    # the 32-request ragged paged batch at its real size would allocate ~9 GB here, so count the
    # calls its draw would issue from its shape instead of drawing it
    spec = dict(synth.NAMED["ragged_paged_b32_t4"])
    g = synth._generator(spec["seed"], "lens", "cpu")
    lens = torch.randint(8192, 131073, (spec["batch"],), generator=g).tolist()
    pages = sum(-(-L // 16) for L in lens)
    values = pages * spec["num_kv_heads"] * 16 * spec["head_dim"]
    slabs = -(-values // synth._SLAB_VALUES)
    assert pages > 100_000          # ~1.4e5 pages: one call per page was ~2.8e5 draws
    assert 2 * slabs + 1 < 100       # now a few dozen


def test_slab_draw_is_standard_normal_in_bf16(monkeypatch):
    monkeypatch.setattr(synth, "_SLAB_VALUES", 1 << 14)
    x = synth._normal_bf16((64, 2, 16, 64), synth._generator(1, "t", "cpu"), "cpu")
    assert x.dtype == torch.bfloat16 and x.shape == (64, 2, 16, 64)
    f = x.float().reshape(-1)
    n = f.numel()
    assert abs(float(f.mean())) < 4.0 / n ** 0.5
    assert abs(float(f.var()) - 1.0) < 0.05
    # every value is a bf16 (the low 16 bits of its float32 image are zero)
    assert int((f.view(torch.int32) & 0xFFFF).abs().sum()) == 0
    # slabs are not repeated: no two pages are equal
    pages = x.reshape(64, -1)
    assert torch.unique(pages, dim=0).shape[0] == 64


def test_named_workload_reproducible():
    a = make_named("tiny_d64_n1024")
    b = make_named("tiny_d64_n1024")
    assert torch.equal(a.k_cache, b.k_cache) and torch.equal(a.q, b.q)
    assert a.needles.tolist() == b.needles.tolist()
