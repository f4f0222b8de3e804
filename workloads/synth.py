"""Seeded synthetic long-context decode inputs.

Each workload is one decode step of a GQA attention layer: queries for T new tokens per request,
a bf16 KV cache (contiguous or paged), per-request cached lengths and per-request selection sizes.
The shapes follow the decode settings discussed on the pages about inference-time context
sparsity (page "Inference Time Context Sparsity: Illusion or Opportunity?", method section:
retrieval at 32K and 128K context, agentic coding past 100K; results section C: sparse decode at
50x sparsity, i.e. about 2% of tokens kept).  The pages' task suites are not used; these seeded
tensors stand in for them and only reproduce their context lengths.

Everything here is input drawing.  No score, selection or attention arithmetic lives in this
module, so the CPU oracle and the HIP library can both consume its output without sharing code.

Random streams: every tensor draws from its own ``torch.Generator`` seeded from
``numpy.random.SeedSequence([seed, crc32(tag)])``, so a workload is reproducible on a given
device type.  CPU and GPU generators are different algorithms; a test that needs the same values
on both sides generates once and copies.
"""

from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = ["Workload", "make_workload", "make_named", "random_index_sets", "NAMED"]


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.

    Layouts (all row-major):
      q          bf16 [B, T, Hq, d]
      k_cache    bf16 contiguous [B, Hkv, max_len, d]  or paged pool [num_pages, Hkv, page_size, d]
      v_cache    same as k_cache
      page_table int32 [B, max_pages] (paged only); entries past a request's last page are 0
      seq_lens   int32 [B]: cached length L_b, counting the T new tokens
      k_per_req  int32 [B]: selection size per (token, query head) row of request b
      needles    int64 [n, 4] rows (b, t, hq, position): keys planted as 3x the unit query of
                 (b, t, hq) at that logical position
    """

    name: str
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    layout: str
    max_len: int
    page_size: int
    num_pages: int
    seq_lens: torch.Tensor
    k_per_req: torch.Tensor
    k_max: int
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    page_table: Optional[torch.Tensor]
    needles: torch.Tensor
    seed: int
    structure: str

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        return self.batch * self.q_len * self.num_q_heads

    @property
    def max_pages(self) -> int:
        return 0 if self.page_table is None else int(self.page_table.shape[1])

    def to(self, device) -> "Workload":
        """Copy every tensor to `device` (e.g. a CPU-drawn workload onto the GPU)."""
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return dataclasses.replace(
            self,
            seq_lens=mv(self.seq_lens),
            k_per_req=mv(self.k_per_req),
            q=mv(self.q),
            k_cache=mv(self.k_cache),
            v_cache=mv(self.v_cache),
            page_table=mv(self.page_table),
            needles=mv(self.needles),
        )

    def kv_bytes(self) -> int:
        """Bytes of K plus V actually cached (sum of lengths, all KV heads)."""
        total_tokens = int(self.seq_lens.to("cpu", torch.int64).sum())
        return 2 * total_tokens * self.num_kv_heads * self.head_dim * 2


def _generator(seed: int, tag: str, device) -> torch.Generator:
    ss = np.random.SeedSequence([int(seed), zlib.crc32(tag.encode())])
    state = int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(state)
    return g


# values per generator call when drawing N(0, 1) tensors (256 MB of float32 staging)
_SLAB_VALUES = 1 << 26


def _normal_bf16(shape: Sequence[int], gen: torch.Generator, device) -> torch.Tensor:
    """i.i.d. N(0, 1) drawn in fp32 and rounded to bf16 (round to nearest even).

    The draw goes in slabs of whole leading slices, up to 2^26 values (256 MB of fp32 staging)
    per call, so a paged pool of ~10^5 small pages costs a few dozen generator calls, not one per
    page.  A tensor of at most 2^26 values is drawn in a single call."""
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    per_row = max(1, flat.shape[1])
    rows_per_slab = max(1, _SLAB_VALUES // per_row)
    for i in range(0, shape[0], rows_per_slab):
        j = min(shape[0], i + rows_per_slab)
        slab = torch.randn((j - i) * flat.shape[1], generator=gen, device=device, dtype=torch.float32)
        flat[i:j] = slab.view(j - i, flat.shape[1]).to(torch.bfloat16)
        del slab
    return out


def _lowrank_keys(shape, rank: int, gen: torch.Generator, device) -> torch.Tensor:
    """Keys with a per-position random low-rank component: for each (request, KV head) a fixed
    A (d x rank, entries N(0, 1/rank)), and per position K_n = z_n + sigma_n * A g_n with
    z_n ~ N(0, I_d), g_n ~ N(0, I_rank), sigma_n = exp(N(0, 1)).  The log-normal scale makes the
    q.K scores heavy-tailed."""
    B, H, N, d = shape
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=device)
    for b in range(B):
        for h in range(H):
            a = torch.randn(d, rank, generator=gen, device=device) / math.sqrt(rank)
            z = torch.randn(N, d, generator=gen, device=device)
            g = torch.randn(N, rank, generator=gen, device=device)
            sigma = torch.exp(torch.randn(N, 1, generator=gen, device=device))
            out[b, h] = (z + sigma * (g @ a.T)).to(torch.bfloat16)
    return out


def make_workload(
    *,
    name: str = "custom",
    batch: int,
    q_len: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    seq_lens: Sequence[int],
    k: "int | Sequence[int] | float",
    layout: str = "contiguous",
    page_size: int = 16,
    max_len: Optional[int] = None,
    structure: str = "plain",
    needles_per_head: int = 0,
    seed: int = 0,
    device="cpu",
) -> Workload:
    """Draw a decode-step workload.

    k: an int (same k for every request), a per-request sequence, or a float fraction f giving
       k_b = floor(f * L_b).
    structure: "plain" (K, V ~ N(0,1)), "lowrank" (heavy-tailed keys, see `_lowrank_keys`).
    needles_per_head: planted keys per (request, query head); needle j of head hq targets query
       token j % T and is set to 3 * q[b, t, hq] / |q[b, t, hq]| (rounded to bf16) at a position
       drawn uniformly without replacement among the request's L_b positions, distinct within a
       KV head.
    """
    device = torch.device(device)
    B, T, Hq, Hkv, d = batch, q_len, num_q_heads, num_kv_heads, head_dim
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    lens = [int(x) for x in seq_lens]
    if len(lens) != B:
        raise ValueError("seq_lens must have one entry per request")
    if max_len is None:
        max_len = max(lens)
    if max(lens) > max_len or min(lens) < T:
        raise ValueError("need q_len <= L_b <= max_len")
    if isinstance(k, float):
        ks = [int(math.floor(k * L)) for L in lens]
    elif isinstance(k, int):
        ks = [k] * B
    else:
        ks = [int(x) for x in k]
    k_max = max(1, max(ks))

    g_q = _generator(seed, "q", device)
    q = _normal_bf16((B, T, Hq, d), g_q, device)

    if layout == "contiguous":
        kshape = (B, Hkv, max_len, d)
        page_table = None
        num_pages = 0
        psz = 0
    elif layout == "paged":
        if page_size < 1 or page_size & (page_size - 1):
            raise ValueError("page_size must be a power of two")
        psz = page_size
        pages = [-(-L // psz) for L in lens]
        num_pages = sum(pages)
        max_pages = -(-max_len // psz)
        perm = torch.randperm(num_pages, generator=_generator(seed, "pages", device), device=device)
        page_table = torch.zeros((B, max_pages), dtype=torch.int32, device=device)
        off = 0
        for b in range(B):
            page_table[b, : pages[b]] = perm[off : off + pages[b]].to(torch.int32)
            off += pages[b]
        kshape = (num_pages, Hkv, psz, d)
    else:
        raise ValueError(f"unknown layout {layout!r}")

    g_k = _generator(seed, "k", device)
    if structure == "plain":
        k_cache = _normal_bf16(kshape, g_k, device)
    elif structure == "lowrank":
        if layout != "contiguous":
            raise ValueError("lowrank keys are drawn for contiguous caches")
        k_cache = _lowrank_keys(kshape, 8, g_k, device)
    else:
        raise ValueError(f"unknown structure {structure!r}")
    v_cache = _normal_bf16(kshape, _generator(seed, "v", device), device)

    needle_rows = []
    if needles_per_head > 0:
        G = Hq // Hkv
        g_n = _generator(seed, "needles", device)
        for b in range(B):
            L = lens[b]
            count = G * needles_per_head
            if count > L:
                raise ValueError("more needles than positions")
            for h in range(Hkv):
                pos = torch.randperm(L, generator=g_n, device=device)[:count].tolist()
                for gi in range(G):
                    for j in range(needles_per_head):
                        needle_rows.append((b, j % T, h * G + gi, pos[gi * needles_per_head + j]))
    needles = torch.tensor(needle_rows, dtype=torch.int64).reshape(-1, 4)
    if needles.shape[0]:
        qf = q.float()
        unit = qf / torch.linalg.vector_norm(qf, dim=-1, keepdim=True)
        keys = (3.0 * unit).to(torch.bfloat16)  # [B, T, Hq, d]
        nb, nt, nh, npos = (needles[:, i].to(device) for i in range(4))
        nkv = torch.div(nh, Hq // Hkv, rounding_mode="floor")
        if layout == "contiguous":
            k_cache[nb, nkv, npos] = keys[nb, nt, nh]
        else:
            page = page_table[nb, torch.div(npos, psz, rounding_mode="floor")].to(torch.int64)
            k_cache[page, nkv, npos % psz] = keys[nb, nt, nh]
    needles = needles.to(device)

    return Workload(
        name=name,
        batch=B,
        q_len=T,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=d,
        layout=layout,
        max_len=int(max_len),
        page_size=psz,
        num_pages=num_pages,
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        k_per_req=torch.tensor(ks, dtype=torch.int32, device=device),
        k_max=k_max,
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        page_table=page_table,
        needles=needles,
        seed=seed,
        structure=structure,
    )


# Named decode settings.  The seed of each is 1000 + its position in this list (1-based).
NAMED = {
    # Tiny decode step: one request, 4 query heads on one KV head, d=64, N=1024, k=32,
    # one needle per query head.
    "tiny_d64_n1024": dict(
        batch=1, q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64, seq_lens=[1024], k=32,
        structure="plain", needles_per_head=1, seed=1001,
    ),
    # Llama-3-8B-shaped decode: 8 requests, GQA 32/8, d=128, N=32768, k=655 (50x sparsity),
    # 16 needles per query head.
    "llama3_8b_n32k_k655": dict(
        batch=8, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=[32768] * 8,
        k=655, structure="plain", needles_per_head=16, seed=1002,
    ),
    # Qwen2.5-72B-shaped decode, one GPU's full head set: 4 requests, GQA 64/8, d=128,
    # N=131072, k=2621 (50x), heavy-tailed low-rank keys.
    "qwen25_72b_n128k_k2621": dict(
        batch=4, q_len=1, num_q_heads=64, num_kv_heads=8, head_dim=128, seq_lens=[131072] * 4,
        k=2621, structure="lowrank", needles_per_head=0, seed=1003,
    ),
    # Sparsity sweep at fixed shape: 16 requests, GQA 32/8, d=128, N=131072; k is one of
    # N/2, N/5, N/10, N/20, N/50, N/100, N/500, N/1000 (default N/50).
    "sweep_b16_n128k": dict(
        batch=16, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=[131072] * 16,
        k=2621, structure="plain", needles_per_head=0, seed=1004,
    ),
    # The same sweep at a large batch: 64 requests (34 GB of K and V), default k = N/500.
    "sweep_b64_n128k": dict(
        batch=64, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=[131072] * 64,
        k=262, structure="plain", needles_per_head=0, seed=1006,
    ),
    # Agentic ragged paged batch: 32 requests, L_b uniform in [8192, 131072], 4 query tokens,
    # GQA 32/8, d=128, page size 16 with a permuted page table, k_b = floor(0.02 * L_b),
    # 16 needles per query head.
    "ragged_paged_b32_t4": dict(
        batch=32, q_len=4, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=None,
        k=0.02, layout="paged", page_size=16, max_len=131072, structure="plain",
        needles_per_head=16, seed=1005,
    ),
}

SWEEP_K = {"s2": 65536, "s5": 26214, "s10": 13107, "s20": 6553, "s50": 2621, "s100": 1310, "s500": 262,
           "s1000": 131}


def make_named(name: str, device="cpu", **overrides) -> Workload:
    """Draw one of the named decode settings (see `NAMED`); `overrides` replace entries."""
    spec = dict(NAMED[name])
    spec.update(overrides)
    if spec.get("seq_lens") is None:
        # ragged lengths: uniform integers in [8192, 131072]
        g = _generator(spec["seed"], "lens", "cpu")
        spec["seq_lens"] = torch.randint(8192, 131073, (spec["batch"],), generator=g).tolist()
    return make_workload(name=name, device=device, **spec)


def random_index_sets(wl: Workload, k: Optional[int] = None, seed: int = 0) -> torch.Tensor:
    """Uniform random index sets drawn without replacement: for each row (b, t, hq) pick
    min(k_b, visible_t) distinct positions in [0, L_b - T + t]; pad with -1 to k_max.
    Returns int32 [B, T, Hq, k_max] on the workload's device."""
    dev = wl.q.device
    B, T, Hq = wl.batch, wl.q_len, wl.num_q_heads
    kmax = wl.k_max if k is None else int(k)
    out = torch.full((B, T, Hq, kmax), -1, dtype=torch.int32, device=dev)
    g = _generator(seed, "random_sets", dev)
    lens = wl.seq_lens.to("cpu").tolist()
    kreq = wl.k_per_req.to("cpu").tolist() if k is None else [kmax] * B
    for b in range(B):
        L = lens[b]
        for t in range(T):
            vis = L - T + t + 1
            kk = min(kreq[b], vis)
            if kk <= 0:
                continue
            r = torch.rand((Hq, vis), generator=g, device=dev)
            sel = torch.topk(r, kk, dim=1).indices.to(torch.int32)
            out[b, t, :, :kk] = sel
    return out
