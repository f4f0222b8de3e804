#!/usr/bin/env python3
"""Benchmark: one oracle-top-k sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload ragged_paged_b32_t4]

The default workload is the largest single-GPU setting: the agentic ragged paged batch (32
requests, cached lengths uniform in [8192, 131072], 4 new tokens each, GQA 32/8, d = 128, pages of
16 positions in a permuted page table, k_b = 2% of L_b per token and head).

A step is one pass of the whole hot path over one decode batch, on one stream:
    flush -> topk_index -> flush -> sparse_decode_attn -> flush -> dense_decode_attn
          -> flush -> sparse_decode_step (indexer + sparse attention in one call)
          -> flush -> topk_index_sketch -> flush -> sparse_decode_step_sketch
The last two run the reduced-byte indexer (int8 key sketch, cand_mult * k candidates re-ranked
on exact scores) on a sketch built before the timed region; the per-step sketch update of the
T new positions per request (key_sketch_build with last_n = T) is timed as its own call.
`flush` reads a 2 GiB scratch buffer so that neither L2 nor the 256 MB Infinity Cache holds any
KV bytes when a hot-path call starts (every call is measured from cold caches).  Each call is
bracketed by HIP events recorded on the stream it runs on.  Inputs are seeded synthetic tensors
drawn on the GPU before the timed region.

Prints ONE JSON line.  `ms_per_step` is one pass of the hot path on the batch: the mean event
times of topk_index + sparse_decode_attn + dense_decode_attn (the indexer, the sparse attention
and the dense baseline; flushes and the other calls excluded; the wall time of a whole timed
iteration is `wall_ms_per_iteration`).  `value` is the sparse decode attention's gathered-KV
throughput: the
distinct K/V rows the step's index lists name (counted once per (request, KV head) group, 512 B
each at d=128) plus index, query and output bytes, divided by the mean duration of the
sparse_decode_attn call.  Also reported: µs of every call (mean, and p10/p50/p90), speedup over
the dense decode on the same inputs, a roofline object per kernel and the CPU oracle timed on the
host cores; beside the timed steps, the sparse call on uniform random index sets of the same
sizes (cold) and warm-cache timings of the main calls.  `per_config` then repeats the indexer, the
sparse attention, the one-call step and the dense baseline (fewer steps, same flush discipline) on
the other decode settings: the tiny case, the Llama-3-8B- and Qwen2.5-72B-shaped batches at 50x,
and the 16-request sweep at 10x/50x/100x/1000x sparsity (oracle top-k lists, plus uniform random
sets of the same sizes for the sparse call), with the reduced-byte indexer's one-call step at
cand_mult 1 and 2 (each with the per-step sketch update) and the recall of its cand_mult-1 lists.
Call durations come from HIP events created with hipEventDisableSystemFence; an event pair
around one call still counts about 4 µs of dispatch latency on top of the kernels' run time.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode µs/step + gathered-KV GB/s (% HBM peak), speedup vs dense at 50×"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "ragged_paged_b32_t4"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the launch planning (splits, chunks, kernel variants) decides the traffic as much as the kernels
_CS = "long_context_sparse_oracle_amd/csrc/"
_LAUNCH_SOURCES = [_CS + "api.hip", _CS + "launch.h"]
KERNEL_SOURCES = {
    "sparse_decode_attn": [_CS + "attention.hip", _CS + "device_common.h", *_LAUNCH_SOURCES],
    "dense_decode_attn": [_CS + "attention.hip", _CS + "device_common.h", *_LAUNCH_SOURCES],
    "topk_index": [_CS + "topk.hip", _CS + "device_common.h", *_LAUNCH_SOURCES],
    "sparse_decode_step": [_CS + "topk.hip", _CS + "attention.hip", _CS + "device_common.h", *_LAUNCH_SOURCES],
    "topk_index_sketch": [_CS + "topk.hip", _CS + "sketch.hip", _CS + "device_common.h", *_LAUNCH_SOURCES],
    "sparse_decode_step_sketch": [_CS + "topk.hip", _CS + "sketch.hip", _CS + "device_common.h",
                                  *_LAUNCH_SOURCES],
}


def source_hash(name: str) -> str:
    """Hash of the code (comments and blank space removed) of the sources behind an entry point:
    traffic figures recorded for another hash are stale."""
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--sweep-k", default=None, help="k for a sweep workload (s2/s5/s10/s20/s50/s100/s500/s1000)")
    p.add_argument("--cand-mult", type=int, default=2,
                   help="candidates per selected position of the reduced-byte indexer")
    p.add_argument("--sparse-splits", type=int, default=0)
    p.add_argument("--dense-splits", type=int, default=0)
    p.add_argument("--no-flush", action="store_true", help="warm caches (not the reported figure)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the random-set and warm-cache timings after the steps (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the CPU oracle leg (0 disables it)")
    p.add_argument("--no-per-config", action="store_true",
                   help="skip the other decode settings after the main workload (profiling runs)")
    p.add_argument("--per-config-steps", type=int, default=10)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for counter calibration runs)")
    return p.parse_args()


def algorithmic_bytes(wl, idx, cand_mult):
    """Bytes the method must move per call (d-dim bf16 rows, int32 indices, fp32 outputs)."""
    import torch

    B, T, Hq, Hkv, d = wl.batch, wl.q_len, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    G = Hq // Hkv
    rows = B * T * Hq
    row_bytes = d * 2
    q_bytes = rows * d * 2
    o_bytes = rows * d * 4 + rows * 4
    tokens = int(wl.seq_lens.to(torch.int64).sum())
    # distinct selected rows per (request, KV head) group
    grp = idx.view(B, T, Hkv, G, -1).permute(0, 2, 1, 3, 4).reshape(B * Hkv, -1).long()
    mark = torch.zeros((B * Hkv, wl.max_len + 1), dtype=torch.bool, device=idx.device)
    mark.scatter_(1, torch.where(grp < 0, wl.max_len, grp), True)
    distinct = int(mark[:, : wl.max_len].sum())
    nominal = int((idx >= 0).sum())
    index_bytes = idx.numel() * 4
    return {
        "sparse": 2 * distinct * row_bytes + index_bytes + q_bytes + o_bytes,
        "sparse_nominal": 2 * nominal * row_bytes + index_bytes + q_bytes + o_bytes,
        "distinct_rows": distinct,
        "selected_rows": nominal,
        "dense": 2 * tokens * Hkv * row_bytes + q_bytes + o_bytes,
        "topk": tokens * Hkv * row_bytes + index_bytes + q_bytes,
        # the one-call step: all of K once (scores), V of the distinct selected rows, q, outputs
        "step": tokens * Hkv * row_bytes + distinct * row_bytes + q_bytes + o_bytes,
        # reduced-byte indexer: every position's codes and scale once per KV head, then each row's
        # min(cand_mult * k', visible) candidate K rows for the exact re-rank
        "sketch_topk": tokens * Hkv * (d + 4) + rerank_rows(wl, cand_mult) * row_bytes + index_bytes + q_bytes,
        "sketch_step": tokens * Hkv * (d + 4) + rerank_rows(wl, cand_mult) * row_bytes + distinct * row_bytes
                       + q_bytes + o_bytes,
        "rerank_rows": rerank_rows(wl, cand_mult),
    }


def rerank_rows(wl, cand_mult):
    """K rows the re-rank of the reduced-byte indexer reads: min(cand_mult * k', visible) per row."""
    total = 0
    lens = wl.seq_lens.tolist()
    kreq = wl.k_per_req.tolist()
    for b in range(wl.batch):
        for t in range(wl.q_len):
            vis = max(0, lens[b] - wl.q_len + t + 1)
            kk = min(min(kreq[b], wl.k_max), vis)
            total += min(cand_mult * kk, vis) * wl.num_q_heads
    return total


def recall(idx_a, idx_b, max_len):
    """Fraction of idx_b's entries (>= 0) that idx_a's row also holds."""
    import torch

    rows = idx_a.shape[0] * idx_a.shape[1] * idx_a.shape[2]
    a = idx_a.reshape(rows, -1).long()
    bb = idx_b.reshape(rows, -1).long()
    hit = 0
    for r0 in range(0, rows, 256):
        ma = torch.zeros((min(256, rows - r0), max_len + 1), dtype=torch.bool, device=a.device)
        ma.scatter_(1, torch.where(a[r0:r0 + 256] < 0, max_len, a[r0:r0 + 256]), True)
        ma[:, max_len] = False
        vb = bb[r0:r0 + 256]
        hit += int(torch.gather(ma, 1, torch.where(vb < 0, max_len, vb)).sum())
    total = int((bb >= 0).sum())
    return hit / total if total else 1.0


def mean_of(values):
    return statistics.fmean(values)


def percentiles(values):
    """p10, p50, p90 of a list of timings (linear interpolation between order statistics)."""
    import numpy as np

    return [round(float(x), 2) for x in np.percentile(np.asarray(values, dtype=np.float64), [10, 50, 90])]


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def cpu_baseline(wl, gathered_bytes, seconds):
    """The CPU oracle (top-k + sparse attention per row) timed on the host on a bounded sample
    of the same workload, scaled to the full step."""
    import numpy as np
    import torch

    import oracle  # CPU oracle: benchmark baseline leg only

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    B, T, Hq, Hkv = wl.batch, wl.q_len, wl.num_q_heads, wl.num_kv_heads
    G = Hq // Hkv
    groups = [(b, h) for b in range(B) for h in range(Hkv)]
    order = np.random.default_rng(7).permutation(len(groups))
    qb = wl.q.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    q = oracle.bf16_bits_to_f64(qb)
    kreq = wl.k_per_req.cpu().numpy()
    lens = wl.seq_lens.cpu().numpy()
    done_rows = 0
    elapsed = 0.0
    n_groups = 0
    for gi in order:
        b, h = groups[gi]
        L = int(lens[b])
        if wl.layout == "contiguous":
            kb = wl.k_cache[b, h, :L].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            vb = wl.v_cache[b, h, :L].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        else:
            n = torch.arange(L, device=wl.page_table.device)
            pages = wl.page_table[b, n // wl.page_size].long()
            kb = wl.k_cache[pages, h, n % wl.page_size].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            vb = wl.v_cache[pages, h, n % wl.page_size].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        K = oracle.bf16_bits_to_f64(kb)
        V = oracle.bf16_bits_to_f64(vb)
        for t in range(T):
            vis = oracle.visible_length(L, T, t)
            for g in range(G):
                hq = h * G + g
                sel = oracle.row_topk(q[b, t, hq], K, vis, int(kreq[b]))
                oracle.row_sparse(q[b, t, hq], K, V, sel, vis)
                done_rows += 1
        elapsed += time.perf_counter() - t0
        n_groups += 1
        if elapsed >= seconds:
            break
    rows = B * T * Hq
    step_s = elapsed / done_rows * rows
    return {
        "value": round(gathered_bytes / step_s / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "us_per_step": round(step_s * 1e6, 1),
        "sample": (
            f"{done_rows} of {rows} rows ({n_groups} of {len(groups)} (request, KV head) groups): "
            f"float64 NumPy oracle top-k + sparse attention per row, {elapsed:.1f} s, scaled "
            f"linearly to the full step" if done_rows < rows else
            f"all {rows} rows: float64 NumPy oracle top-k + sparse attention, {elapsed:.1f} s"
        ),
    }


# The other decode settings, each timed with the same flush discipline after the main workload:
# (label, named workload, sweep level or None).  The sweep's K and V do not depend on k, so its
# four sparsity levels share one draw.
PER_CONFIG = [
    ("tiny_d64_n1024", "tiny_d64_n1024", None),
    ("llama3_8b_n32k_k655", "llama3_8b_n32k_k655", None),
    ("qwen25_72b_n128k_k2621", "qwen25_72b_n128k_k2621", None),
    ("sweep_b16_n128k_s10", "sweep_b16_n128k", "s10"),
    ("sweep_b16_n128k_s50", "sweep_b16_n128k", "s50"),
    ("sweep_b16_n128k_s100", "sweep_b16_n128k", "s100"),
    ("sweep_b16_n128k_s1000", "sweep_b16_n128k", "s1000"),
]


def time_calls(calls, steps, warmup, flush, hev, sh):
    """Mean µs of every call over `steps` iterations (after `warmup` untimed ones), each call
    after a flush and between fence-free events on stream handle `sh`."""
    import torch

    for _ in range(warmup):
        for fn in calls.values():
            flush()
            fn()
    torch.cuda.synchronize()
    evs = []
    gc.collect()
    gc.disable()
    for _ in range(steps):
        for name, fn in calls.items():
            e0, e1 = hev.create(), hev.create()
            flush()
            hev.record(e0, sh)
            fn()
            hev.record(e1, sh)
            evs.append((name, e0, e1))
    torch.cuda.synchronize()
    gc.enable()
    times = {k: [] for k in calls}
    for name, e0, e1 in evs:
        times[name].append(hev.elapsed_us(e0, e1))
        hev.destroy(e0)
        hev.destroy(e1)
    return {k: statistics.fmean(v) for k, v in times.items()}


def per_config_results(args, flush, hev, sh):
    """Indexer, sparse attention (oracle lists, and uniform random sets of the same sizes), the
    one-call step and the dense baseline on every other decode setting."""
    import dataclasses

    import torch

    import long_context_sparse_oracle_amd as cs
    from workloads import make_named, random_index_sets
    from workloads.synth import SWEEP_K

    dev = torch.device("cuda", 0)
    out = {}
    drawn = {}
    sketches = {}
    for label, name, level in PER_CONFIG:
        if label == args.workload or (level and f"{name}_{level}" == f"{args.workload}_{args.sweep_k}"):
            continue
        print(f"[bench] per-config {label}", file=sys.stderr, flush=True)
        if name not in drawn:
            drawn.clear()
            sketches.clear()
            torch.cuda.empty_cache()
            drawn[name] = make_named(name, device=dev)
        wl = drawn[name]
        if level:
            k = SWEEP_K[level]
            wl = dataclasses.replace(wl, k_per_req=torch.full_like(wl.k_per_req, k), k_max=k)
        cache = cs.KVCache(wl.k_cache, wl.v_cache, wl.seq_lens, page_table=wl.page_table, max_len=wl.max_len)
        B, T, Hq, d, k_max, kptr = wl.batch, wl.q_len, wl.num_q_heads, wl.head_dim, wl.k_max, wl.k_per_req
        indices = torch.empty((B, T, Hq, k_max), dtype=torch.int32, device=dev)
        o = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
        ws_t = torch.empty(max(1, cs.topk_index_workspace_size(wl.q, cache, k_max)), dtype=torch.uint8, device=dev)
        ws_s = torch.empty(max(1, cs.sparse_decode_attn_workspace_size(wl.q, cache, k_max)), dtype=torch.uint8,
                           device=dev)
        ws_d = torch.empty(max(1, cs.dense_decode_attn_workspace_size(wl.q, cache)), dtype=torch.uint8, device=dev)
        ws_st = torch.empty(max(1, cs.sparse_decode_step_workspace_size(wl.q, cache, k_max)), dtype=torch.uint8,
                            device=dev)
        idx_rand = random_index_sets(wl)
        calls = {
            "topk_index": lambda: cs.topk_index(wl.q, cache, kptr, k_max=k_max, indices=indices, workspace=ws_t),
            "sparse_decode_attn": lambda: cs.sparse_decode_attn(wl.q, cache, indices, out=o, lse=lse,
                                                                workspace=ws_s),
            "sparse_random_sets": lambda: cs.sparse_decode_attn(wl.q, cache, idx_rand, out=o, lse=lse,
                                                                workspace=ws_s),
            "sparse_decode_step": lambda: cs.sparse_decode_step(wl.q, cache, kptr, k_max=k_max, out=o, lse=lse,
                                                                workspace=ws_st),
            "dense_decode_attn": lambda: cs.dense_decode_attn(wl.q, cache, out=o, lse=lse, workspace=ws_d),
        }
        mean = time_calls(calls, args.per_config_steps, 3, flush, hev, sh)
        # the reduced-byte indexer's step at cand_mult 1 and 2, with the per-step sketch update
        if name not in sketches:
            sketches.clear()
            sketches[name] = cs.key_sketch_build(cache)
        sk = sketches[name]
        idx_m1 = torch.empty_like(indices)
        ws_k1 = torch.empty(max(1, cs.topk_index_sketch_workspace_size(wl.q, cache, k_max, 1)), dtype=torch.uint8,
                            device=dev)
        ws_s1 = torch.empty(max(1, cs.sparse_decode_step_sketch_workspace_size(wl.q, cache, k_max, 1)),
                            dtype=torch.uint8, device=dev)
        ws_s2 = torch.empty(max(1, cs.sparse_decode_step_sketch_workspace_size(wl.q, cache, k_max, 2)),
                            dtype=torch.uint8, device=dev)
        sk_calls = {
            "update": lambda: cs.key_sketch_build(cache, sk, last_n=wl.q_len),
            "step_m1": lambda: cs.sparse_decode_step_sketch(wl.q, cache, sk, kptr, k_max=k_max, cand_mult=1, out=o,
                                                            lse=lse, workspace=ws_s1),
            "step_m2": lambda: cs.sparse_decode_step_sketch(wl.q, cache, sk, kptr, k_max=k_max, cand_mult=2, out=o,
                                                            lse=lse, workspace=ws_s2),
        }
        skm = time_calls(sk_calls, args.per_config_steps, 2, flush, hev, sh)
        cs.topk_index_sketch(wl.q, cache, sk, kptr, k_max=k_max, cand_mult=1, indices=idx_m1, workspace=ws_k1)
        torch.cuda.synchronize()
        rec_m1 = recall(idx_m1, indices, wl.max_len)
        del idx_m1, ws_k1, ws_s1, ws_s2, sk_calls
        ab = algorithmic_bytes(wl, indices, args.cand_mult)
        ab_r = algorithmic_bytes(wl, idx_rand, args.cand_mult)
        frac = lambda nbytes, us: round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)  # noqa: E731
        dense = mean["dense_decode_attn"]
        out[label] = {
            "k": k_max,
            "sparsity": round(wl.max_len / k_max, 1),
            "sparse_us": round(mean["sparse_decode_attn"], 2),
            "sparse_frac": frac(ab["sparse"], mean["sparse_decode_attn"]),
            "sparse_random_sets_us": round(mean["sparse_random_sets"], 2),
            "sparse_random_sets_frac": frac(ab_r["sparse"], mean["sparse_random_sets"]),
            "topk_us": round(mean["topk_index"], 2),
            "topk_frac": frac(ab["topk"], mean["topk_index"]),
            "step_us": round(mean["sparse_decode_step"], 2),
            "dense_us": round(dense, 2),
            "dense_frac": frac(ab["dense"], dense),
            "speedup_vs_dense": round(dense / mean["sparse_decode_attn"], 3),
            "random_sets_speedup_vs_dense": round(dense / mean["sparse_random_sets"], 3),
            "topk_plus_sparse_vs_dense": round(dense / (mean["topk_index"] + mean["sparse_decode_attn"]), 3),
            "step_vs_dense": round(dense / mean["sparse_decode_step"], 3),
            "sketch_update_us": round(skm["update"], 2),
            "sketch_m1_step_us": round(skm["step_m1"], 2),
            "sketch_m1_step_vs_dense": round(dense / (skm["step_m1"] + skm["update"]), 3),
            "sketch_m1_recall": round(rec_m1, 5),
            "sketch_m2_step_us": round(skm["step_m2"], 2),
            "sketch_m2_step_vs_dense": round(dense / (skm["step_m2"] + skm["update"]), 3),
            "gathered_bytes": ab["sparse"],
        }
        del calls, indices, o, lse, ws_t, ws_s, ws_d, ws_st, idx_rand, cache, wl
    drawn.clear()
    sketches.clear()
    torch.cuda.empty_cache()
    return out


class HipEvents:
    """HIP events created with hipEventDisableSystemFence: recording them skips the system-scope
    cache writeback/invalidate that default events perform, which would otherwise add about
    1.6 µs of idle time to every timed call.  Recorded on the stream the library launches on."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch

        path = None
        for cand in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
            try:
                self.hip = ctypes.CDLL(cand)
                path = cand
                break
            except OSError:
                continue
        if path is None:
            raise RuntimeError("libamdhip64 not found")
        self.ct = ctypes
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        torch.cuda.synchronize()

    def create(self):
        e = self.ct.c_void_p()
        st = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        return e

    def record(self, e, stream_handle):
        st = self.hip.hipEventRecord(e, self.ct.c_void_p(stream_handle))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_us(self, e0, e1):
        ms = self.ct.c_float()
        st = self.hip.hipEventElapsedTime(self.ct.byref(ms), e0, e1)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value * 1000.0

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the decode step "
              f"runs on a single device and has no multi-GPU execution path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_sparse_oracle_amd as cs
    from workloads import make_named
    from workloads.synth import SWEEP_K

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    overrides = {}
    if args.workload.startswith("sweep_") and args.sweep_k:
        overrides["k"] = SWEEP_K[args.sweep_k]
    wl = make_named(args.workload, device=dev, **overrides)
    torch.cuda.synchronize()
    cache = cs.KVCache(wl.k_cache, wl.v_cache, wl.seq_lens, page_table=wl.page_table,
                       max_len=wl.max_len)
    B, T, Hq, d = wl.batch, wl.q_len, wl.num_q_heads, wl.head_dim
    k_max = wl.k_max
    kptr = wl.k_per_req

    # buffers allocated once: the timed region allocates nothing
    indices = torch.empty((B, T, Hq, k_max), dtype=torch.int32, device=dev)
    out_s = torch.empty((B, T, Hq, d), dtype=torch.float32, device=dev)
    lse_s = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
    out_d = torch.empty_like(out_s)
    lse_d = torch.empty_like(lse_s)
    ws_t = torch.empty(max(1, cs.topk_index_workspace_size(wl.q, cache, k_max)), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(1, cs.sparse_decode_attn_workspace_size(wl.q, cache, k_max, args.sparse_splits)),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, cs.dense_decode_attn_workspace_size(wl.q, cache, args.dense_splits)),
                       dtype=torch.uint8, device=dev)
    out_st = torch.empty_like(out_s)
    lse_st = torch.empty_like(lse_s)
    ws_st = torch.empty(max(1, cs.sparse_decode_step_workspace_size(wl.q, cache, k_max)), dtype=torch.uint8,
                        device=dev)
    # reduced-byte indexer: the sketch of every cached key, built once (in serving it is kept up to
    # date by sketching each step's new positions, the timed `key_sketch_update` call)
    m = args.cand_mult
    sketch = cs.key_sketch_build(cache)
    idx_sk = torch.empty_like(indices)
    ws_tk = torch.empty(max(1, cs.topk_index_sketch_workspace_size(wl.q, cache, k_max, m)), dtype=torch.uint8,
                        device=dev)
    out_sk = torch.empty_like(out_s)
    lse_sk = torch.empty_like(lse_s)
    ws_sk = torch.empty(max(1, cs.sparse_decode_step_sketch_workspace_size(wl.q, cache, k_max, m)),
                        dtype=torch.uint8, device=dev)
    # cache flush by reading 2 GiB: evicts every KV line from L2 and the Infinity Cache and leaves
    # clean lines behind (a write flush would leave dirty lines whose write-back the next call
    # would pay for)
    flush_buf = None if args.no_flush else torch.ones((2 << 30) // 8, dtype=torch.int64, device=dev)
    flush_out = torch.empty((), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def flush():
        if flush_buf is not None:
            torch.sum(flush_buf, dim=0, out=flush_out)

    calls = {
        "topk_index": lambda: cs.topk_index(wl.q, cache, kptr, k_max=k_max, indices=indices, workspace=ws_t),
        "sparse_decode_attn": lambda: cs.sparse_decode_attn(wl.q, cache, indices, num_splits=args.sparse_splits,
                                                            out=out_s, lse=lse_s, workspace=ws_s),
        "dense_decode_attn": lambda: cs.dense_decode_attn(wl.q, cache, num_splits=args.dense_splits,
                                                          out=out_d, lse=lse_d, workspace=ws_d),
        "sparse_decode_step": lambda: cs.sparse_decode_step(wl.q, cache, kptr, k_max=k_max, out=out_st,
                                                            lse=lse_st, workspace=ws_st),
        "key_sketch_update": lambda: cs.key_sketch_build(cache, sketch, last_n=T),
        "topk_index_sketch": lambda: cs.topk_index_sketch(wl.q, cache, sketch, kptr, k_max=k_max, cand_mult=m,
                                                          indices=idx_sk, workspace=ws_tk),
        "sparse_decode_step_sketch": lambda: cs.sparse_decode_step_sketch(wl.q, cache, sketch, kptr, k_max=k_max,
                                                                          cand_mult=m, out=out_sk, lse=lse_sk,
                                                                          workspace=ws_sk),
    }
    times = {k: [] for k in calls}

    hev = HipEvents()
    sh = stream.cuda_stream
    pool = [(hev.create(), hev.create()) for _ in range(len(calls) * args.steps)]

    def step(record, k=0):
        evs = []
        for j, (name, fn) in enumerate(calls.items()):
            flush()
            if record:
                e0, e1 = pool[k * len(calls) + j]
                hev.record(e0, sh)
                fn()
                hev.record(e1, sh)
                evs.append((name, e0, e1))
            else:
                fn()
        return evs

    print(f"[bench] workload {args.workload}: B{B} T{T} Hq{Hq} Hkv{wl.num_kv_heads} d{d} "
          f"max_len {wl.max_len} k_max {k_max} layout {wl.layout}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    all_evs = []
    torch.cuda.synchronize()
    # no garbage collection while calls are queued: a collector pause between an event record and
    # the launch after it would leave the GPU idle inside the timed window
    gc.collect()
    gc.disable()
    t0 = time.perf_counter()
    for k in range(args.steps):
        all_evs.extend(step(True, k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    for name, e0, e1 in all_evs:
        times[name].append(hev.elapsed_us(e0, e1))
    for e0, e1 in pool:
        hev.destroy(e0)
        hev.destroy(e1)

    ab = algorithmic_bytes(wl, indices, m)
    hev2 = HipEvents()

    def timed(fn, n, cold):
        """Mean µs of n back-to-back calls of fn between fence-free events (each after a flush when
        cold), synchronised once at the end as the timed steps are."""
        evs = [(hev2.create(), hev2.create()) for _ in range(n)]
        for e0, e1 in evs:
            if cold:
                flush()
            hev2.record(e0, sh)
            fn()
            hev2.record(e1, sh)
        torch.cuda.synchronize()
        ts = [hev2.elapsed_us(e0, e1) for e0, e1 in evs]
        for e0, e1 in evs:
            hev2.destroy(e0)
            hev2.destroy(e1)
        return statistics.fmean(ts)

    # the reduced-byte indexer's lists and outputs against the exact ones, before the extras below
    # reuse its buffers
    sk_recall = recall(idx_sk, indices, wl.max_len)
    sk_out_diff = float((out_sk - out_st).abs().max())
    # Beside the timed steps (not part of `value`): the sparse call on uniform random index sets of
    # the same sizes (drawn without replacement), cold; and warm-cache timings of the main calls.
    from workloads import random_index_sets

    random_sets = None
    if not args.no_extras:
        idx_rand = random_index_sets(wl)
        ab_rand = algorithmic_bytes(wl, idx_rand, m)
        rand_us = timed(lambda: cs.sparse_decode_attn(wl.q, cache, idx_rand, num_splits=args.sparse_splits,
                                                      out=out_s, lse=lse_s, workspace=ws_s), max(args.steps, 5), True)
        rand_gbs = ab_rand["sparse"] / (rand_us * 1e-6) / 1e9
        random_sets = {
            "sparse_us": round(rand_us, 2),
            "gathered_bytes": ab_rand["sparse"],
            "gbs": round(rand_gbs, 1),
            "pct_hbm_peak": round(100.0 * rand_gbs / HBM_PEAK_GBS, 2),
            "speedup_vs_dense": round(mean_of(times["dense_decode_attn"]) / rand_us, 3),
        }
    # the reduced-byte indexer without re-rank (cand_mult = 1: the sketch's own top-k), cold
    sketch_m1 = None
    if not args.no_extras:
        idx_m1 = torch.empty_like(indices)
        ws_m1 = torch.empty(max(1, cs.topk_index_sketch_workspace_size(wl.q, cache, k_max, 1)), dtype=torch.uint8,
                            device=dev)
        ws_m1s = torch.empty(max(1, cs.sparse_decode_step_sketch_workspace_size(wl.q, cache, k_max, 1)),
                             dtype=torch.uint8, device=dev)
        n_ex = max(args.steps // 2, 5)
        m1_topk = timed(lambda: cs.topk_index_sketch(wl.q, cache, sketch, kptr, k_max=k_max, cand_mult=1,
                                                     indices=idx_m1, workspace=ws_m1), n_ex, True)
        m1_step = timed(lambda: cs.sparse_decode_step_sketch(wl.q, cache, sketch, kptr, k_max=k_max, cand_mult=1,
                                                             out=out_sk, lse=lse_sk, workspace=ws_m1s), n_ex, True)
        torch.cuda.synchronize()
        sketch_m1 = {"topk_us": round(m1_topk, 2), "step_us": round(m1_step, 2),
                     "recall_vs_exact_topk": round(recall(idx_m1, indices, wl.max_len), 5)}
        del ws_m1, ws_m1s
    warm = None
    if flush_buf is not None and not args.no_extras:
        warm = {}
        for name in ("topk_index", "sparse_decode_attn", "dense_decode_attn", "sparse_decode_step"):
            calls[name]()
            warm[name] = round(timed(calls[name], 5, False), 2)
    # the HBM read rate a plain streaming kernel reaches on this GPU: the flush itself (a sum over
    # 2 GiB read from cold caches), timed after a flush
    read_ceiling = None
    if flush_buf is not None and not args.no_extras:
        fl_us = timed(flush, 5, True)
        gbs = flush_buf.numel() * 8 / (fl_us * 1e-6) / 1e9
        read_ceiling = {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "how": "torch.sum over a 2 GiB int64 buffer from cold caches, HIP events"}
    # one full build of the sketch (every cached key), timed on its own after the steps
    eb0, eb1 = hev2.create(), hev2.create()
    flush()
    hev2.record(eb0, sh)
    cs.key_sketch_build(cache, sketch)
    hev2.record(eb1, sh)
    torch.cuda.synchronize()
    build_us = hev2.elapsed_us(eb0, eb1)
    hev2.destroy(eb0)
    hev2.destroy(eb1)
    mean = {k: statistics.fmean(v) for k, v in times.items()}
    med = {k: statistics.median(v) for k, v in times.items()}
    traffic = load_traffic()

    def roofline(name, bytes_per_launch):
        achieved = bytes_per_launch / (mean[name] * 1e-6) / 1e9
        tag = args.workload + ("_" + args.sweep_k if args.sweep_k else "")
        tr = traffic.get(tag, {}).get(name)
        tr_val = None
        if tr and tr.get("source_sha256") == source_hash(name):
            tr_val = tr.get("bytes_per_launch")
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": tr_val}

    sparse_gbs = ab["sparse"] / (mean["sparse_decode_attn"] * 1e-6) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(sparse_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((mean["topk_index"] + mean["sparse_decode_attn"] + mean["dense_decode_attn"]) / 1e3,
                             4),
        "wall_ms_per_iteration": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "batch": B, "q_len": T, "num_q_heads": Hq, "num_kv_heads": wl.num_kv_heads,
            "head_dim": d, "context": wl.max_len, "k": k_max, "layout": wl.layout,
            "sparsity": round(wl.max_len / k_max, 1) if wl.layout == "contiguous" else 50.0,
            "cold_cache": flush_buf is not None,
        },
        "sparse_us": round(mean["sparse_decode_attn"], 2),
        "sparse_us_median": round(med["sparse_decode_attn"], 2),
        "topk_us": round(mean["topk_index"], 2),
        "dense_us": round(mean["dense_decode_attn"], 2),
        "speedup_vs_dense": round(mean["dense_decode_attn"] / mean["sparse_decode_attn"], 3),
        "e2e_speedup_vs_dense": round(mean["dense_decode_attn"] / (mean["topk_index"] + mean["sparse_decode_attn"]), 3),
        "step_us": round(mean["sparse_decode_step"], 2),
        "step_speedup_vs_dense": round(mean["dense_decode_attn"] / mean["sparse_decode_step"], 3),
        "sketch": {
            "cand_mult": m,
            "topk_us": round(mean["topk_index_sketch"], 2),
            "step_us": round(mean["sparse_decode_step_sketch"], 2),
            "update_us": round(mean["key_sketch_update"], 2),
            "step_speedup_vs_dense": round(mean["dense_decode_attn"] /
                                           (mean["sparse_decode_step_sketch"] + mean["key_sketch_update"]), 3),
            "full_build_us": round(build_us, 2),
            "recall_vs_exact_topk": round(sk_recall, 5),
            "max_abs_out_diff_vs_exact_step": sk_out_diff,
            "rerank_rows": ab["rerank_rows"],
            "m1": None if sketch_m1 is None else dict(
                sketch_m1, step_speedup_vs_dense=round(mean["dense_decode_attn"] /
                                                       (sketch_m1["step_us"] + mean["key_sketch_update"]), 3)),
        },
        "pct_hbm_peak": round(100.0 * sparse_gbs / HBM_PEAK_GBS, 2),
        "percentiles_us": {name: percentiles(v) for name, v in times.items()},
        "random_sets": random_sets,
        "warm_us": warm,
        "hbm_read_ceiling": read_ceiling,
        "kernel_us_per_step": round(sum(mean.values()), 2),
        "gathered_bytes": ab["sparse"],
        "algorithmic_bytes": {"topk_index": ab["topk"], "sparse_decode_attn": ab["sparse"],
                              "dense_decode_attn": ab["dense"], "sparse_decode_step": ab["step"],
                              "topk_index_sketch": ab["sketch_topk"],
                              "sparse_decode_step_sketch": ab["sketch_step"]},
        "distinct_rows": ab["distinct_rows"],
        "selected_rows": ab["selected_rows"],
        "roofline": roofline("sparse_decode_attn", ab["sparse"]),
        "roofline_kernels": {
            "topk_index": roofline("topk_index", ab["topk"]),
            "dense_decode_attn": roofline("dense_decode_attn", ab["dense"]),
            "sparse_decode_step": roofline("sparse_decode_step", ab["step"]),
            "topk_index_sketch": roofline("topk_index_sketch", ab["sketch_topk"]),
            "sparse_decode_step_sketch": roofline("sparse_decode_step_sketch", ab["sketch_step"]),
        },
    }
    if args.cpu_seconds > 0:
        print("[bench] CPU oracle baseline ...", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(wl, ab["sparse"], args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    if not args.no_per_config:
        # free the main workload before drawing the others
        del calls, wl, cache, sketch, indices, out_s, lse_s, out_d, lse_d, ws_t, ws_s, ws_d, out_st, lse_st
        del ws_st, idx_sk, ws_tk, out_sk, lse_sk, ws_sk
        if random_sets is not None:
            del idx_rand
        if sketch_m1 is not None:
            del idx_m1
        torch.cuda.empty_cache()
        rec["per_config"] = per_config_results(args, flush, hev2, sh)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
