"""CPU checks of bench.py's accounting: algorithmic bytes, re-rank row counts and recall."""

import torch

import bench
from workloads import make_workload


def _wl():
    return make_workload(batch=2, q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                         seq_lens=[100, 10], k=[8, 20], max_len=128, seed=3)


def test_rerank_rows_counts_min_of_mk_and_visible():
    wl = _wl()
    # request 0: k' = 8 for both tokens (visible 99, 100); request 1: k' = min(20, 9) = 9, then 10
    want_m2 = 4 * (min(16, 99) + min(16, 100)) + 4 * (min(18, 9) + min(20, 10))
    assert bench.rerank_rows(wl, 2) == want_m2
    want_m1 = 4 * (8 + 8) + 4 * (9 + 10)
    assert bench.rerank_rows(wl, 1) == want_m1


def test_recall():
    a = torch.tensor([[[[0, 1, 2, -1]]]], dtype=torch.int32)
    b = torch.tensor([[[[1, 2, 3, -1]]]], dtype=torch.int32)
    assert abs(bench.recall(a, b, 8) - 2 / 3) < 1e-12
    assert bench.recall(b, b, 8) == 1.0
    empty = torch.full((1, 1, 1, 4), -1, dtype=torch.int32)
    assert bench.recall(a, empty, 8) == 1.0


def test_algorithmic_bytes_distinct_rows():
    wl = _wl()
    B, T, Hq, d = 2, 2, 4, 64
    # every query row selects positions 0..3: per (request, KV head) 4 distinct rows
    idx = torch.full((B, T, Hq, 20), -1, dtype=torch.int32)
    idx[..., :4] = torch.arange(4, dtype=torch.int32)
    ab = bench.algorithmic_bytes(wl, idx, 2)
    assert ab["distinct_rows"] == B * 2 * 4
    assert ab["selected_rows"] == B * T * Hq * 4
    rows = B * T * Hq
    q_bytes, o_bytes = rows * d * 2, rows * d * 4 + rows * 4
    assert ab["sparse"] == 2 * ab["distinct_rows"] * d * 2 + idx.numel() * 4 + q_bytes + o_bytes
    tokens = 110
    assert ab["dense"] == 2 * tokens * 2 * d * 2 + q_bytes + o_bytes
    assert ab["sketch_topk"] == tokens * 2 * (d + 4) + bench.rerank_rows(wl, 2) * d * 2 + idx.numel() * 4 + q_bytes


def test_percentiles_linear_interpolation():
    # p10/p50/p90 of 0..10 are 1, 5, 9; of a constant list the constant
    assert bench.percentiles(list(range(11))) == [1.0, 5.0, 9.0]
    assert bench.percentiles([3.5] * 4) == [3.5, 3.5, 3.5]


def test_cpu_model_is_text_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_profile_harness_groups_and_names_calls():
    import bench_profile as bp

    def row(name, t):
        return {"Kernel_Name": name, "Start_Timestamp": str(t), "End_Timestamp": str(t + 1000)}

    flush = "void at::native::reduce_kernel<512, 1>(...)"
    seq = ["void cs::key_sketch_kernel<128, false>(...)",  # the full build before the steps
           flush, "void cs::sample_tau_kernel<128, false, false>(...)", "void cs::score_cand_kernel<128, false, 1, false>(...)",
           "void cs::cand_select_kernel<128, false, false, 3>(...)",
           flush, "void cs::sparse_partial_kernel<128, false, 16, 8>(...)",
           flush, "void cs::dense_partial_kernel<128, false, 4>(...)", "cs::combine_kernel(...)",
           flush, "void cs::sample_tau_kernel<128, false, false>(...)", "void cs::score_cand_kernel<128, false, 1, false>(...)",
           "void cs::cand_select_kernel<128, false, true, 3>(...)",
           flush, "void cs::score_hist_kernel<128, false, false>(...)", "void cs::select_kernel(...)",
           "void cs::attend_scores_kernel<128, false>(...)",
           flush, "void cs::key_sketch_kernel<128, false>(...)",
           flush, "void cs::sample_tau_kernel<128, false, true>(...)", "void cs::score_cand_kernel<128, false, 1, true>(...)",
           "void cs::sketch_select_kernel<128, false, false, 3>(...)",
           flush, "void cs::sketch_select_kernel<128, false, true, 3>(...)",
           flush, "void cs::key_sketch_kernel<128, false>(...)"]  # the timed full build after the steps
    rows = [row(n, 10000 * i) for i, n in enumerate(seq)]
    segs = bp.segments(rows, lambda r: 1.0)
    assert [e for e, _ in segs] == ["key_sketch_build", "topk_index", "sparse_decode_attn", "dense_decode_attn",
                                    "sparse_decode_step", "sparse_decode_step", "key_sketch_update",
                                    "topk_index_sketch", "sparse_decode_step_sketch", "key_sketch_build"]
    assert segs[1][1] == {"cs::sample_tau_kernel<128, false, false>": 1.0,
                          "cs::score_cand_kernel<128, false, 1, false>": 1.0,
                          "cs::cand_select_kernel<128, false, false, 3>": 1.0}


def test_profile_counter_parsing_groups_calls_and_counters(tmp_path):
    """bench_profile's counter parser: one row per (dispatch, counter), calls separated by the
    flush kernels, the calibration copy picked out, every counter kept apart."""
    import csv

    import bench_profile as bp

    rows = []
    disp = [
        (1, "void at::native::reduce_kernel<512, 1>(...)", 10),
        (2, "void cs::sparse_partial_kernel<128, true, 16, 8>(...)", 20),
        (3, "void at::native::reduce_kernel<512, 1>(...)", 30),
        (4, "void cs::score_cand_kernel<128, true, 4, false, false>(...)", 40),
        (5, "void cs::cand_select_kernel<128, true, false, 3>(...)", 50),
        (6, "void at::native::reduce_kernel<512, 1>(...)", 60),
        (7, "__amd_rocclr_copyBuffer", 70),
    ]
    vals = {"TCC_HIT_sum": {2: 30.0, 4: 5.0, 5: 7.0, 7: 2e6}, "TCC_MISS_sum": {2: 70.0, 4: 95.0, 5: 3.0, 7: 1e6}}
    for did, name, ts in disp:
        for cname, per in vals.items():
            rows.append({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": cname,
                         "Counter_Value": per.get(did, 1.0), "Start_Timestamp": ts, "End_Timestamp": ts + 1})
    d = tmp_path / "l2"
    d.mkdir()
    with open(d / "l2_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)
    per_call, per_kernel, calib = bp.counters(str(d), ["TCC_HIT_sum", "TCC_MISS_sum"])
    assert per_call["TCC_HIT_sum"]["sparse_decode_attn"] == 30.0
    assert per_call["TCC_MISS_sum"]["topk_index"] == 98.0
    assert per_kernel["TCC_HIT_sum"]["topk_index"]["cs::cand_select_kernel<128, true, false, 3>"] == 7.0
    assert calib == {"TCC_HIT_sum": 2e6, "TCC_MISS_sum": 1e6}
