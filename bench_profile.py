#!/usr/bin/env python3
"""rocprofv3 harness for bench.py: per-kernel durations of every library call and, with
--counters, the HBM bytes each call moves; writes the summaries under profiles/.

    python bench_profile.py --workload llama3_8b_n32k_k655 [--sweep-k s100] [--counters]

Run from anywhere on a machine with one MI355X (rocprofv3 on PATH).  Steps, each a child process
under its own time limit:
  1. `python3 bench.py --workload W` for the JSON line (HIP-event means of every call);
  2. `rocprofv3 --kernel-trace --stats` over a short bench.py run (5 steps, no extras);
  3. with --counters: one rocprofv3 --pmc run per counter pass (each within the per-block limits
     of one pass), every run with a plain 1 GiB device copy to calibrate the byte counters:
       fetch   FETCH_SIZE                          HBM bytes read (calibrated by the copy)
       write   WRITE_SIZE                          HBM bytes written (calibrated by the copy)
       l2      TCC_HIT_sum, TCC_MISS_sum           L2 hit rate
       lds     SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE   LDS bank-conflict cycles per LDS cycle
       xlat    TCP_UTCL1_TRANSLATION_MISS_sum, TCP_UTCL1_REQUEST_sum, TCC_EA0_RDREQ_DRAM_sum
                                                   address-translation misses, DRAM read requests
       stall   TCC_TAG_STALL_sum, TCP_TCP_TA_DATA_STALL_CYCLES_sum   L2 tag and TA data stalls
Dispatches are grouped into calls by the cache-flush kernels bench.py runs between calls, and a
call is named by the library kernels it ran.  Outputs: profiles/<tag>_kernel_stats.md and, with
--counters, profiles/<tag>_traffic.md plus the per-call bytes in profiles/traffic.json, stored with
a hash of the kernel sources (bench.py reports a recorded figure only while the hash matches), and
profiles/<tag>_counters.md (L2 hit rate, LDS bank conflicts, translation and DRAM counters per
kernel).
Raw rocprofv3 output goes to --raw (default /tmp/ctxsparse_prof) and is not kept in the tree.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (source hashes and the traffic file of the benchmark)

ENTRIES = ["topk_index", "sparse_decode_attn", "dense_decode_attn", "sparse_decode_step", "key_sketch_update",
           "topk_index_sketch", "sparse_decode_step_sketch", "key_sketch_build"]
GiB_KiB = 1048576.0


def short(name):
    return name.replace("void ", "").split("(")[0]


def _third_template_arg_true(names, kern):
    """Whether a kernel of the call is the FUSED variant (third template argument true)."""
    for n in names:
        m = re.search(kern + r"<\d+, (true|false), (true|false)", n)
        if m and m.group(2) == "true":
            return True
    return False


def classify(names):
    """The entry point a call's library kernels belong to."""
    if any("key_sketch_kernel" in n for n in names):
        return "key_sketch_update"
    if any("q_sketch_kernel" in n or "sketch_select_kernel" in n for n in names):
        return "sparse_decode_step_sketch" if _third_template_arg_true(names, "sketch_select_kernel") \
            else "topk_index_sketch"
    if _third_template_arg_true(names, "cand_select_kernel") or any("attend_scores_kernel" in n for n in names):
        return "sparse_decode_step"
    has_sel = any("select_kernel" in n for n in names)
    if any("sparse_partial" in n for n in names):
        return "sparse_decode_step" if has_sel else "sparse_decode_attn"
    if any("dense_partial" in n for n in names):
        return "dense_decode_attn"
    return "topk_index"


def segments(rows, value):
    """[(entry, {kernel: value summed over the call})] per call, from dispatch rows in start order;
    any kernel outside the library (the flushes, the calibration copy) ends a call."""
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    segs, cur = [], {}
    for r in rows:
        n = short(r["Kernel_Name"])
        if not n.startswith("cs::"):
            if cur:
                segs.append(cur)
            cur = {}
            continue
        cur.setdefault(n, []).append(value(r))
    if cur:
        segs.append(cur)
    out = [(classify(list(s.keys())), {k: sum(v) for k, v in s.items()}) for s in segs]
    # the sketch of the whole cache is built once before the first step and once, timed, after the
    # last: the first and last sketch calls of the run
    ks = [i for i, (e, _) in enumerate(out) if e == "key_sketch_update"]
    for i in (ks[:1] + ks[-1:]) if len(ks) >= 2 else []:
        out[i] = ("key_sketch_build", out[i][1])
    return out


def run(cmd, limit, log):
    """Runs cmd (a list) from /tmp with TMPDIR=/tmp under `timeout -s KILL`, output to log; returns
    the exit status."""
    env = dict(os.environ, TMPDIR="/tmp")
    print("[profile] " + " ".join(cmd), flush=True)
    with open(log, "w") as f:
        return subprocess.call(["timeout", "-s", "KILL", str(limit)] + cmd, cwd="/tmp", env=env, stdout=f,
                               stderr=subprocess.STDOUT)


def program_finished(log):
    with open(log) as f:
        return '"metric"' in f.read()


def find_csv(d, kind):
    files = glob.glob(os.path.join(d, "**", f"*{kind}.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no {kind}.csv under {d}")
    return files[0]


def counter_dispatches(d):
    """One row per dispatch of a counter run: Kernel_Name, Start_Timestamp and every counter's
    value (summed over the rows rocprofv3 wrote for that dispatch and counter)."""
    disp = {}
    for r in csv.DictReader(open(find_csv(d, "counter_collection"))):
        key = r.get("Dispatch_Id") or r.get("Correlation_Id") or (r["Kernel_Name"], r["Start_Timestamp"])
        row = disp.setdefault(key, {"Kernel_Name": r["Kernel_Name"], "Start_Timestamp": r["Start_Timestamp"],
                                    "values": {}})
        name = r.get("Counter_Name", "value")
        row["values"][name] = row["values"].get(name, 0.0) + float(r["Counter_Value"])
    return list(disp.values())


def counters(d, names):
    """Per-call and per-kernel means of each counter of one run, and the calibration copy's
    values: ({counter: {entry: mean}}, {counter: {entry: {kernel: mean}}}, {counter: copy value})."""
    rows = counter_dispatches(d)
    per_call, per_kernel, calib = {}, {}, {}
    for name in names:
        # the calibration copy is the run's largest device copy (1 GiB)
        copies = [r["values"].get(name, 0.0) for r in rows if short(r["Kernel_Name"]) == "__amd_rocclr_copyBuffer"]
        calib[name] = max(copies) if copies else None
        pc = {e: [] for e in ENTRIES}
        pk = {e: {} for e in ENTRIES}
        for e, ks in segments(rows, lambda r, n=name: r["values"].get(n, 0.0)):
            pc[e].append(sum(ks.values()))
            for k, v in ks.items():
                pk[e].setdefault(k, []).append(v)
        per_call[name] = {e: statistics.fmean(v) for e, v in pc.items() if v}
        per_kernel[name] = {e: {k: statistics.fmean(v) for k, v in dd.items()} for e, dd in pk.items()}
    return per_call, per_kernel, calib


# counter passes: (short name, counters) -- each within one pass's per-block limits
# (at most 4 TCC counters with FETCH_SIZE taking 3 and WRITE_SIZE 2, 8 SQ, 4 TCP)
PASSES = [
    ("fetch", ["FETCH_SIZE"]),
    ("write", ["WRITE_SIZE"]),
    ("l2", ["TCC_HIT_sum", "TCC_MISS_sum"]),
    ("lds", ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"]),
    ("xlat", ["TCP_UTCL1_TRANSLATION_MISS_sum", "TCP_UTCL1_REQUEST_sum", "TCC_EA0_RDREQ_DRAM_sum"]),
    ("stall", ["TCC_TAG_STALL_sum", "TCP_TCP_TA_DATA_STALL_CYCLES_sum"]),
]


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--workload", default="llama3_8b_n32k_k655")
    p.add_argument("--sweep-k", default=None)
    p.add_argument("--counters", action="store_true", help="also the counter passes")
    p.add_argument("--raw", default="/tmp/ctxsparse_prof", help="directory for raw rocprofv3 output")
    p.add_argument("--out", default=None, help="where the summaries go (default: profiles/ of the tree)")
    p.add_argument("--parse-only", action="store_true",
                   help="run nothing: rebuild the summaries from the raw output already under --raw")
    args = p.parse_args()

    W = args.workload
    extra = ["--sweep-k", args.sweep_k] if args.sweep_k else []
    tag = W + ("_" + args.sweep_k if args.sweep_k else "")
    raw = os.path.abspath(args.raw)
    os.makedirs(raw, exist_ok=True)
    py = sys.executable or "python3"
    bench_py = os.path.join(ROOT, "bench.py")
    prof_dir = os.path.abspath(args.out) if args.out else os.path.join(ROOT, "profiles")
    os.makedirs(prof_dir, exist_ok=True)
    # --parse-only: every output already exists under --raw
    runner = (lambda cmd, limit, log: 0) if args.parse_only else run
    ex = (" " + " ".join(extra)) if extra else ""

    # 1. the bench line
    blog = os.path.join(raw, f"bench_{tag}.log")
    if runner([py, bench_py, "--workload", W] + extra, 900, blog) != 0:
        raise SystemExit(f"bench.py failed, see {blog}")
    with open(blog) as f:
        bline = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])

    # 2. kernel trace
    kdir = os.path.join(raw, f"ks_{tag}")
    klog = kdir + ".log"
    ktrace = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", kdir, "-o", "ks", "--",
              py, bench_py, "--workload", W] + extra + ["--steps", "5", "--warmup", "2", "--cpu-seconds", "0",
                                                      "--no-extras", "--no-per-config"]
    rc = runner(ktrace, 600, klog)
    if rc != 0 and not program_finished(klog):
        raise SystemExit(f"kernel trace failed ({rc}), see {klog}")
    trace = list(csv.DictReader(open(find_csv(kdir, "kernel_trace"))))
    segs = segments(trace, lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000)
    per_entry = {e: [] for e in ENTRIES}
    per_kernel = {e: {} for e in ENTRIES}
    for e, ks in segs:
        per_entry[e].append(sum(ks.values()))
        for k, v in ks.items():
            per_kernel[e].setdefault(k, []).append(v)

    cmd_ks = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <raw>/ks_{tag} -o ks -- python3 bench.py "
              f"--workload {W}{ex} --steps 5 --warmup 2 --cpu-seconds 0 --no-extras --no-per-config")
    cmd_b = f"python3 bench.py --workload {W}{ex}"
    sk = bline.get("sketch", {})
    ev = {"topk_index": bline["topk_us"], "sparse_decode_attn": bline["sparse_us"],
          "dense_decode_attn": bline["dense_us"], "sparse_decode_step": bline.get("step_us"),
          "key_sketch_update": sk.get("update_us"), "topk_index_sketch": sk.get("topk_us"),
          "sparse_decode_step_sketch": sk.get("step_us"), "key_sketch_build": sk.get("full_build_us")}
    lines = [f"# rocprofv3 kernel statistics — {tag}", "",
             f"Made by `python3 bench_profile.py --workload {W}{ex}` on one MI355X, which runs:", "",
             "    " + cmd_ks, "",
             "Dispatches are grouped into calls (the cache-flush kernels between calls separate them);",
             "`avg us` is the mean kernel duration over every call of the run, warm-up included.", "",
             "| entry point | kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for e in ENTRIES:
        for k, v in sorted(per_kernel[e].items(), key=lambda kv: -statistics.fmean(kv[1])):
            lines.append(f"| {e} | `{k.replace('cs::', '')}` | {len(v)} | {statistics.fmean(v):.2f} | "
                         f"{min(v):.2f} | {max(v):.2f} |")
    lines += ["", "Per entry point (kernel durations of a call, summed, averaged over calls):", "",
              "| entry point | sum of kernel us | bench.py event mean us |", "|---|---|---|"]
    for e in ENTRIES:
        if per_entry[e]:
            evv = ev[e] if ev[e] is not None else float("nan")
            lines.append(f"| {e} | {statistics.fmean(per_entry[e]):.2f} | {evv:.2f} |")
    lines += ["", "bench.py's HIP events (hipEventDisableSystemFence) bracket each call; the difference to the",
              "kernel sum is the dispatch latency after an event record and between a call's kernels (about",
              "4 µs for an empty kernel between two such events).", "",
              "bench.py line of the same workload (`" + cmd_b + "`):", "", "```", json.dumps(bline), "```"]
    with open(os.path.join(prof_dir, f"{tag}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:12 + sum(len(v) for v in per_kernel.values())]), flush=True)
    if not args.counters:
        return

    # 3. counter runs, one pass each
    res, cmds = {}, {}
    for pname, names in PASSES:
        d = os.path.join(raw, f"{pname}_{tag}")
        log = d + ".log"
        cmd = ["rocprofv3", "--pmc", *names, "--kernel-include-regex", "cs::|copyBuffer|reduce_kernel",
               "--output-format", "csv", "-d", d, "-o", pname, "--", py, bench_py, "--workload", W] + extra + \
              ["--steps", "2", "--warmup", "1", "--cpu-seconds", "0", "--no-extras", "--no-per-config",
               "--copy-calibration"]
        rc = runner(cmd, 240, log)
        if rc != 0 and not program_finished(log):  # rocprofv3 may end with a fault of its own after the program
            raise SystemExit(f"{pname} counter run failed ({rc}), see {log}")
        res[pname] = counters(d, names)
        cmds[pname] = (f"rocprofv3 --pmc {' '.join(names)} --kernel-include-regex 'cs::|copyBuffer|reduce_kernel' "
                       f"--output-format csv -d <raw>/{pname}_{tag} -o {pname} -- python3 bench.py --workload {W}{ex} "
                       f"--steps 2 --warmup 1 --cpu-seconds 0 --no-extras --no-per-config --copy-calibration")
    fetch = res["fetch"][0]["FETCH_SIZE"]
    fetch_k = res["fetch"][1]["FETCH_SIZE"]
    fcal = res["fetch"][2]["FETCH_SIZE"]
    write = res["write"][0]["WRITE_SIZE"]
    write_k = res["write"][1]["WRITE_SIZE"]
    wcal = res["write"][2]["WRITE_SIZE"]
    if not fcal or not wcal or fcal < 100000 or wcal < 100000:
        raise SystemExit("calibration copy not found in the counter runs")
    ff, wf = GiB_KiB / fcal, GiB_KiB / wcal
    tl = [f"# HBM traffic per call — {tag}", "",
          f"Made by `python3 bench_profile.py --workload {W}{ex} --counters`; the counter runs:", "",
          "    " + cmds["fetch"], "    " + cmds["write"], "",
          f"Calibration: a plain 1 GiB device-to-device copy in the same runs reads FETCH_SIZE = {fcal:.0f} KiB",
          f"and WRITE_SIZE = {wcal:.0f} KiB, so bytes read = FETCH_SIZE x {ff:.4f} x 1024 and bytes written =",
          f"WRITE_SIZE x {wf:.4f} x 1024.", "",
          "| entry point | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (calibrated) | written MB (calibrated) |",
          "|---|---|---|---|---|---|"]
    for e in ENTRIES:
        for k in sorted(set(fetch_k.get(e, {})) | set(write_k.get(e, {}))):
            fk, wk = fetch_k[e].get(k, 0), write_k[e].get(k, 0)
            tl.append(f"| {e} | `{k.replace('cs::', '')}` | {fk:.0f} | {wk:.0f} | {fk * ff * 1024 / 1e6:.1f} | "
                      f"{wk * wf * 1024 / 1e6:.2f} |")
    try:
        tpath = os.path.join(prof_dir, "traffic.json")
        with open(tpath if os.path.exists(tpath) else bench.TRAFFIC_FILE) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        tj = {}
    tj[tag] = {}
    tl += ["", "Per entry point (sum over a call's kernels) against the algorithmic bytes bench.py counts:", "",
           "| entry point | HBM bytes per call (read + write) | algorithmic bytes | ratio |", "|---|---|---|---|"]
    alg = bline.get("algorithmic_bytes", {})
    for e in ENTRIES:
        if e not in fetch or e not in bench.KERNEL_SOURCES:
            continue
        tot = (fetch[e] * ff + write.get(e, 0) * wf) * 1024
        tj[tag][e] = {"bytes_per_launch": round(tot), "source_sha256": bench.source_hash(e),
                      "fetch_calibration": round(ff, 4), "write_calibration": round(wf, 4),
                      "commands": [cmds["fetch"], cmds["write"]]}
        a = alg.get(e)
        ratio = f"{tot / a:.3f}" if a else "—"
        tl.append(f"| {e} | {tot / 1e6:.1f} MB | {(a or float('nan')) / 1e6:.1f} MB | {ratio} |")
    with open(os.path.join(prof_dir, f"{tag}_traffic.md"), "w") as f:
        f.write("\n".join(tl) + "\n")
    with open(os.path.join(prof_dir, "traffic.json"), "w") as f:
        json.dump(tj, f, indent=1)
    print("\n".join(tl), flush=True)

    # per-kernel counter table
    def kv(pname, name):
        return res[pname][1][name]

    hit, miss = kv("l2", "TCC_HIT_sum"), kv("l2", "TCC_MISS_sum")
    conf, ldsa = kv("lds", "SQ_LDS_BANK_CONFLICT"), kv("lds", "SQ_LDS_IDX_ACTIVE")
    xm, xr, dram = (kv("xlat", "TCP_UTCL1_TRANSLATION_MISS_sum"), kv("xlat", "TCP_UTCL1_REQUEST_sum"),
                    kv("xlat", "TCC_EA0_RDREQ_DRAM_sum"))
    tag_st, ta_st = kv("stall", "TCC_TAG_STALL_sum"), kv("stall", "TCP_TCP_TA_DATA_STALL_CYCLES_sum")
    ct = [f"# L2, LDS, translation and DRAM counters per kernel — {tag}", "",
          f"Made by `python3 bench_profile.py --workload {W}{ex} --counters`; one rocprofv3 --pmc run per pass:", ""]
    ct += ["    " + cmds[p] for p, _ in PASSES[2:]]
    ct += ["", "Means per dispatch over the runs' calls (warm-up included).  L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS);",
           "LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (stall cycles per LDS-active cycle, summed over",
           "shader engines); UTCL1 miss = TCP_UTCL1_TRANSLATION_MISS / TCP_UTCL1_REQUEST (first-level address",
           "translation); DRAM rd req = TCC_EA0_RDREQ_DRAM (32- or 64-byte requests from L2 to memory); read MB is the",
           "calibrated FETCH_SIZE of the traffic table; stalls are summed cycle counts over all instances.", "",
           "| entry point | kernel | L2 hit % | L2 hit+miss | LDS conflict / LDS active | UTCL1 miss % | "
           "UTCL1 req | DRAM rd req | read MB | L2 tag stall | TA data stall |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for e in ENTRIES:
        for k in sorted(hit.get(e, {})):
            h, m_ = hit[e].get(k, 0.0), miss[e].get(k, 0.0)
            c, a_ = conf.get(e, {}).get(k, 0.0), ldsa.get(e, {}).get(k, 0.0)
            tm, tr_ = xm.get(e, {}).get(k, 0.0), xr.get(e, {}).get(k, 0.0)
            l2 = f"{100 * h / (h + m_):.1f}" if h + m_ else "—"
            lds = f"{c / a_:.3f} ({c:.3g} / {a_:.3g})" if a_ else "no LDS"
            ut = f"{100 * tm / tr_:.2f}" if tr_ else "—"
            rd = fetch_k.get(e, {}).get(k, 0.0) * ff * 1024 / 1e6
            ct.append(f"| {e} | `{k.replace('cs::', '')}` | {l2} | {h + m_:.4g} | {lds} | {ut} | {tr_:.4g} | "
                      f"{dram.get(e, {}).get(k, 0.0):.4g} | {rd:.1f} | {tag_st.get(e, {}).get(k, 0.0):.4g} | "
                      f"{ta_st.get(e, {}).get(k, 0.0):.4g} |")
    with open(os.path.join(prof_dir, f"{tag}_counters.md"), "w") as f:
        f.write("\n".join(ct) + "\n")
    print("\n".join(ct), flush=True)


if __name__ == "__main__":
    main()
