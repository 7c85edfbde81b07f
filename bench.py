#!/usr/bin/env python3
"""Throughput of the exact Top-K selector on one MI355X.

One step = one topk_exact call (the whole hot path: dispatch, sampler, fused
full-row pass, certification, refinement, fallbacks, commit) over one group of
rows of a synthetic workload already resident in HBM. Timing follows the
protocol of page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K",
section "什么叫精确，时间怎么量": warm-up, state-conditioning replays, then timed
graph replays with events on the executing stream, groups rotated between
replays, only operator execution inside the timed region, and every timed
configuration gated on a passing contract check.

Prints one JSON line. Default workload: 8192 rows x 1,048,576 columns, causal
ragged lengths (the 1M-width persistent-path configuration).

--workload chain_c1 (or chain_n512k_m1024) times the score + select chain instead:
the FP8 indexer score kernel (Eq. (1) of page "LiteTopK: Exploiting the Curse of
Dimensionality for a Fused Indexer-TopK Kernel ...") feeding the selector, both
captured in one graph, as the pages chain the selector behind an FP8 score
kernel (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section
"框架轨迹"). Its roofline is the score kernel's, against the dense FP8 matrix peak.

--summarize-counters FETCH_DIR WRITE_DIR does no GPU work: it turns two
rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, both with
--copy-calibration) into profiles/hbm_traffic_<workload>.json, scaling each
counter by what it reads for the plain 1 GiB device copy.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Top-K rows/s and achieved HBM GB/s (frac of peak), K=2048, FP32 ragged rows"
HBM_PEAK_GBPS = 8000.0
K_DEFAULT = 2048
EXECUTIONS = {"auto": 0, "persistent": 1, "row": 2, "rowsplit": 3}  # TOPK_EXEC_* values
CHAIN_NAMES = ("chain_c1", "chain_n512k_m1024")  # score + select workloads (workloads.CHAINS)


# Timing schedules. "pages": the protocol of page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确
# Top-K", section "什么叫精确，时间怎么量": 10 warm-up replays, 2 x 50 state-conditioning
# replays, then 7 rounds of 100 timed replays with the groups rotated between replays.
# "quick": a short version of the same.
PROTOCOLS = {"pages": {"warmup": 10, "condition": 100, "steps": 700},
             "quick": {"warmup": 5, "condition": 20, "steps": 40}}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--protocol", choices=sorted(PROTOCOLS), default="pages",
                    help="timing schedule; --steps/--warmup/--condition override its counts")
    ap.add_argument("--steps", type=int, default=None, help="timed calls (graph replays)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed warm-up replays")
    ap.add_argument("--condition", type=int, default=None, help="untimed state-conditioning replays")
    ap.add_argument("--workload", default="c3b")
    ap.add_argument("--k", type=int, default=K_DEFAULT, help="K (the method's operating point is 2048)")
    ap.add_argument("--calls-per-graph", type=int, default=None,
                    help="calls captured in one graph (default 100 for c0, whose calls take microseconds, "
                         "else 1); the per-call time is the replay time divided by it")
    ap.add_argument("--eager", action="store_true", help="direct launches instead of graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work for the oracle leg")
    ap.add_argument("--check-rows", type=int, default=32, help="rows per group checked before timing")
    ap.add_argument("--no-probe", action="store_true", help="skip timing the stream-read probe")
    ap.add_argument("--execution", choices=sorted(EXECUTIONS), default="auto",
                    help="row-to-workgroup mapping (auto: the library's shape-based choice)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy first (known bytes, for counter calibration)")
    ap.add_argument("--sorted", action="store_true",
                    help="time topk_exact_sorted (indices by score descending plus their values) instead")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "script with --copy-calibration into profiles/hbm_traffic_<workload>.json")
    ap.add_argument("--phases", action="store_true",
                    help="after the timed region, one more call per group records per-row phase stamps "
                         "(sample, proposal, pass, commit, recovery) and the line reports their medians")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="no GPU work: per-kernel durations and per-call spans of a rocprofv3 "
                         "--kernel-trace run of this script, as one JSON line")
    args = ap.parse_args(argv)
    for key, v in PROTOCOLS[args.protocol].items():
        if getattr(args, key) is None:
            setattr(args, key, v)
    if args.calls_per_graph is None:
        args.calls_per_graph = 100 if args.workload == "c0" else 1
    return args


def _code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


SOURCES = {
    "selector": ("exact_top_selection_stride_amd/csrc/topk_exact.hip", "include/topk_exact.h"),
    "indexer": ("exact_top_selection_stride_amd/csrc/indexer_scores.hip", "include/topk_exact.h",
                "exact_top_selection_stride_amd/build.py"),
}


def kernel_source_digest(part: str = "selector") -> str:
    """Digest of one kernel family's code (comments and layout ignored): counter summaries
    taken on one digest describe exactly the kernels of any source with the same digest."""
    h = hashlib.sha256()
    for rel in SOURCES[part]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def order_keys(x):
    """IEEE totalOrder keys of float32 values as int64 (for the torch-side gate)."""
    import torch
    u = x.contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    neg = u >= 0x80000000
    return torch.where(neg, 0xFFFFFFFF - u, u + 0x80000000)


def gate_rows(scores, lengths, out, K, sentinel, rows):
    """Contract check of chosen rows on the GPU with plain torch ops (no oracle):
    distinct in-prefix indices, exactly K for L > K, min(selected) >= max(unselected),
    and the short-row layout. Returns the number of violating rows."""
    import torch
    bad = 0
    for r in rows:
        L = int(lengths[r])
        o = out[r].to(torch.int64)
        if L <= K:
            ok = bool(torch.equal(torch.sort(o[:L]).values, torch.arange(L, device=o.device))) and \
                bool(torch.all(o[L:] == sentinel))
        else:
            ok = bool(torch.all((o >= 0) & (o < L)))
            ok = ok and int(torch.unique(o).numel()) == K
            if ok:
                keys = order_keys(scores[r, :L])
                sel = torch.zeros(L, dtype=torch.bool, device=o.device)
                sel[o] = True
                ok = bool(keys[sel].min() >= keys[~sel].max())
        bad += 0 if ok else 1
    return bad


def cpu_baseline(scores, lengths, K, sentinel, target_s, max_rows=1024):
    """Times the CPU oracle on a bounded leading block of the group's rows, repeating
    the block until about target_s seconds of selection work have been timed."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    n = min(int(lengths.shape[0]), max_rows)
    blk_s = scores[:n].cpu().numpy()
    blk_l = lengths[:n].cpu().numpy().astype(np.int32)
    done_rows, spent, reps = 0, 0.0, 0
    while spent < target_s and reps < 50:
        t0 = time.perf_counter()
        oracle.topk(blk_s, blk_l, K, sentinel, n_threads=threads)
        spent += time.perf_counter() - t0
        done_rows += n
        reps += 1
    return {"value": done_rows / spent, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} rows of the timed group (same lengths and values) selected "
                      f"{reps} times on host copies, {spent:.1f} s of selection"}


def copy_calibration(dev):
    """Three plain device copies of exactly 2^28 floats (1 GiB read + 1 GiB written each):
    known bytes that scale the HBM counters of the same run."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _counter_rows(d):
    """(kernel name, dispatch id, counter value) rows of a rocprofv3 --pmc csv output dir."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


SELECTOR_KERNELS = r"topk_rows_kernel|split_[a-z]+_kernel"
RECOVERY_KERNELS = r"recovery_[a-z]+_kernel"
CALL_FIRST_KERNELS = r"topk_rows_kernel|split_sample_kernel"   # one per selector call


def summarize_counters(args, out_dir=None):
    """Writes profiles/hbm_traffic_<workload>.json (or into out_dir) from a FETCH_SIZE and a
    WRITE_SIZE run. Selector calls: bytes per call of the whole call (selector and exact-
    recovery kernels) and of the selector kernels alone; chain workloads: the score kernel."""
    import re
    chain = args.workload in CHAIN_NAMES
    sel_re = re.compile(r"indexer_scores_kernel" if chain else SELECTOR_KERNELS)
    rec_re = re.compile(r"(?!x)x" if chain else RECOVERY_KERNELS)
    first_re = re.compile(r"indexer_scores_kernel" if chain else CALL_FIRST_KERNELS)
    out = {"workload": args.workload,
           "kernel_source_digest": kernel_source_digest("indexer" if chain else "selector"),
           "calibration": "plain device copy of 2^28 floats (1 GiB read, 1 GiB written)"}
    total = sel_total = 0.0
    names = set()
    for counter, d, known_kib in (("FETCH_SIZE", args.summarize_counters[0], 1 << 20),
                                  ("WRITE_SIZE", args.summarize_counters[1], 1 << 20)):
        sel, rec, calib = {}, {}, {}
        calls = set()
        for name, disp, v in _counter_rows(d):
            if "copyBuffer" in name:
                calib[disp] = calib.get(disp, 0.0) + v
            elif sel_re.search(name):
                sel[disp] = sel.get(disp, 0.0) + v
                names.add(sel_re.search(name).group(0) + ("<true>" if "<true>" in name else
                                                          "<false>" if "<false>" in name else ""))
                if first_re.search(name):
                    calls.add(disp)
            elif rec_re.search(name):
                rec[disp] = rec.get(disp, 0.0) + v
                names.add(rec_re.search(name).group(0))
        # The calibration copies are the script's first three device copies (1 GiB each).
        first = [calib[k] for k in sorted(calib)[:3]]
        if len(first) < 3 or not sel or not calls or max(first) > 1.01 * min(first):
            raise SystemExit(f"{counter}: calibration copies or kernel dispatches missing in {d}")
        cal = sum(first) / len(first)
        scale = known_kib / cal
        n_calls = len(calls)
        sel_mean = sum(sel.values()) / n_calls
        whole_mean = (sum(sel.values()) + sum(rec.values())) / n_calls
        key = counter.split("_")[0].lower()
        out["kernel"] = " + ".join(sorted(names))
        out[f"{key}_raw_kib_per_call"] = whole_mean
        out[f"{key}_selector_raw_kib_per_call"] = sel_mean
        out[f"{key}_calibration_kib"] = cal
        out[f"{key}_scale"] = scale
        out[f"{key}_bytes"] = whole_mean * scale * 1024
        out[f"{key}_calls"] = n_calls
        total += whole_mean * scale * 1024
        sel_total += sel_mean * scale * 1024
    out["bytes_per_launch"] = total
    out["selector_bytes_per_launch"] = sel_total
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"hbm_traffic_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)
    return 0


def summarize_trace(d):
    """Per-kernel durations and per-call spans from a rocprofv3 --kernel-trace output dir.
    A call starts at each selector kernel that opens one (topk_rows_kernel, split_sample)
    and holds the selector, recovery and sort kernels that follow it; its span runs from
    the first kernel's start to the last one's end."""
    import csv
    import glob
    import re
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows.sort()
    short = re.compile(r"(topk_rows_kernel<(?:true|false)>|split_[a-z]+_kernel|recovery_[a-z]+_kernel|"
                       r"sort_rows_kernel<\d+>|indexer_scores_kernel<\d+>|stream_read_probe_kernel)")
    first = re.compile(CALL_FIRST_KERNELS)
    member = re.compile(SELECTOR_KERNELS + "|" + RECOVERY_KERNELS + r"|sort_rows_kernel")
    per = {}
    calls, cur = [], None
    for t0, t1, name in rows:
        m = short.search(name)
        key = m.group(1) if m else name[:60]
        per.setdefault(key, []).append(t1 - t0)
        if first.search(name):
            if cur:
                calls.append(cur)
            cur = [t0, t1]
        elif cur and member.search(name):
            cur[1] = max(cur[1], t1)
        elif cur:
            calls.append(cur)
            cur = None
    if cur:
        calls.append(cur)
    spans = [b - a for a, b in calls]
    out = {"kernels": {k: {"calls": len(v), "average_ns": sum(v) / len(v), "min_ns": min(v), "max_ns": max(v)}
                       for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))}}
    if spans:
        out["call_spans"] = {"calls": len(spans), "mean_ns": sum(spans) / len(spans),
                             "median_ns": statistics.median(spans), "p10_ns": _quantile(spans, 0.1),
                             "p90_ns": _quantile(spans, 0.9)}
    return out


def _traffic(workload, part, field="bytes_per_launch"):
    """Counter bytes per call from profiles/hbm_traffic_<workload>.json, or None when the
    file is missing or was taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if os.path.exists(path):
        with open(path) as f:
            prof = json.load(f)
        if prof.get("kernel_source_digest") == kernel_source_digest(part):
            return prof.get(field)
    return None


def cpu_baseline_chain(q, k, w, lengths, K, sentinel, target_s):
    """Times the CPU oracles (indexer scores, then selection) on whole rows of the call
    until about target_s seconds have been spent."""
    import numpy as np
    import oracle
    from oracle import indexer_scores as O
    threads = oracle.default_threads()
    qh, kh, wh = q.cpu().numpy(), k.cpu().numpy(), w.cpu().numpy()
    lh = lengths.cpu().numpy().astype(np.int32)
    done, spent, r = 0, 0.0, 0
    while spent < target_s and done < lh.shape[0]:
        t0 = time.perf_counter()
        sc = O.indexer_scores(qh[r:r + 1], kh, wh[r:r + 1], lh[r:r + 1])
        oracle.topk(sc.astype(np.float32), lh[r:r + 1], K, sentinel, n_threads=threads)
        spent += time.perf_counter() - t0
        done += 1
        r += 1
    return {"value": done / spent, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"first {done} rows of the call scored (float64 numpy) and selected on host "
                      f"copies, {spent:.1f} s"}


def run_chain(args):
    """Score + select chain: the FP8 indexer score kernel and the selector in one graph."""
    import torch
    import exact_top_selection_stride_amd as tk
    from exact_top_selection_stride_amd import workloads as W

    K, sentinel = K_DEFAULT, -1
    c = W.get_chain(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)
    q, k, w, L = W.make_chain(c, dev)
    scores = torch.empty((c.M, c.n_alloc), dtype=torch.float32, device=dev)
    idx = torch.empty((c.M, K), dtype=torch.int32, device=dev)
    tk.reserve(c.M, c.n_alloc, K)

    tk.reset_stats()
    tk.indexer_topk(q, k, w, L, K=K, sentinel=sentinel, scores=scores, out=idx)
    torch.cuda.synchronize()
    stats = tk.get_stats()
    rows = sorted(set([0, c.M - 1] + [int(i) for i in torch.linspace(0, c.M - 1, min(args.check_rows, c.M)).round().tolist()]))
    violations = gate_rows(scores, L, idx, K, sentinel, rows)
    if violations:
        print(json.dumps({"error": "contract violations before timing", "violations": violations}), flush=True)
        return 1

    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    graph = None
    if not args.eager:
        with torch.cuda.stream(stream):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                tk.indexer_topk(q, k, w, L, K=K, sentinel=sentinel, scores=scores, out=idx)
        torch.cuda.synchronize()

    def launch():
        if graph is not None:
            graph.replay()
        else:
            tk.indexer_topk(q, k, w, L, K=K, sentinel=sentinel, scores=scores, out=idx, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup + args.condition):
            launch()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            starts[i].record(stream)
            launch()
            ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [starts[i].elapsed_time(ends[i]) for i in range(args.steps)]

    # Kernel times: the score kernel between events on the bench stream (one kernel), the
    # selector kernels through the library's timing hook.
    s0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    s1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    k0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    k1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for e in k0 + k1:
            e.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            s0[i].record(stream)
            tk.indexer_scores(q, k, w, L, out=scores, stream=stream)
            s1[i].record(stream)
            tk.time_next_call(k0[i], k1[i])
            tk.topk_exact(scores, L, K=K, sentinel=sentinel, out=idx, stream=stream)
    torch.cuda.synchronize()
    score_ms = sum(s0[i].elapsed_time(s1[i]) for i in range(args.steps)) / args.steps
    select_ms = sum(k0[i].elapsed_time(k1[i]) for i in range(args.steps)) / args.steps
    post_bad = gate_rows(scores, L, idx, K, sentinel, [0, c.M // 2, c.M - 1])

    Lsum = int(L.to(torch.int64).sum())
    flops = 2.0 * c.heads * c.dim * Lsum          # q.k products of the valid (t, s) pairs
    achieved = flops / (score_ms / 1e3) / 1e12
    sel_bytes = 4 * Lsum + 4 * int(((L.to(torch.int64) + 127) // 128).sum()) + 4 * c.M * K + 4 * c.M
    result = {
        "metric": "Score + select chain rows/s (FP8 indexer scores, then exact Top-K K=2048 of the "
                  "ragged FP32 rows, one hipGraph)",
        "value": c.M * args.steps / wall,
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 (scores), u32 (selection)", "data": "synthetic",
        "config": {"workload": c.name, "M": c.M, "N_alloc": c.n_alloc, "K": K, "heads": c.heads,
                   "head_dim": c.dim, "lengths": "causal", "hot_p": c.hot_p,
                   "launch": "eager" if graph is None else "hipGraph replay (scores + select)"},
        "median_call_ms": statistics.median(per_call_ms),
        "p10_call_ms": sorted(per_call_ms)[int(0.1 * (len(per_call_ms) - 1))],
        "p90_call_ms": sorted(per_call_ms)[int(0.9 * (len(per_call_ms) - 1))],
        "roofline": {"bound": "mfma", "kernel": "indexer_scores_kernel", "achieved": achieved,
                     "peak": 5000.0, "unit": "TFLOP/s", "frac": achieved / 5000.0,
                     "traffic": _traffic(c.name, "indexer"), "mean_launch_ms": score_ms,
                     "timing": f"HIP events around the score kernel, {args.steps} direct launches on the bench stream",
                     "algorithmic_flops_per_launch": flops,
                     "peak_note": "MI355X dense FP8 matrix peak"},
        "selector": {"mean_launch_ms": select_ms, "algorithmic_bytes_per_launch": sel_bytes,
                     "achieved_gbps": sel_bytes / (select_ms / 1e3) / 1e9,
                     "frac_of_8tbps": sel_bytes / (select_ms / 1e3) / 1e9 / HBM_PEAK_GBPS},
        "parity": {"rows_checked": len(rows), "violations": violations, "post_timing_violations": post_bad,
                   "gate": "torch contract check of the selection on the GPU's scores"},
        "path_stats_first_call": stats,
        "kernel_source_digest": kernel_source_digest("indexer"),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_chain(q, k, w, L, K, sentinel, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0 if post_bad == 0 else 1


PATH_NAMES = {1: "sentinel", 2: "direct", 3: "tau0", 4: "tau1", 5: "recover_inplace", 6: "recover_queued",
              7: "forced_recovery", 8: "tau_a"}


def phase_summary(records, khz):
    """Per-row phase records (rows x 8 int64: stamps start, sampled, proposed, passed, end,
    recovered; where; counts) of one or more calls, each call's rows a list, reduced to
    medians in microseconds per path: sample, proposal (tau selection), pass, refine +
    commit, the row's time in its workgroup, and for recovery rows the recovery time after
    the row's own work; plus, per call, when the last row ended relative to the first
    start and how far the rows' ends spread."""
    us = 1e3 / khz
    paths, calls = {}, []
    for rec in records:
        starts, ends, rec_ends = [], [], []
        for r in rec:
            start, sampled, proposed, passed, end, recovered, where, counts = (int(v) for v in r)
            code = where & 0xFF
            if code == 0:
                continue
            name = PATH_NAMES.get(code & 0x7F, str(code)) + ("_split" if code & 0x80 else "")
            d = paths.setdefault(name, {"rows": 0, "row": [], "sample": [], "proposal": [], "pass": [],
                                        "refine_commit": [], "recovery": [], "c_tau1": []})
            d["rows"] += 1
            d["row"].append((end - start) * us)
            if sampled and proposed and passed and not code & 0x80:
                d["sample"].append((sampled - start) * us)
                d["proposal"].append((proposed - sampled) * us)
                d["pass"].append((passed - proposed) * us)
                if code & 0x7F in (3, 4):
                    d["refine_commit"].append((end - passed) * us)
            if code & 0x7F in (5, 6) and recovered:
                d["recovery"].append((recovered - end) * us)
                rec_ends.append(recovered)
            if counts:
                d["c_tau1"].append(counts & 0xFFFFFFFF)
            starts.append(start)
            ends.append(end)
        if starts:
            t0 = min(starts)
            calls.append({"last_end_us": (max(ends) - t0) * us, "first_end_us": (min(ends) - t0) * us,
                          "last_recovered_us": (max(rec_ends) - t0) * us if rec_ends else None})
    out = {}
    for name, d in sorted(paths.items()):
        out[name] = {"rows": d["rows"]}
        for key in ("row", "sample", "proposal", "pass", "refine_commit", "recovery", "c_tau1"):
            if d[key]:
                out[name][f"median_{key}" + ("" if key == "c_tau1" else "_us")] = statistics.median(d[key])
    med = lambda k: statistics.median([c[k] for c in calls if c[k] is not None]) if any(
        c[k] is not None for c in calls) else None
    return {"paths": out, "calls": len(calls), "median_last_end_us": med("last_end_us"),
            "median_first_end_us": med("first_end_us"), "median_last_recovered_us": med("last_recovered_us")}


def versions():
    """Software versions recorded with every line (a drift in torch's RNG stream between
    versions would change the synthetic inputs; the checksums below detect it)."""
    import torch
    v = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None), "rocm": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            v["rocm"] = f.read().strip()
    except OSError:
        pass
    return v


def device_checksum(t) -> str:
    """64-bit sum of the 32-bit patterns of a GPU tensor (row chunks on the GPU), as hex."""
    import torch
    x = t.view(torch.int32) if t.dtype == torch.float32 else t.to(torch.int32)
    x = x.reshape(x.shape[0], -1) if x.dim() > 1 else x.reshape(-1, 1)
    step = max(1, (1 << 26) // max(1, x.shape[1]))
    total = 0
    for r0 in range(0, x.shape[0], step):
        total += int(x[r0:r0 + step].to(torch.int64).sum())
    return f"{total & 0xFFFFFFFFFFFFFFFF:016x}"


def _quantile(v, q):
    v = sorted(v)
    return v[int(q * (len(v) - 1))]


def path_model_line(w, stats, lengths, K):
    """Rows of the first calls (every row of the window once) that missed K at tau0 and at
    tau1, beside the beta-binomial model of the stride-128 thresholds for rows of
    independently drawn scores (exact_top_selection_stride_amd.path_model; the bench runs
    the method's stride and targets). FP32 windows only: bf16-rounded rows have ties, which
    the model excludes."""
    if w.bf16 or stats.get("sampled", 0) == 0:
        return None
    from exact_top_selection_stride_amd import path_model as PM
    e0, e1 = PM.expected_short_rows(lengths.cpu().tolist(), K)
    n1 = stats["tau_a"] + stats["recover_under"]
    return {"rows_short_at_tau0": stats["tau1"] + n1, "model_rows_short_at_tau0": round(e0, 1),
            "rows_short_at_tau1": n1, "model_rows_short_at_tau1": round(e1, 1)}


def main(argv=None):
    args = parse(argv)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace)), flush=True)
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "the selector runs on one GPU only (--gpus 1); sharding rows "
                                   "across GPUs, with no exchange between them, is not implemented",
                          "n_gpus_requested": args.gpus}), flush=True)
        return 2
    if args.workload in CHAIN_NAMES:
        return run_chain(args)
    import torch
    import exact_top_selection_stride_amd as tk
    from exact_top_selection_stride_amd import workloads as W

    K, sentinel = args.k, -1
    w = W.get(args.workload)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(dev)
    t_gen = time.perf_counter()
    window, lengths = W.make_window(w, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    checksums = {"scores": device_checksum(window), "row_len": device_checksum(lengths)}
    groups = [(window[g * w.M:(g + 1) * w.M], lengths[g * w.M:(g + 1) * w.M].contiguous())
              for g in range(w.groups)]
    outs = [torch.empty((w.M, K), dtype=torch.int32, device=dev) for _ in range(w.groups)]
    vals = [torch.empty((w.M, K), dtype=torch.float32, device=dev) for _ in range(w.groups)] if args.sorted else None
    tk.reserve(w.M, w.n_alloc, K)

    def select(g, stream=None):
        s, l = groups[g]
        if args.sorted:
            tk.topk_exact_sorted(s, l, K=K, sentinel=sentinel, out=outs[g], out_values=vals[g], stream=stream)
        else:
            tk.topk_exact(s, l, K=K, sentinel=sentinel, out=outs[g], stream=stream)
    tk.set_execution(EXECUTIONS[args.execution])

    # Contract gate on every group before anything is timed.
    tk.reset_stats()
    violations, checked = 0, 0
    for g, (s, l) in enumerate(groups):
        select(g)
        torch.cuda.synchronize()
        n_chk = min(args.check_rows, w.M)
        rows = sorted(set([0, w.M - 1] + [int(i) for i in torch.linspace(0, w.M - 1, n_chk).round().tolist()]))
        violations += gate_rows(s, l, outs[g], K, sentinel, rows)
        checked += len(rows)
    stats = tk.get_stats()
    if violations:
        print(json.dumps({"metric": METRIC, "error": "contract violations before timing",
                          "violations": violations, "rows_checked": checked}), flush=True)
        return 1

    # One graph per group, holding calls_per_graph calls of it.
    cpg = max(1, args.calls_per_graph)
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    if not args.eager:
        with torch.cuda.stream(stream):
            for g in range(w.groups):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=stream):
                    for _ in range(cpg):
                        select(g)
                graphs.append(gr)
        torch.cuda.synchronize()

    def launch(i):
        g = i % w.groups
        if graphs:
            graphs[g].replay()
        else:
            for _ in range(cpg):
                select(g, stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup + args.condition):
            launch(i)
    torch.cuda.synchronize()

    # Timed region: steps launches, groups rotated, each bracketed by events on the stream.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            starts[i].record(stream)
            launch(i)
            ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [starts[i].elapsed_time(ends[i]) / cpg for i in range(args.steps)]
    by_group = {}
    for i, ms in enumerate(per_call_ms):
        by_group.setdefault(i % w.groups, []).append(ms)
    group_medians = [statistics.median(v) for _, v in sorted(by_group.items())]

    # Selector kernels alone (the library's timing hook brackets them, before the exact-
    # recovery kernels): the same calls, launched directly on the same stream.
    n_hook = min(args.steps, 100)
    kstart = [torch.cuda.Event(enable_timing=True) for _ in range(n_hook)]
    kstop = [torch.cuda.Event(enable_timing=True) for _ in range(n_hook)]
    with torch.cuda.stream(stream):
        for e in kstart + kstop:
            e.record(stream)  # creates the HIP events
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(n_hook):
            g = i % w.groups
            s, l = groups[g]
            tk.time_next_call(kstart[i], kstop[i])
            tk.topk_exact(s, l, K=K, sentinel=sentinel, out=outs[g], stream=stream)
    torch.cuda.synchronize()
    kernel_ms = [kstart[i].elapsed_time(kstop[i]) for i in range(n_hook)]

    phases = None
    if args.phases:
        buf = torch.zeros((w.M, 8), dtype=torch.int64, device=dev)
        khz = tk.record_phases(buf)
        recs = []
        try:
            for g in range(w.groups):
                buf.zero_()
                select(g, stream=stream)
                torch.cuda.synchronize()
                recs.append(buf.cpu().tolist())
        finally:
            tk.record_phases(None)
        phases = phase_summary(recs, khz)
        phases["wall_clock_khz"] = khz

    # Post-timing contract check of the last output of every group.
    post_bad = 0
    for g, (s, l) in enumerate(groups):
        post_bad += gate_rows(s, l, outs[g], K, sentinel, [0, w.M // 2, w.M - 1])

    # Bytes. The metric's bytes are the valid FP32 scores a call must read, 4 L per row with
    # L > K; the selector kernels' algorithmic bytes add the logical sample reads (4 bytes
    # per stride-128 sample), the index writes and the row lengths.
    group_bytes = [W.valid_score_bytes(l, K) for _, l in groups]
    group_alg = []
    for _, l in groups:
        L = l.to(torch.int64)
        long_rows = L > K
        group_alg.append(4 * int(L[long_rows].sum()) + 4 * int(((L[long_rows] + 127) // 128).sum())
                         + 4 * w.M * K + 4 * w.M)
    steps_bytes = sum(group_bytes[i % w.groups] for i in range(args.steps)) * cpg
    mean_call_ms = sum(per_call_ms) / args.steps
    mean_bytes = sum(group_bytes[i % w.groups] for i in range(args.steps)) / args.steps
    call_achieved = mean_bytes / (mean_call_ms / 1e3) / 1e9
    alg_hook = sum(group_alg[i % w.groups] for i in range(n_hook)) / n_hook
    kernel_mean_ms = sum(kernel_ms) / n_hook
    sel_achieved = alg_hook / (kernel_mean_ms / 1e3) / 1e9
    digest = kernel_source_digest("selector")
    split = bool(stats.get("rowsplit"))
    sel_kernels = "split_{sample,select,pass,finish}_kernel" if split else (
        "topk_rows_kernel<true> (persistent)" if stats.get("persistent") else "topk_rows_kernel<false> (row per WG)")
    metric = METRIC if K == K_DEFAULT else METRIC.replace("K=2048", f"K={K}")
    median_call = statistics.median(group_medians)

    result = {
        "metric": metric,
        "value": w.M * args.steps * cpg / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N_alloc": w.n_alloc, "K": K, "groups": w.groups,
                   "lengths": w.lengths, "tail_p": w.tail_p, "bf16_rounded": w.bf16,
                   "launch": "eager" if args.eager else "hipGraph replay", "calls_per_graph": cpg,
                   "execution": args.execution, "protocol": args.protocol, "condition": args.condition,
                   "output": "sorted indices + values" if args.sorted else "unordered indices"},
        "hbm_gbps": steps_bytes / wall / 1e9,
        "hbm_frac_of_peak": steps_bytes / wall / 1e9 / HBM_PEAK_GBPS,
        "median_call_ms": median_call,
        "median_call_ms_by_group": group_medians,
        "rows_per_s_at_median_call": w.M / (median_call / 1e3),
        "mean_call_ms": mean_call_ms,
        "p10_call_ms": _quantile(per_call_ms, 0.1),
        "p90_call_ms": _quantile(per_call_ms, 0.9),
        "roofline": {"bound": "hbm",
                     "kernel": f"whole call: {sel_kernels} + recovery_{{hist,collect,finish}}_kernel",
                     "achieved": call_achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": call_achieved / HBM_PEAK_GBPS,
                     "traffic": None if args.sorted or K != K_DEFAULT else _traffic(w.name, "selector"),
                     "mean_launch_ms": mean_call_ms,
                     "timing": f"HIP events on the bench stream around each of the {args.steps} timed "
                               f"graph replays (all kernels of the call, recovery included)"
                               + (f", divided by the {cpg} calls each replay holds" if cpg > 1 else ""),
                     "bytes_per_launch": mean_bytes,
                     "bytes": "valid FP32 score bytes, 4 L per row with L > K"},
        "roofline_selector_kernels": {
                     "bound": "hbm", "kernel": sel_kernels, "achieved": sel_achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": sel_achieved / HBM_PEAK_GBPS,
                     "traffic": None if K != K_DEFAULT else _traffic(w.name, "selector", "selector_bytes_per_launch"),
                     "mean_launch_ms": kernel_mean_ms,
                     "timing": f"library-recorded HIP events around the selector kernels (before the "
                               f"exact-recovery kernels), {n_hook} direct calls on the bench stream",
                     "bytes_per_launch": alg_hook,
                     "bytes": "4 L + 4 ceil(L / 128) per row with L > K, 4 K per row written, 4 per row length"},
        "parity": {"rows_checked": checked, "violations": violations, "post_timing_violations": post_bad,
                   "gate": "torch contract check on device"},
        "path_stats_first_calls": stats,
        "path_model": path_model_line(w, stats, lengths, K),
        "kernel_source_digest": digest,
        "generation_s": round(t_gen, 2),
        "input_checksums": checksums,
        "phases": phases,
        "versions": versions(),
    }
    if not args.no_probe:
        sink = torch.empty(4096, device=dev)
        flat = window.view(-1)
        tk.stream_read_probe(flat, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            tk.stream_read_probe(flat, sink)
        e1.record()
        torch.cuda.synchronize()
        probe_s = e0.elapsed_time(e1) / 1e3 / reps
        result["stream_read_probe_gbps"] = flat.numel() * 4 / probe_s / 1e9
        result["roofline"]["frac_of_measured_read"] = call_achieved / result["stream_read_probe_gbps"]
    if not args.no_cpu_baseline:
        s0, l0 = groups[0]
        result["cpu_baseline"] = cpu_baseline(s0, l0, K, sentinel, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0 if post_bad == 0 else 1


if __name__ == "__main__":
    sys.exit(main())
