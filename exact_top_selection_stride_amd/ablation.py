"""Ablation harness for the proposal mechanism on MI355X.

Sweeps the sample stride s and the primary target rho0 (secondary rho1 = rho0 + 0.25)
of the sampled path, the direct exact proposal and the default dispatch, over the short-row widths where
the pages place the crossover between sampled and exact proposals (page
"几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section
"采样不是处处都该开": stride and target ablations, sampled against exact proposal at
16K to 64K). Every setting gives the same exact result; what changes is the time per
call and how often each certification path is taken, which is what the sweep prints.

    python -m exact_top_selection_stride_amd.ablation [--widths 16384 32768 65536]
           [--rows 4096] [--strides 16 32 64 128 256] [--rho0 1 1.25 1.5 1.75] [--steps 20]

One JSON line per setting: workload, mode, stride, rho0, rho1, median call time over
graph replays, rows/s and the path rates from the device counters of the first calls.
Inputs are the bf16-rounded causal C4 windows of `workloads.py`.

    python -m exact_top_selection_stride_amd.ablation --crossover [--widths ...] [--row-counts ...]

The crossover sweep of the same section: for every width and row count of the C4
configurations (groups of the causal window, tiled past 8192 rows), the call time of
the exact proposal (the direct path: rows staged in LDS up to 16K, a full-row radix
select beyond), of the sampled proposal at the method's stride and targets, and of the
default dispatch; per-group median, then the median across groups, as the pages report.
One JSON line per cell, then a markdown table.
"""
import argparse
import json
import statistics
import sys

import torch

from . import _binding as tk
from . import workloads as W


def _time_groups(groups, outs, K, steps, stream):
    """Median per group of the call times over graph replays (groups rotated), then the
    median across groups."""
    graphs = []
    with torch.cuda.stream(stream):
        for g, (s, l) in enumerate(groups):
            tk.topk_exact(s, l, K=K, out=outs[g], stream=stream)  # outside capture first
        torch.cuda.synchronize()
        for g, (s, l) in enumerate(groups):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                tk.topk_exact(s, l, K=K, out=outs[g], stream=stream)
            graphs.append(gr)
    torch.cuda.synchronize()
    n = len(graphs)
    total = max(steps, 3 * n)
    ev = []
    with torch.cuda.stream(stream):
        for i in range(total + n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graphs[i % n].replay()
            e1.record(stream)
            if i >= n:
                ev.append((i % n, e0, e1))
    torch.cuda.synchronize()
    per = {}
    for g, a, b in ev:
        per.setdefault(g, []).append(a.elapsed_time(b))
    return statistics.median(statistics.median(v) for v in per.values())


def crossover(args):
    K = 2048
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    modes = (("direct", tk.PATH_DIRECT), ("sampled", tk.PATH_SAMPLED), ("auto", tk.PATH_AUTO))
    table = {}
    for n in args.widths:
        big = W.get(f"c4_n{n}_m{max(args.row_counts)}")
        window, lengths = W.make_window(big, dev)
        for M in args.row_counts:
            w = W.get(f"c4_n{n}_m{M}")
            groups = [(window[g * w.M:(g + 1) * w.M], lengths[g * w.M:(g + 1) * w.M].contiguous())
                      for g in range(w.groups)]
            outs = [torch.empty((w.M, K), dtype=torch.int32, device=dev) for _ in groups]
            tk.reserve(w.M, w.n_alloc, K)
            cell = {}
            for name, path in modes:
                with tk.path_override(path):
                    cell[name] = _time_groups(groups, outs, K, args.steps, stream)
            cell["sampled_over_direct"] = cell["direct"] / cell["sampled"]
            table[(n, M)] = cell
            print(json.dumps({"width": n, "rows": M, "groups": w.groups,
                              **{k: round(v, 5) for k, v in cell.items()}}), flush=True)
            del groups, outs
        del window, lengths
        torch.cuda.empty_cache()
    print("\n| width \\ rows | " + " | ".join(str(M) for M in args.row_counts) + " |")
    print("|---|" + "---|" * len(args.row_counts))
    for n in args.widths:
        cells = []
        for M in args.row_counts:
            c = table[(n, M)]
            cells.append(f"{c['direct']:.3f} / {c['sampled']:.3f} / {c['auto']:.3f}")
        print(f"| {n} | " + " | ".join(cells) + " |")
    return 0


def _time_call(groups, outs, K, steps, stream):
    graphs = []
    with torch.cuda.stream(stream):
        for g, (s, l) in enumerate(groups):
            tk.topk_exact(s, l, K=K, out=outs[g], stream=stream)  # outside capture first
        torch.cuda.synchronize()
        for g, (s, l) in enumerate(groups):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                tk.topk_exact(s, l, K=K, out=outs[g], stream=stream)
            graphs.append(gr)
    torch.cuda.synchronize()
    ev = []
    with torch.cuda.stream(stream):
        for i in range(steps + 4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            graphs[i % len(graphs)].replay()
            e1.record(stream)
            if i >= 4:
                ev.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ev)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--widths", type=int, nargs="+", default=list(W.C4_WIDTHS))
    ap.add_argument("--rows", type=int, default=4096)
    ap.add_argument("--strides", type=int, nargs="+", default=[16, 32, 64, 128, 256])
    ap.add_argument("--rho0", type=float, nargs="+", default=[1.0, 1.25, 1.5, 1.75])
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--crossover", action="store_true",
                    help="direct / sampled / default dispatch over widths x row counts instead")
    ap.add_argument("--row-counts", type=int, nargs="+", default=list(W.C4_ROWS))
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("the ablation harness needs a GPU", file=sys.stderr)
        return 2
    if args.crossover:
        return crossover(args)
    K = 2048
    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    for n in args.widths:
        w = W.get(f"c4_n{n}_m{args.rows}")
        window, lengths = W.make_window(w, dev)
        groups = [(window[g * w.M:(g + 1) * w.M], lengths[g * w.M:(g + 1) * w.M].contiguous())
                  for g in range(w.groups)]
        outs = [torch.empty((w.M, K), dtype=torch.int32, device=dev) for _ in groups]
        tk.reserve(w.M, w.n_alloc, K)
        # "auto" is the library's own choice at the method's stride and targets: direct
        # up to 16K, above that the sampled path with element-wise sampling (line
        # sampling, which the forced sampled path uses at stride 128, is reserved for
        # the longest rows).
        # rho_a: the admission target of element-sampled rows (0: admission at tau1, the
        # pages' design; the library's default admits down to 2.25 K).
        settings = [("direct", 128, 1.5, 1.75, 2.25), ("auto", 128, 1.5, 1.75, 2.25), ("auto", 128, 1.5, 1.75, 0.0)]
        settings += [("sampled", s, r, r + 0.25, 2.25) for s in args.strides for r in args.rho0]
        paths = {"direct": tk.PATH_DIRECT, "auto": tk.PATH_AUTO, "sampled": tk.PATH_SAMPLED}
        for mode, stride, rho0, rho1, rho_a in settings:
            path = paths[mode]
            with tk.path_override(path), tk.proposal(stride, rho0, rho1), tk.admission(rho_a):
                tk.reset_stats()
                for g, (s, l) in enumerate(groups):
                    tk.topk_exact(s, l, K=K, out=outs[g])
                torch.cuda.synchronize()
                st = tk.get_stats()
                ms = _time_call(groups, outs, K, args.steps, stream)
            rows = max(st["rows"], 1)
            print(json.dumps({
                "workload": w.name, "mode": mode, "stride": stride, "rho0": rho0, "rho1": rho1, "rho_a": rho_a,
                "median_call_ms": round(ms, 5), "rows_per_s": round(w.M / ms * 1e3),
                "tau0_rate": st["tau0"] / rows, "tau1_rate": st["tau1"] / rows, "tau_a_rate": st["tau_a"] / rows,
                "recovery_rate": (st["recover_under"] + st["recover_over"]) / rows,
                "long_exact_rate": st["long_exact"] / rows,
            }), flush=True)
        del window, lengths, groups, outs
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
