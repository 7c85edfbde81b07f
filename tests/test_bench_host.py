"""Host-side logic of bench.py (no GPU): the counter summarizer that turns two rocprofv3
--pmc runs into the traffic figure, and the torch-side contract gate of the timed calls."""
import argparse
import csv
import json
import os

import numpy as np
import torch

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, value in rows:
            r = {k: 0 for k in FIELDS}
            r.update(Dispatch_Id=disp, Kernel_Name=name, Counter_Name=counter, Counter_Value=value)
            w.writerow(r)


def test_summarize_counters_scales_by_the_copy(tmp_path):
    # Three 1 GiB calibration copies first; FETCH_SIZE reads half the copy's bytes (x2 scale),
    # WRITE_SIZE all of them (x1). Selector dispatches read 1000 and 1200 KiB raw (mean 1100),
    # a later large torch copy and an unrelated kernel must be ignored.
    copy = "__amd_rocclr_copyBuffer"
    sel = "void (anonymous namespace)::topk_rows_kernel<true>((anonymous namespace)::Params)"
    fetch = [(2, copy, 524288.0), (3, copy, 524290.0), (4, copy, 524286.0), (5, "other_kernel", 9e9),
             (6, sel, 1000.0), (7, copy, 262144.0), (8, sel, 1200.0)]
    write = [(2, copy, 1048576.0), (3, copy, 1048576.0), (4, copy, 1048576.0), (6, sel, 10.0), (8, sel, 30.0)]
    _write_run(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_run(str(tmp_path / "w"), "WRITE_SIZE", write)
    args = argparse.Namespace(workload="c3b", summarize_counters=[str(tmp_path / "f"), str(tmp_path / "w")])
    assert bench.summarize_counters(args, out_dir=str(tmp_path)) == 0
    out = json.load(open(tmp_path / "hbm_traffic_c3b.json"))
    assert out["kernel"] == "topk_rows_kernel<true>"
    assert out["fetch_dispatches"] == 2 and out["write_dispatches"] == 2
    assert abs(out["fetch_scale"] - 2.0) < 1e-5 and out["write_scale"] == 1.0
    assert abs(out["fetch_bytes"] - 1100.0 * 2.0 * 1024) < 1.0
    assert out["write_bytes"] == 20.0 * 1024
    assert out["kernel_source_digest"] == bench.kernel_source_digest("selector")


def test_gate_rows_flags_each_violation():
    K, L = 4, 12
    scores = torch.arange(L, dtype=torch.float32).reshape(1, L).repeat(5, 1)
    lengths = torch.tensor([L, L, L, L, 3], dtype=torch.int32)
    good = torch.tensor([[11, 10, 9, 8]], dtype=torch.int32)
    outs = torch.cat([good,
                      torch.tensor([[11, 10, 9, 7]], dtype=torch.int32),     # boundary violated
                      torch.tensor([[11, 10, 9, 9]], dtype=torch.int32),     # duplicate
                      torch.tensor([[11, 10, 9, 12]], dtype=torch.int32),    # past the length
                      torch.tensor([[2, 0, 1, -1]], dtype=torch.int32)])     # short row, valid
    assert bench.gate_rows(scores, lengths, outs, K, -1, [0]) == 0
    assert bench.gate_rows(scores, lengths, outs, K, -1, [1]) == 1
    assert bench.gate_rows(scores, lengths, outs, K, -1, [2]) == 1
    assert bench.gate_rows(scores, lengths, outs, K, -1, [3]) == 1
    assert bench.gate_rows(scores, lengths, outs, K, -1, [4]) == 0
    bad_short = outs.clone()
    bad_short[4, 3] = 5
    assert bench.gate_rows(scores, lengths, bad_short, K, -1, [4]) == 1


def test_order_keys_follow_total_order():
    x = torch.tensor([-np.inf, -1.0, -0.0, 0.0, 1e-45, 1.0, np.inf], dtype=torch.float32)
    k = bench.order_keys(x)
    assert bool((k[1:] > k[:-1]).all())
