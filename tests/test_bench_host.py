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
    # WRITE_SIZE all of them (x1). Two calls: selector dispatches read 1000 and 1200 KiB raw,
    # the recovery kernels after them 10 + 20 + 30 KiB once; a later large torch copy and an
    # unrelated kernel must be ignored.
    copy = "__amd_rocclr_copyBuffer"
    sel = "void (anonymous namespace)::topk_rows_kernel<true>((anonymous namespace)::Params)"
    rec = "(anonymous namespace)::recovery_%s_kernel((anonymous namespace)::Params)"
    fetch = [(2, copy, 524288.0), (3, copy, 524290.0), (4, copy, 524286.0), (5, "other_kernel", 9e9),
             (6, sel, 1000.0), (7, rec % "hist", 10.0), (8, rec % "collect", 20.0), (9, rec % "finish", 30.0),
             (10, copy, 262144.0), (11, sel, 1200.0), (12, rec % "hist", 0.0)]
    write = [(2, copy, 1048576.0), (3, copy, 1048576.0), (4, copy, 1048576.0), (6, sel, 10.0), (11, sel, 30.0),
             (8, rec % "collect", 4.0)]
    _write_run(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _write_run(str(tmp_path / "w"), "WRITE_SIZE", write)
    args = argparse.Namespace(workload="c3b", summarize_counters=[str(tmp_path / "f"), str(tmp_path / "w")])
    assert bench.summarize_counters(args, out_dir=str(tmp_path)) == 0
    out = json.load(open(tmp_path / "hbm_traffic_c3b.json"))
    assert out["kernel"] == ("recovery_collect_kernel + recovery_finish_kernel + recovery_hist_kernel + "
                             "topk_rows_kernel<true>")
    assert out["fetch_calls"] == 2 and out["write_calls"] == 2
    assert abs(out["fetch_scale"] - 2.0) < 1e-5 and out["write_scale"] == 1.0
    assert abs(out["fetch_bytes"] - (2200.0 + 60.0) / 2 * 2.0 * 1024) < 1.0
    assert out["write_bytes"] == 22.0 * 1024
    assert abs(out["selector_bytes_per_launch"] - (1100.0 * 2.0 + 20.0) * 1024) < 1.0
    assert abs(out["bytes_per_launch"] - ((1130.0 * 2.0) + 22.0) * 1024) < 1.0
    assert out["kernel_source_digest"] == bench.kernel_source_digest("selector")


def test_summarize_trace_groups_calls(tmp_path):
    # Two calls (selector + three recovery kernels each) with a probe kernel between them.
    d = tmp_path / "t"
    d.mkdir()
    sel = "void (anonymous namespace)::topk_rows_kernel<false>((anonymous namespace)::Params)"
    rec = "(anonymous namespace)::recovery_%s_kernel((anonymous namespace)::Params)"
    rows = [(100, 200, sel), (210, 220, rec % "hist"), (220, 240, rec % "collect"), (240, 250, rec % "finish"),
            (300, 330, "(anonymous namespace)::stream_read_probe_kernel(float const*, unsigned long, float*)"),
            (400, 520, sel), (530, 540, rec % "hist"), (540, 560, rec % "collect"), (560, 580, rec % "finish")]
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for a, b, n in rows:
            w.writerow([n, a, b])
    out = bench.summarize_trace(str(d))
    assert out["call_spans"]["calls"] == 2
    assert out["call_spans"]["mean_ns"] == (150 + 180) / 2
    k = out["kernels"]["topk_rows_kernel<false>"]
    assert k["calls"] == 2 and k["average_ns"] == 110 and k["min_ns"] == 100 and k["max_ns"] == 120
    assert out["kernels"]["recovery_finish_kernel"]["average_ns"] == 15


def test_protocol_defaults_and_overrides():
    a = bench.parse([])
    assert (a.warmup, a.condition, a.steps, a.calls_per_graph, a.workload) == (10, 100, 700, 1, "c3b")
    b = bench.parse(["--steps", "20", "--warmup", "5", "--workload", "c0"])
    assert (b.warmup, b.condition, b.steps, b.calls_per_graph) == (5, 100, 20, 100)
    c = bench.parse(["--protocol", "quick"])
    assert (c.warmup, c.condition, c.steps) == (5, 20, 40)


def test_phase_summary_medians_per_path():
    # Clock at 100 MHz (10 ns per tick). Call 1: a tau0 row (sample 2 us, proposal 1 us, pass
    # 10 us, refine 1 us), a tau1 row, a row recovered in place (6 us after its end) and an
    # empty record; call 2: one tau0 row and a queued row recovered 20 us after its end.
    def row(start, sampled, proposed, passed, end, recovered, code, c1=3000):
        return [start, sampled, proposed, passed, end, recovered, code | (3 << 8) | (77 << 32), c1 | (2900 << 32)]
    call1 = [row(1000, 1200, 1300, 2300, 2400, 0, 3), row(1000, 1250, 1350, 2350, 2500, 0, 4),
             row(1100, 1300, 1400, 2400, 2400, 3000, 5, 1800), [0] * 8]
    call2 = [row(0, 200, 300, 1300, 1400, 0, 3), row(0, 200, 300, 1300, 1300, 3300, 6, 1500)]
    out = bench.phase_summary([call1, call2], khz=100_000)
    p = out["paths"]
    assert p["tau0"]["rows"] == 2 and abs(p["tau0"]["median_sample_us"] - 2.0) < 1e-9
    assert abs(p["tau0"]["median_proposal_us"] - 1.0) < 1e-9 and abs(p["tau0"]["median_pass_us"] - 10.0) < 1e-9
    assert abs(p["tau0"]["median_refine_commit_us"] - 1.0) < 1e-9 and abs(p["tau0"]["median_row_us"] - 14.0) < 1e-9
    assert p["tau1"]["rows"] == 1 and abs(p["tau1"]["median_row_us"] - 15.0) < 1e-9
    assert abs(p["recover_inplace"]["median_recovery_us"] - 6.0) < 1e-9
    assert abs(p["recover_queued"]["median_recovery_us"] - 20.0) < 1e-9 and p["recover_queued"]["median_c_tau1"] == 1500
    assert out["calls"] == 2
    # call 1: first start 1000, last end 2500 -> 15 us; call 2: last end 1400 -> 14 us
    assert abs(out["median_last_end_us"] - 14.5) < 1e-9
    assert abs(out["median_last_recovered_us"] - (20.0 + 33.0) / 2) < 1e-9


def test_device_checksum_is_a_64_bit_pattern_sum():
    x = torch.tensor([[1.0, -2.0], [float("-inf"), 0.5]], dtype=torch.float32)
    u = x.view(torch.int32).to(torch.int64)
    assert bench.device_checksum(x) == f"{int(u.sum()) & 0xFFFFFFFFFFFFFFFF:016x}"
    y = x.clone()
    y[1, 1] = 0.25
    assert bench.device_checksum(y) != bench.device_checksum(x)
    assert bench.device_checksum(torch.tensor([3, 4], dtype=torch.int32)) == f"{7:016x}"


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


def test_more_than_one_gpu_is_refused(capsys):
    # The selector runs on one GPU: --gpus N > 1 prints one JSON line saying so and exits 2.
    assert bench.main(["--gpus", "2"]) == 2
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["n_gpus_requested"] == 2 and "one GPU" in line["error"]


def test_path_model_line():
    # Measured rows short of K at tau0 / tau1 from the counters, beside the model's
    # expectations; none for bf16-rounded windows (ties) or calls without sampled rows.
    from exact_top_selection_stride_amd import path_model as PM
    from exact_top_selection_stride_amd import workloads as W
    lengths = torch.tensor([131072 - 8192 + r + 1 for r in range(0, 8192, 512)], dtype=torch.int32)
    st = {"sampled": 16, "tau1": 3, "tau_a": 1, "recover_under": 1}
    d = bench.path_model_line(W.get("c1"), st, lengths, 2048)
    e0, e1 = PM.expected_short_rows(lengths.tolist(), 2048)
    assert d == {"rows_short_at_tau0": 5, "model_rows_short_at_tau0": round(e0, 1),
                 "rows_short_at_tau1": 2, "model_rows_short_at_tau1": round(e1, 1)}
    assert bench.path_model_line(W.get("c4_n65536_m8192"), st, lengths, 2048) is None
    assert bench.path_model_line(W.get("c1"), dict(st, sampled=0), lengths, 2048) is None
