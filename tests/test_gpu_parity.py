"""GPU parity: the HIP selector against the CPU oracle, bit-exact under the set
contract (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section
"什么叫精确，时间怎么量"): distinct in-prefix indices; for L > K exactly K of
them with min(selected) >= max(unselected) and the sorted selected key multiset
equal to the oracle's bit for bit; for L <= K all valid indices then the
sentinel. Integer work, so the bar is 0 mismatches.

All calls go through the C ABI via the ctypes binding.
"""
import numpy as np
import pytest
import torch

import oracle
import exact_top_selection_stride_amd as tk
from exact_top_selection_stride_amd import path_model as PM
from exact_top_selection_stride_amd import workloads as W

pytestmark = pytest.mark.gpu

K = 2048
DEV = "cuda"


def _check(scores, lengths, out, K=K, sentinel=-1, label=""):
    """Contract + oracle multiset check on host copies; returns the oracle output."""
    s = scores.detach().cpu().numpy()
    L = lengths.detach().cpu().numpy().astype(np.int32)
    o = out.detach().cpu().numpy()
    ref = oracle.topk(s, L, K, sentinel)
    n_bad, status = oracle.check_contract(s, L, K, sentinel, o, ref)
    if n_bad:
        bad = np.nonzero(status)[0][:10]
        detail = [(int(r), oracle.CHK_NAMES[int(status[r])], int(L[r])) for r in bad]
        pytest.fail(f"{label}: {n_bad} rows violate the contract, first: {detail}")
    return ref


def _run(scores, lengths, K=K, sentinel=-1, mode=tk.PATH_AUTO):
    tk.set_path_override(mode)
    try:
        tk.reset_stats()
        out = tk.topk_exact(scores, lengths, K=K, sentinel=sentinel)
        torch.cuda.synchronize()
        stats = tk.get_stats()
    finally:
        tk.set_path_override(tk.PATH_AUTO)
    return out, stats


def _window_rows(name, rows):
    """Rows of a workload's causal window, generated on the GPU, gathered by index."""
    w = W.get(name)
    out_s, out_l = [], []
    for r0, n in rows:
        s, l = W.make_window(w, DEV, row_start=r0, n_rows=n)
        out_s.append(s)
        out_l.append(l)
    return torch.cat(out_s).contiguous(), torch.cat(out_l).contiguous()


# ----------------------------------------------------------------- configs


def test_c0_full():
    w = W.get("c0")
    s, l = W.make_window(w, DEV)
    out, st = _run(s, l)
    _check(s, l, out, label="c0")
    n_short = int((l <= K).sum())
    assert st["rows"] == 256 and st["sentinel"] == n_short and st["direct"] == 256 - n_short


# Reduced-row windows, run in the execution mode their configuration takes at its full
# size (a few rows alone would be row-split by the automatic choice); the full-size
# launches, every row, are in test_gpu_configs.py.

def test_c1_rows():
    s, l = _window_rows("c1", [(0, 24), (4000, 8), (8192 - 32, 32)])
    with tk.execution(tk.EXEC_ROW_PER_WG):
        out, st = _run(s, l)
    _check(s, l, out, label="c1")
    assert st["sampled"] == 64 and st["row_per_wg"] == 64 and st["rowsplit"] == 0
    assert st["tau0"] + st["tau1"] + st["tau_a"] + st["recover_under"] + st["recover_over"] == 64


def test_c2_rows():
    s, l = _window_rows("c2", [(0, 6), (8192 - 6, 6)])
    with tk.execution(tk.EXEC_PERSISTENT):
        out, st = _run(s, l)
    _check(s, l, out, label="c2")
    assert st["sampled"] == 12 and st["persistent"] == 12 and st["rowsplit"] == 0


def test_c3_rows():
    s, l = _window_rows("c3b", [(0, 3), (5000, 2), (8192 - 3, 3)])
    with tk.execution(tk.EXEC_PERSISTENT):
        out, st = _run(s, l)
    _check(s, l, out, label="c3")
    assert st["sampled"] == 8 and st["persistent"] == 8 and st["rowsplit"] == 0


@pytest.mark.parametrize("n_alloc", W.C4_WIDTHS)
def test_c4_bf16_ties(n_alloc):
    s, l = _window_rows(f"c4_n{n_alloc}_m512", [(0, 20), (8192 - 20, 20)])
    with tk.execution(tk.EXEC_ROW_PER_WG):
        out, st = _run(s, l)
    _check(s, l, out, label=f"c4 n={n_alloc}")
    assert st["rows"] == 40 and st["row_per_wg"] == 40 and st["rowsplit"] == 0


# ------------------------------------------------------------ path forcing


def _sample_positions(L, stride=128):
    return np.arange(0, L, stride)


def _adversarial_row(L, n_mid, seed, n_a=0):
    """Row of length L whose stride-128 sample ranks put tau0 at 100, tau1 at 50 and the
    deeper admission rank tau_a at 45 (ranks 24, 28 and 36 of 1024 samples at L = 131072;
    samples of ranks 29-40 hold 45, the rest 0), with n_mid non-sample entries at 75,
    n_a at 47 (between tau_a and tau1) and everything else below 40:
    C(tau0) = 24, C(tau1) = 28 + n_mid, C(tau_a) = 40 + n_mid + n_a."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(0.0, 40.0, size=L).astype(np.float32)
    sp = _sample_positions(L)
    x[sp] = 0.0
    pick = rng.permutation(len(sp))
    x[sp[pick[:24]]] = 100.0
    x[sp[pick[24:28]]] = 50.0
    x[sp[pick[28:40]]] = 45.0
    non_sample = np.setdiff1d(np.arange(L), sp)
    chosen = rng.choice(non_sample, size=n_mid + n_a, replace=False)
    x[chosen[:n_mid]] = 75.0
    x[chosen[n_mid:]] = 47.0
    return x


def test_forced_tau1_fallback():
    L = 131072
    rows = np.stack([_adversarial_row(L, 2030, seed) for seed in range(4)])
    s = torch.from_numpy(rows).to(DEV)
    l = torch.full((4,), L, dtype=torch.int32, device=DEV)
    out, st = _run(s, l)
    _check(s, l, out, label="tau1 fallback")
    assert st["tau1"] == 4 and st["tau0"] == 0 and st["recover_under"] == 0


@pytest.mark.parametrize("execution", [tk.EXEC_AUTO, tk.EXEC_ROW_PER_WG])
def test_forced_exact_recovery_underfill(execution):
    # Auto dispatch row-splits 4 rows (admission at tau1); one workgroup per row admits
    # down to tau_a, which underfills too, and recovers the rows in place (rows sampled
    # element by element are recovered by their own workgroup at any length).
    L = 131072
    rows = np.stack([_adversarial_row(L, 1000, 10 + seed) for seed in range(4)])
    s = torch.from_numpy(rows).to(DEV)
    l = torch.full((4,), L, dtype=torch.int32, device=DEV)
    with tk.execution(execution):
        out, st = _run(s, l)
    _check(s, l, out, label="underfill recovery")
    assert st["recover_under"] == 4
    if execution == tk.EXEC_ROW_PER_WG:
        assert st["recover_inplace"] == 4 and st["queued"] == 0


@pytest.mark.parametrize("execution", [tk.EXEC_ROW_PER_WG, tk.EXEC_PERSISTENT])
def test_deeper_admission_rescues_tau1_underfill(execution):
    # C(tau1) = 1028 < K <= C(tau_a) = 2540: certified at the deeper admission rank in the
    # one pass; with the deeper admission off (every row admits at tau1, the pages' design)
    # the same rows underfill and take exact recovery. Both results are exact.
    L = 131072
    rows = np.stack([_adversarial_row(L, 1000, 20 + seed, n_a=1500) for seed in range(4)])
    s = torch.from_numpy(rows).to(DEV)
    l = torch.full((4,), L, dtype=torch.int32, device=DEV)
    with tk.execution(execution):
        out, st = _run(s, l)
        _check(s, l, out, label="tau_a rescue")
        assert st["tau_a"] == 4 and st["tau1"] == 0 and st["recover_under"] == 0
        with tk.admission(0):
            out, st = _run(s, l)
        _check(s, l, out, label="tau_a off")
        assert st["recover_under"] == 4 and st["tau_a"] == 0


def test_forced_overflow_recovery_negative_threshold():
    # Samples at -1000 make tau0 = tau1 negative (unsigned admission compare) and
    # admit every entry: the candidate buffer overflows and recovery runs; the 50s tie.
    L = 131072
    x = np.full((2, L), 50.0, dtype=np.float32)
    x[:, _sample_positions(L)] = -1000.0
    s = torch.from_numpy(x).to(DEV)
    l = torch.tensor([L, L - 5], dtype=torch.int32, device=DEV)
    out, st = _run(s, l)
    _check(s, l, out, label="overflow")
    assert st["recover_over"] == 2


def test_sentinel_lengths():
    N = 4096
    s = torch.randn(6, N, device=DEV)
    l = torch.tensor([0, 1, K - 1, K, K + 1, N], dtype=torch.int32, device=DEV)
    for sentinel in (-1, N, -12345):
        out, st = _run(s, l, sentinel=sentinel)
        _check(s, l, out, sentinel=sentinel, label="sentinel")
        assert st["sentinel"] == 4
        o = out.cpu()
        assert torch.all(o[0] == sentinel) and o[1, 0] == 0 and torch.all(o[1, 1:] == sentinel)


@pytest.mark.parametrize("mode", [tk.PATH_SAMPLED, tk.PATH_DIRECT, tk.PATH_RECOVERY, tk.PATH_ROWSPLIT])
def test_forced_modes_on_short_and_long_rows(mode):
    s0, l0 = W.make_window(W.get("c0"), DEV)
    out, st = _run(s0, l0, mode=mode)
    _check(s0, l0, out, label=f"c0 mode {mode}")
    s1, l1 = _window_rows("c1", [(100, 6)])
    out, st = _run(s1, l1, mode=mode)
    _check(s1, l1, out, label=f"c1 mode {mode}")


def test_cooperative_recovery_queue_and_overflow():
    # Forced recovery queues rows for the cooperative recovery kernels; past the
    # queue's capacity (256 rows per call) rows are recovered in place.
    N = 20000
    for M in (5, 256, 300):
        s, l = W.make_rows(M, N, [N - (i % 7) for i in range(M)], tail_p=0.01, seed=M, device=DEV)
        out, st = _run(s, l, mode=tk.PATH_RECOVERY)
        _check(s, l, out, label=f"recovery M={M}")
        assert st["forced_recovery"] == M
        assert st["queued"] == min(M, 256)


def test_recovery_rows_mixed_with_normal_rows():
    # Underfilling rows (queued) between ordinary sampled rows of one call.
    L = 131072
    adv = np.stack([_adversarial_row(L, 1000, 40 + i) for i in range(3)])
    s1, l1 = _window_rows("c1", [(0, 5)])
    s = torch.cat([s1[:, :L], torch.from_numpy(adv).to(DEV)]).contiguous()
    l = torch.cat([l1.clamp(max=L), torch.full((3,), L, dtype=torch.int32, device=DEV)]).contiguous()
    out, st = _run(s, l)
    _check(s, l, out, label="mixed recovery")
    # Rows of 128K are recovered in place by their own workgroup; nothing is queued.
    assert st["recover_under"] >= 3 and st["recover_inplace"] >= 3 and st["queued"] == 0


def _controlled_row(L, kind, seed):
    """Rows of L = 65536 (512 samples; sample ranks r0 = 24, r1 = 28, r_a = 36 and
    r2 = 46 at the method's targets, as for any L that is a multiple of 128) that take
    each branch of in-place exact recovery:
      under_certified  tau1 = 50 and tau_a = 45 underfill (1028 and 1040 keys) but the
                       deeper tau2 = 40 holds 4046 keys: one more pass certifies;
      under_full       tau1 and tau_a underfill and every key below them is >= tau2 = 0:
                       the second pass overflows, the exact full-row select runs;
      over_certified   9028 keys >= tau1 = 50 (overflow), spread over distinct values: the
                       boundary bin of the pass histogram bounds a second pass;
      over_full        9000 copies of one value above tau1: the boundary bin alone exceeds
                       the buffer, the exact full-row select runs."""
    rng = np.random.default_rng(seed)
    sp = _sample_positions(L)
    rest = np.setdiff1d(np.arange(L), sp)
    pick = rng.permutation(len(sp))
    x = rng.uniform(0.0, 30.0, size=L).astype(np.float32)
    x[sp] = 0.0
    x[sp[pick[:24]]] = 100.0
    x[sp[pick[24:28]]] = 50.0
    if kind == "under_certified":
        x[sp[pick[28:40]]] = 45.0
        x[sp[pick[40:46]]] = 40.0
        chosen = rng.choice(rest, size=4000, replace=False)
        x[chosen[:1000]] = 75.0
        x[chosen[1000:]] = 42.0
    elif kind == "under_full":
        x = rng.uniform(0.0, 40.0, size=L).astype(np.float32)
        x[sp] = 0.0
        x[sp[pick[:24]]] = 100.0
        x[sp[pick[24:28]]] = 50.0
        x[sp[pick[28:40]]] = 45.0
        x[rng.choice(rest, size=1000, replace=False)] = 75.0
    elif kind == "over_certified":
        x[rng.choice(rest, size=9000, replace=False)] = rng.uniform(55.0, 95.0, size=9000).astype(np.float32)
    else:
        x[rng.choice(rest, size=9000, replace=False)] = 60.0
    return x


@pytest.mark.parametrize("execution", [tk.EXEC_ROW_PER_WG, tk.EXEC_PERSISTENT, tk.EXEC_ROWSPLIT])
def test_inplace_recovery_branches(execution):
    # Each in-place recovery branch on rows built from the known sample positions, in
    # every execution mode (row-split recovers in its finish kernel); the counters prove
    # which branch ran, the oracle that the result is exact.
    L = 65536
    kinds = ["under_certified", "under_full", "over_certified", "over_full"]
    rows = np.stack([_controlled_row(L, k, 300 + i) for i, k in enumerate(kinds)])
    s = torch.from_numpy(rows).to(DEV)
    l = torch.full((4,), L, dtype=torch.int32, device=DEV)
    with tk.execution(execution):
        out, st = _run(s, l)
    _check(s, l, out, label=f"in-place recovery branches, execution {execution}")
    assert st["recover_under"] == 2 and st["recover_over"] == 2
    assert st["recover_inplace"] == 4 and st["queued"] == 0
    assert st["inplace_certified"] == 2 and st["inplace_full"] == 2


# ---------------------------------------------------- inputs and edge cases


@pytest.mark.parametrize("n_alloc", [8191, 16387, 131071, 131073])
def test_unaligned_rows(n_alloc):
    # Odd N_alloc misaligns every other row start; lengths cover all residues mod 4.
    M = 16
    lengths = [n_alloc - i for i in range(M)]
    s, l = W.make_rows(M, n_alloc, lengths, tail_p=0.01, seed=n_alloc, device=DEV)
    out, st = _run(s, l)
    _check(s, l, out, label=f"unaligned {n_alloc}")
    for mode in (tk.PATH_SAMPLED, tk.PATH_RECOVERY):
        out, st = _run(s, l, mode=mode)
        _check(s, l, out, label=f"unaligned {n_alloc} mode {mode}")


@pytest.mark.parametrize("fill", [float("inf"), float("nan"), 1e30])
def test_suffix_is_never_read(fill):
    w = W.get("c1")
    s, l = W.make_window(w, DEV, row_start=0, n_rows=8)
    s2 = s.clone()
    cols = torch.arange(s.shape[1], device=DEV)
    s2[cols[None, :] >= l[:, None]] = fill
    out, _ = _run(s2, l)
    _check(s2, l, out, label=f"suffix {fill}")
    s0, l0 = W.make_window(W.get("c0"), DEV)
    s0[torch.arange(s0.shape[1], device=DEV)[None, :] >= l0[:, None]] = fill
    out, _ = _run(s0, l0)
    _check(s0, l0, out, label=f"suffix c0 {fill}")


@pytest.mark.parametrize("kind", ["negative", "mixed_sign", "signed_zero", "all_equal", "neg_inf_prefix",
                                  "small_ints"])
def test_value_edge_cases(kind):
    g = torch.Generator(device=DEV).manual_seed(77)
    M, N = 9, 140000
    if kind == "negative":
        s = torch.randn(M, N, device=DEV, generator=g) * 2.5 - 30.0
    elif kind == "mixed_sign":
        s = torch.randn(M, N, device=DEV, generator=g)
    elif kind == "signed_zero":
        s = torch.where(torch.rand(M, N, device=DEV, generator=g) < 0.5, 0.0, -0.0)
        s[:, :100] = 1.0
    elif kind == "all_equal":
        s = torch.full((M, N), 3.25, device=DEV)
    elif kind == "neg_inf_prefix":
        s = torch.randn(M, N, device=DEV, generator=g)
        s[torch.rand(M, N, device=DEV, generator=g) < 0.995] = float("-inf")
    else:
        s = torch.randint(0, 8, (M, N), device=DEV, generator=g).float()
    # Long rows (sampled / full-row exact) and short ones (the LDS-staged direct path).
    l = torch.tensor([N, N - 1, N - 2, N - 3, 70000, 20000, 16384, 9000, 3000], dtype=torch.int32, device=DEV)
    for mode in (tk.PATH_AUTO, tk.PATH_SAMPLED, tk.PATH_DIRECT, tk.PATH_RECOVERY):
        out, _ = _run(s, l, mode=mode)
        _check(s, l, out, label=f"{kind} mode {mode}")


@pytest.mark.parametrize("Ksmall", [1, 7, 64, 1000, 2047, 3000, 4096])
def test_other_k(Ksmall):
    s, l = _window_rows("c1", [(0, 4)])
    s0, l0 = W.make_window(W.get("c0"), DEV)
    for ss, ll in ((s, l), (s0, l0)):
        out, _ = _run(ss, ll, K=Ksmall)
        _check(ss, ll, out, K=Ksmall, label=f"K={Ksmall}")


@pytest.mark.parametrize("execution", [tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG, tk.EXEC_ROWSPLIT])
def test_execution_modes_agree_with_oracle(execution):
    # Both row-to-workgroup mappings on short, medium and long rows, with recovery rows.
    cases = [W.make_window(W.get("c0"), DEV), _window_rows("c1", [(0, 12), (8000, 12)]),
             _window_rows("c3b", [(10, 3)]), _window_rows("c4_n16384_m512", [(0, 30)])]
    L = 131072
    adv = torch.from_numpy(np.stack([_adversarial_row(L, 1000, 70 + i) for i in range(2)])).to(DEV)
    cases.append((adv, torch.full((2,), L, dtype=torch.int32, device=DEV)))
    with tk.execution(execution):
        for s, l in cases:
            out, st = _run(s, l)
            _check(s, l, out, label=f"execution {execution} shape {tuple(s.shape)}")


def test_rowsplit_merges_segments():
    # Row-split on long rows (several workgroups per row), with a forced underfill
    # row, an overflow row with a negative threshold, a long unaligned row and a
    # short row taken whole; the stats prove the split kernels ran.
    L = 131072
    rows = [_adversarial_row(L, 1000, 90), _adversarial_row(L, 2030, 91)]
    ovf = np.full(L, 50.0, dtype=np.float32)
    ovf[_sample_positions(L)] = -1000.0
    rows.append(ovf)
    s1, l1 = _window_rows("c1", [(3, 4)])
    s = torch.cat([torch.from_numpy(np.stack(rows)).to(DEV), s1]).contiguous()
    l = torch.cat([torch.full((3,), L, dtype=torch.int32, device=DEV), l1]).contiguous()
    l[4] = 5000  # short row: direct path, taken whole
    with tk.execution(tk.EXEC_ROWSPLIT):
        out, st = _run(s, l)
    _check(s, l, out, label="row-split mix")
    assert st["rowsplit"] == 6 and st["direct"] == 1
    assert st["recover_under"] >= 1 and st["recover_over"] >= 1 and st["tau1"] >= 1
    s3, l3 = _window_rows("c3b", [(0, 4)])
    for n_alloc in (1048576, 1048575):
        ss = s3[:, :n_alloc].contiguous()
        ll = l3.clamp(max=n_alloc).contiguous()
        with tk.execution(tk.EXEC_ROWSPLIT):
            out, st = _run(ss, ll)
        _check(ss, ll, out, label=f"row-split 1M n_alloc={n_alloc}")
        assert st["rowsplit"] == 4


@pytest.mark.parametrize("two_keys", [False, True])
def test_wide_boundary_bin_of_ties(two_keys):
    # 3000 copies of one value (or 1500 each of two adjacent floats) above a body below
    # 40: tau1 lands on them, so the boundary bin holds more keys than the frontier
    # buffer; with one key it is resolved as ties directly, with two by narrowing.
    L, rows = 65536, []
    for seed in range(4):
        rng = np.random.default_rng(500 + seed)
        x = rng.uniform(0.0, 40.0, size=L).astype(np.float32)
        pos = rng.choice(L, size=3000, replace=False)
        x[pos] = np.float32(50.0)
        if two_keys:
            x[pos[:1500]] = np.nextafter(np.float32(50.0), np.float32(60.0))
        rows.append(x)
    s = torch.from_numpy(np.stack(rows)).to(DEV)
    l = torch.full((4,), L, dtype=torch.int32, device=DEV)
    for mode in (tk.PATH_SAMPLED, tk.PATH_AUTO):
        for ex in (tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG):
            with tk.execution(ex):
                out, st = _run(s, l, mode=mode)
            _check(s, l, out, label=f"wide tie bin two_keys={two_keys} mode {mode} exec {ex}")
            if mode == tk.PATH_SAMPLED:
                assert st["frontier_wide"] == 4


def _random_case(seed):
    """A seeded random shape: width, rows, K, lengths (0, <= K, near the width) and one of
    several value families (continuous, bf16-rounded, few distinct values, signed)."""
    rng = np.random.default_rng(seed)
    n_alloc = int(rng.choice([3000, 8192, 20001, 65536, 131073, 300007]))
    M = int(rng.integers(1, 9))
    Kr = int(rng.choice([1, 64, 2048, 3000]))
    lens = rng.integers(0, n_alloc + 1, size=M)
    lens[rng.random(M) < 0.25] = n_alloc
    lens[rng.random(M) < 0.15] = min(Kr, n_alloc)
    family = seed % 4
    if family == 0:
        x = rng.normal(30.0, 2.5, size=(M, n_alloc)).astype(np.float32)
        tail = rng.random((M, n_alloc)) < 0.01
        x[tail] = (45.0 + rng.exponential(3.0, size=int(tail.sum()))).astype(np.float32)
    elif family == 1:
        x = torch.from_numpy(rng.normal(30.0, 2.5, size=(M, n_alloc)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    elif family == 2:
        x = rng.integers(0, 5, size=(M, n_alloc)).astype(np.float32)
    else:
        x = rng.standard_normal((M, n_alloc)).astype(np.float32) * np.float32(1e-3)
        x[:, ::7] = -x[:, ::7]
    cols = np.arange(n_alloc)[None, :]
    x[cols >= lens[:, None]] = -np.inf
    return (torch.from_numpy(x).to(DEV), torch.from_numpy(lens.astype(np.int32)).to(DEV), Kr, n_alloc)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_every_mode(seed):
    # Seeded random widths, row counts, K, lengths and value families, in every forced
    # path and every execution mode; each result is checked against the oracle.
    s, l, Kr, n_alloc = _random_case(seed)
    for execution in (tk.EXEC_AUTO, tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG, tk.EXEC_ROWSPLIT):
        for mode in (tk.PATH_AUTO, tk.PATH_SAMPLED, tk.PATH_DIRECT, tk.PATH_RECOVERY):
            with tk.execution(execution):
                out, st = _run(s, l, K=Kr, mode=mode)
            _check(s, l, out, K=Kr, label=f"seed {seed} n_alloc {n_alloc} M {s.shape[0]} K {Kr} exec {execution} mode {mode}")
            assert st["rows"] == s.shape[0]


@pytest.mark.parametrize("seed", range(8))
def test_random_larger_shapes_and_sorted(seed):
    # Seeded random larger calls: widths 16K-1M, up to 600 rows (64 at 512K and beyond),
    # K 512-4096, lengths from K/2 to the width; automatic, row-split and persistent
    # execution, and the sorted output, each checked against the oracle.
    rng = np.random.default_rng(5000 + seed)
    n_alloc = int(rng.choice([16385, 65536, 131072, 262147, 524288, 1048576]))
    M = int(rng.choice([1, 2, 5, 16, 63, 200, 513, 600]))
    if n_alloc >= 524288:
        M = min(M, 64)
    Kr = int(rng.choice([512, 1000, 2048, 4096]))
    lens = rng.integers(Kr // 2, n_alloc + 1, size=M)
    lens[rng.random(M) < 0.3] = n_alloc
    x = rng.normal(30.0, 2.5, size=(M, n_alloc)).astype(np.float32)
    tail = rng.random((M, n_alloc)) < 0.01
    x[tail] = (45.0 + rng.exponential(3.0, size=int(tail.sum()))).astype(np.float32)
    x[np.arange(n_alloc)[None, :] >= lens[:, None]] = -np.inf
    s = torch.from_numpy(x).to(DEV)
    l = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    label = f"seed {seed} n_alloc {n_alloc} M {M} K {Kr}"
    for execution in (tk.EXEC_AUTO, tk.EXEC_ROWSPLIT, tk.EXEC_PERSISTENT):
        with tk.execution(execution):
            out, st = _run(s, l, K=Kr)
        _check(s, l, out, K=Kr, label=f"{label} exec {execution}")
    idx, val = tk.topk_exact_sorted(s, l, K=Kr)
    torch.cuda.synchronize()
    _check_sorted(s, l, idx, val, Kr, label=f"{label} sorted")


def test_consecutive_calls_reuse_the_ticket():
    # Row tickets rewind after every call: calls of different M back to back.
    s, l = _window_rows("c1", [(0, 40)])
    with tk.execution(tk.EXEC_PERSISTENT):
        for M in (40, 3, 1, 17, 40):
            out = tk.topk_exact(s[:M], l[:M].contiguous(), K=K)
            torch.cuda.synchronize()
            _check(s[:M], l[:M], out, label=f"M={M}")


def test_stream_read_probe_sizes():
    # The measurement probe (one workgroup per 4 MiB chunk) on sizes below one chunk, with
    # a ragged tail, and over several chunks; it only has to run cleanly.
    sink = torch.zeros(4096, device=DEV)
    for n in (1, 3, 4, 1000, (1 << 20) + 5, 12 * (1 << 20) + 7):
        x = torch.randn(n, device=DEV)
        tk.stream_read_probe(x, sink)
        torch.cuda.synchronize()


def test_selector_timing_hook():
    # The hook's events bracket the selector kernels inside the call's own events.
    s, l = _window_rows("c1", [(0, 64)])
    stream = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    with torch.cuda.stream(stream):
        for e in ev:
            e.record(stream)
        torch.cuda.synchronize()
        tk.time_next_call(ev[1], ev[2])
        ev[0].record(stream)
        out = tk.topk_exact(s, l, K=K)
        ev[3].record(stream)
    torch.cuda.synchronize()
    _check(s, l, out, label="timed call")
    inner, outer = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < inner <= outer
    assert ev[0].elapsed_time(ev[1]) >= 0.0 and ev[2].elapsed_time(ev[3]) >= 0.0


def test_phase_recording_hook():
    # Per-row phase stamps: ordered in time, path codes matching the row counters, tau1
    # counts certified; disarmed calls write nothing. Admission at tau1 (the deeper
    # admission off), so that the underfilling rows take the cooperative recovery kernels.
    s, l = _window_rows("c1", [(0, 20)])
    L = 131072
    adv = torch.from_numpy(np.stack([_adversarial_row(L, 1000, 700 + i) for i in range(2)])).to(DEV)
    s = torch.cat([s, adv]).contiguous()
    l = torch.cat([l, torch.full((2,), L, dtype=torch.int32, device=DEV)]).contiguous()
    buf = torch.zeros((s.shape[0], 8), dtype=torch.int64, device=DEV)
    khz = tk.record_phases(buf)
    try:
        with tk.execution(tk.EXEC_ROW_PER_WG), tk.admission(0):
            out, st = _run(s, l)
    finally:
        tk.record_phases(None)
    _check(s, l, out, label="phase-recorded call")
    assert khz > 0
    rec = buf.cpu().numpy()
    codes = rec[:, 6] & 0xFF
    names = [tk.PATH_CODES.get(int(c)) for c in codes]
    assert names.count("tau0") == st["tau0"] and names.count("tau1") == st["tau1"]
    assert names.count("tau_a") == st["tau_a"]
    assert names.count("recover_queued") == st["queued"] >= 2
    for r, n in zip(rec, names):
        start, sampled, proposed, passed, end = (int(v) for v in r[:5])
        assert 0 < start <= sampled <= proposed <= passed <= end, n
        c1 = int(r[7]) & 0xFFFFFFFF
        if n in ("tau0", "tau1"):
            assert c1 >= K and r[5] == 0
        elif n == "tau_a":
            assert c1 < K and r[5] == 0
        else:
            assert c1 < K and int(r[5]) >= end  # recovered by the cooperative kernels after
    buf.zero_()
    _run(s, l)
    assert int(buf.abs().sum()) == 0


def _host_keys(row):
    """Order keys of float32 scores (sign flip of the bit pattern, all bits flipped for
    negatives): key order is score order."""
    u = row.view(np.uint32)
    return u ^ np.where(u >> 31 == 1, np.uint32(0xFFFFFFFF), np.uint32(0x80000000))


@pytest.mark.parametrize("name,rows,execution", [
    ("c1", [(0, 24), (4000, 24)], tk.EXEC_ROW_PER_WG),   # element sample, admission to tau_a
    ("c3a", [(0, 6), (8000, 6)], tk.EXEC_ROW_PER_WG),    # line sample, cold lines skipped
    ("c2", [(100, 4), (6000, 4)], tk.EXEC_AUTO),         # few 512K rows: row-split, line sample
    ("c1", [(10, 3), (7000, 3)], tk.EXEC_AUTO),          # few 128K rows: row-split, element sample
])
def test_threshold_counts_equal_sample_rank_counts(name, rows, execution):
    # Each certified row's recorded C(tau0) and C(tau1) equal, on the host, the number of the
    # row's keys at or above the r0-th and r1-th largest of its stride-128 sample keys, with
    # r = ceil(T n_s / L) for the targets T0 = 1.5 K and T1 = 1.75 K: the thresholds are the
    # sample ranks of the method, in every sampling mode and execution.
    s, l = _window_rows(name, rows)
    buf = torch.zeros((s.shape[0], 8), dtype=torch.int64, device=DEV)
    khz = tk.record_phases(buf)
    try:
        with tk.execution(execution):
            out, st = _run(s, l)
    finally:
        tk.record_phases(None)
    _check(s, l, out, label=f"{name} threshold counts")
    assert khz > 0
    rec = buf.cpu().numpy()
    sh, lh = s.cpu().numpy(), l.cpu().numpy()
    t0, t1 = PM.targets(K)
    checked = 0
    for i in range(s.shape[0]):
        code = int(rec[i, 6]) & 0x7F
        if tk.PATH_CODES.get(code) not in ("tau0", "tau1", "tau_a"):
            continue
        L = int(lh[i])
        keys = _host_keys(sh[i, :L])
        n_s = -(-L // 128)
        samp = np.sort(keys[::128][:n_s])[::-1]
        k0 = samp[PM.sample_rank(t0, n_s, L) - 1]
        k1 = samp[PM.sample_rank(t1, n_s, L) - 1]
        want = (int((keys >= k0).sum()), int((keys >= k1).sum()))
        got = (int(rec[i, 7]) >> 32, int(rec[i, 7]) & 0xFFFFFFFF)
        assert got == want, (name, i, L, got, want)
        checked += 1
    assert checked >= s.shape[0] - 2, (checked, st)


def test_graph_replay():
    s, l = _window_rows("c1", [(0, 12)])
    s0, l0 = W.make_window(W.get("c0"), DEV)
    tk.reserve(256, 131072, K)
    stream = torch.cuda.Stream()
    out_a = torch.empty((12, K), dtype=torch.int32, device=DEV)
    out_b = torch.empty((256, K), dtype=torch.int32, device=DEV)
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        tk.topk_exact(s, l, K=K, out=out_a)  # warm-up outside capture
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            tk.topk_exact(s, l, K=K, out=out_a)
            tk.topk_exact(s0, l0, K=K, out=out_b)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    ref_a = _check(s, l, out_a, label="graph warm-up")
    for rep in range(10):
        out_a.fill_(-7)
        out_b.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        _check(s, l, out_a, label=f"graph replay {rep} (c1)")
        _check(s0, l0, out_b, label=f"graph replay {rep} (c0)")
        # eager work between replays
        tk.topk_exact(s[:3], l[:3].contiguous(), K=K)
        torch.cuda.synchronize()


# ---------------------------------------------- full-size launch configurations


def _full_size_sampled_rows(name, group, rows):
    w = W.get(name)
    s, l = W.make_window(w, DEV, row_start=group * w.M, n_rows=w.M)
    out, st = _run(s, l)
    assert st["rows"] == w.M
    idx = torch.tensor(rows, device=DEV)
    _check(s[idx], l[idx], out[idx], label=f"{name} group {group} rows {rows}")
    return st


def test_full_size_c3b_sampled_rows():
    st = _full_size_sampled_rows("c3b", 0, [0, 1, 2047, 4096, 6000, 8190, 8191])
    assert st["sampled"] == 8192


def test_full_size_c2_sampled_rows():
    _full_size_sampled_rows("c2", 1, [0, 1000, 4095])


def test_full_size_c3a_sampled_rows():
    _full_size_sampled_rows("c3a", 15, [0, 255, 511])


def test_full_size_c3a_forced_rowsplit():
    # The 512 x 1M launch configuration through the row-split kernels (auto dispatch
    # keeps one workgroup per row there, which is faster on MI355X).
    with tk.execution(tk.EXEC_ROWSPLIT):
        st = _full_size_sampled_rows("c3a", 3, [0, 100, 511])
    assert st["rowsplit"] == 512


@pytest.mark.parametrize("name", [f"dec_n{n}_m{m}" for n in W.DECODE_WIDTHS for m in W.DECODE_ROWS])
def test_decode_shapes(name):
    # Few long rows: auto dispatch splits each row over several workgroups; every row
    # is checked against the oracle.
    w = W.get(name)
    s, l = W.make_window(w, DEV)
    out, st = _run(s, l)
    _check(s, l, out, label=name)
    assert st["rows"] == w.M and st["rowsplit"] == w.M


@pytest.mark.parametrize("K4", [4096])
def test_large_k_on_long_rows(K4):
    # K = 4096 on 1M rows in persistent and row-split execution: tau1 admits about
    # 1.75 K, so some rows overflow the candidate buffer and are recovered exactly.
    s, l = _window_rows("c3b", [(0, 4), (6000, 4)])
    for ex in (tk.EXEC_PERSISTENT, tk.EXEC_ROWSPLIT):
        with tk.execution(ex):
            out, st = _run(s, l, K=K4)
        _check(s, l, out, K=K4, label=f"K={K4} execution {ex}")
        assert st["rows"] == 8


@pytest.mark.parametrize("stride,rho0,rho1", [(16, 1.5, 1.75), (32, 1.75, 2.0), (64, 1.0, 1.25), (128, 1.0, 1.25),
                                             (128, 1.25, 1.5), (256, 1.5, 1.75), (1, 1.5, 1.75)])
def test_proposal_ablation_stays_exact(stride, rho0, rho1):
    # Any sample stride and candidate targets give the exact result; only the work and
    # the path rates change. 64K bf16 rows (ties), C1 rows and a few 1M rows, with the
    # sampled path forced on the short ones.
    cases = [(_window_rows("c4_n65536_m512", [(0, 24)]), tk.PATH_SAMPLED),
             (_window_rows("c1", [(0, 8), (8000, 8)]), tk.PATH_AUTO),
             (_window_rows("c3b", [(7, 2)]), tk.PATH_AUTO)]
    with tk.proposal(stride, rho0, rho1):
        for (s, l), mode in cases:
            for ex in (tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG):
                with tk.execution(ex):
                    out, st = _run(s, l, mode=mode)
                _check(s, l, out, label=f"stride {stride} rho {rho0}/{rho1} shape {tuple(s.shape)} exec {ex}")
                assert st["rows"] == s.shape[0]


def test_full_size_few_long_rows_take_rowsplit():
    # 64 rows of the 1M causal window: auto dispatch splits each row over several
    # workgroups (few rows per resident slot); sampled rows against the oracle.
    w = W.get("c3a")
    s, l = W.make_window(w, DEV, row_start=8192 - 64, n_rows=64)
    out, st = _run(s, l)
    assert st["rows"] == 64 and st["rowsplit"] == 64
    idx = torch.tensor([0, 31, 63], device=DEV)
    _check(s[idx], l[idx], out[idx], label="1M x 64 rows, row-split")


# ---------------------------------------------- memory safety and long replay runs

GUARD = 4096          # int32 guard words on each side of an output buffer
CANARY = 0x5A5A5A5A


def _guarded_out(M, K):
    buf = torch.full((M * K + 2 * GUARD,), CANARY, dtype=torch.int32, device=DEV)
    return buf, buf[GUARD:GUARD + M * K].view(M, K)


@pytest.mark.parametrize("seed", range(4))
def test_output_guard_canaries(seed):
    # The output view sits between two guard regions of canary words; no path or execution
    # mode may write outside [out, out + M * K).
    s, l, Kr, n_alloc = _random_case(100 + seed)
    M = s.shape[0]
    for execution in (tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG, tk.EXEC_ROWSPLIT):
        for mode in (tk.PATH_AUTO, tk.PATH_SAMPLED, tk.PATH_DIRECT, tk.PATH_RECOVERY):
            buf, out = _guarded_out(M, Kr)
            tk.set_path_override(mode)
            try:
                with tk.execution(execution):
                    tk.topk_exact(s, l, K=Kr, out=out)
                torch.cuda.synchronize()
            finally:
                tk.set_path_override(tk.PATH_AUTO)
            assert bool((buf[:GUARD] == CANARY).all()) and bool((buf[GUARD + M * Kr:] == CANARY).all()), \
                f"write outside the output: seed {seed} exec {execution} mode {mode}"
            _check(s, l, out, K=Kr, label=f"guarded seed {seed} exec {execution} mode {mode}")


def _sorted_selected_keys(scores, out):
    """Per-row sorted order keys of the selected scores (rows with L > K), on the GPU."""
    from bench import order_keys
    idx = out.to(torch.int64).clamp(min=0)
    keys = order_keys(torch.gather(scores, 1, idx))
    return torch.sort(keys, dim=1).values


def test_graph_replay_200():
    # One captured call replayed 200 times: the self-rewinding tickets, queues and counters
    # must give the same selected key multiset every time (compared on the GPU), and the
    # first and last replays pass the full oracle check. Rows include recovery rows.
    s, l = _window_rows("c1", [(0, 24)])
    s[3, : l[3]] = 1.0                          # all-equal row: ties at the boundary
    torch.manual_seed(0)
    s[5, : l[5]] = torch.randint(0, 3, (int(l[5]),), device=DEV).float()  # three values
    tk.reserve(24, s.shape[1], K)
    out = torch.empty((24, K), dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        tk.topk_exact(s, l, K=K, out=out)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            tk.topk_exact(s, l, K=K, out=out)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    _check(s, l, out, label="replay warm-up")
    ref = _sorted_selected_keys(s, out)
    for rep in range(200):
        out.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = _sorted_selected_keys(s, out)
        assert torch.equal(got, ref), f"replay {rep}: selected key multiset changed"
        assert int(torch.unique(out, dim=None).numel()) > K  # not a constant fill
    _check(s, l, out, label="replay 200")


_FRESH_PROCESS = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import exact_top_selection_stride_amd as tk
from exact_top_selection_stride_amd import workloads as W
import oracle
res = {}
s, l = W.make_rows(2, 131072, [131072, 100000], device="cuda")
out = torch.empty((2, 2048), dtype=torch.int32, device="cuda")
stream = torch.cuda.Stream()
# 1. No workspace yet: a call under capture must fail with TOPK_ERR_WORKSPACE, enqueue nothing.
with torch.cuda.stream(stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        try:
            tk.topk_exact(s, l, K=2048, out=out)
            res["capture_without_workspace"] = "ok"
        except tk.TopKError as e:
            res["capture_without_workspace"] = e.code
torch.cuda.synchronize()
# 2. With the workspace (reserve makes it whole, row-split state included): a few long
# rows are split under capture with nothing allocated, and stay exact.
tk.reserve(4096, 1048576, 2048)
s2, l2 = W.make_rows(2, 1048576, [1048576, 1000000], device="cuda")
out2 = torch.empty((2, 2048), dtype=torch.int32, device="cuda")
with torch.cuda.stream(stream):
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=stream):
        tk.topk_exact(s2, l2, K=2048, out=out2)
torch.cuda.synchronize()
tk.reset_stats()
g2.replay()
torch.cuda.synchronize()
res["stats"] = tk.get_stats()
sh, lh, oh = s2.cpu().numpy(), l2.cpu().numpy().astype(np.int32), out2.cpu().numpy()
res["violations"] = int(oracle.check_contract(sh, lh, 2048, -1, oh, oracle.topk(sh, lh, 2048, -1))[0])
print(json.dumps(res))
"""


def test_capture_without_reserve_in_a_fresh_process():
    # A fresh process has no workspace: capturing a call must return TOPK_ERR_WORKSPACE
    # before enqueueing anything; once reserve has made it, a captured call of a few long
    # rows runs row-split and stays exact.
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FRESH_PROCESS, root], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["capture_without_workspace"] == 5  # TOPK_ERR_WORKSPACE
    assert res["violations"] == 0
    assert res["stats"]["rows"] == 2 and res["stats"]["rowsplit"] == 2


# ---------------------------------------------------------- sorted, value-returning output

def _check_sorted(scores, lengths, idx, val, K, sentinel=-1, label=""):
    """GPU sorted output against oracle.topk_sorted. The score sequence is unique, so values
    must match bit for bit; indices must match wherever the score differs from the row's
    boundary score (the K-th), and the boundary-tied indices must ascend. The set itself
    passes the contract check."""
    s = scores.detach().cpu().numpy()
    L = lengths.detach().cpu().numpy().astype(np.int32)
    gi = idx.detach().cpu().numpy()
    ref_i, ref_v = oracle.topk_sorted(s, L, K, sentinel)
    n_bad, status = oracle.check_contract(s, L, K, sentinel, gi, oracle.topk(s, L, K, sentinel))
    assert n_bad == 0, f"{label}: contract {[(int(r), oracle.CHK_NAMES[int(status[r])]) for r in np.nonzero(status)[0][:5]]}"
    if val is not None:
        gv = val.detach().cpu().numpy()
        same = gv.view(np.uint32) == ref_v.view(np.uint32)
        assert same.all(), f"{label}: values differ in rows {np.nonzero(~same.all(axis=1))[0][:8].tolist()}"
    for r in range(s.shape[0]):
        n = min(int(np.clip(L[r], 0, s.shape[1])), K)
        if n == 0:
            assert (gi[r] == sentinel).all()
            continue
        rv = ref_v[r, :n].view(np.uint32)
        b = rv[n - 1]
        strict = rv != b
        assert np.array_equal(gi[r, :n][strict], ref_i[r, :n][strict]), f"{label}: row {r} order differs"
        tied = gi[r, :n][~strict]
        assert (np.diff(tied) > 0).all(), f"{label}: row {r} boundary ties not ascending"
        assert (s[r, tied].view(np.uint32) == b).all()
        assert (gi[r, n:] == sentinel).all()


def test_sorted_output_workloads():
    s0, l0 = W.make_window(W.get("c0"), DEV)
    idx, val = tk.topk_exact_sorted(s0, l0, K=K)
    torch.cuda.synchronize()
    _check_sorted(s0, l0, idx, val, K, label="c0")
    s1, l1 = _window_rows("c1", [(0, 6), (8186, 6)])
    idx, val = tk.topk_exact_sorted(s1, l1, K=K)
    torch.cuda.synchronize()
    _check_sorted(s1, l1, idx, val, K, label="c1")
    s4, l4 = _window_rows("c4_n65536_m512", [(0, 8)])    # bf16 ties at the boundary
    idx, val = tk.topk_exact_sorted(s4, l4, K=K)
    torch.cuda.synchronize()
    _check_sorted(s4, l4, idx, val, K, label="c4 bf16")
    idx2, none = tk.topk_exact_sorted(s4, l4, K=K, values=False)
    torch.cuda.synchronize()
    assert none is None
    _check_sorted(s4, l4, idx2, None, K, label="c4 bf16, indices only")


@pytest.mark.parametrize("seed", range(6))
def test_sorted_output_random_shapes(seed):
    s, l, Kr, n_alloc = _random_case(200 + seed)
    for mode in (tk.PATH_AUTO, tk.PATH_SAMPLED, tk.PATH_RECOVERY, tk.PATH_ROWSPLIT):
        tk.set_path_override(mode)
        try:
            idx, val = tk.topk_exact_sorted(s, l, K=Kr)
            torch.cuda.synchronize()
        finally:
            tk.set_path_override(tk.PATH_AUTO)
        _check_sorted(s, l, idx, val, Kr, label=f"seed {seed} K {Kr} mode {mode}")


@pytest.mark.parametrize("execution", [tk.EXEC_PERSISTENT, tk.EXEC_ROW_PER_WG, tk.EXEC_ROWSPLIT])
def test_sorted_output_every_execution(execution):
    # The selector leaves each selected key in out_val for the sort (rows longer than K);
    # every commit path (tau0 / tau1 refinement, in-place and queued exact recovery, the
    # direct path, short rows) in every execution mode, with values and without them (the
    # indices-only call gathers the scores instead).
    L = 131072
    s1, l1 = _window_rows("c1", [(0, 6)])
    adv = torch.from_numpy(np.stack([_adversarial_row(L, 1000, 900), _adversarial_row(L, 2030, 901)])).to(DEV)
    short = torch.from_numpy(np.stack([_controlled_row(65536, "under_certified", 902),
                                       _controlled_row(65536, "over_full", 903)])).to(DEV)
    short = torch.nn.functional.pad(short, (0, L - 65536), value=float("-inf"))
    s = torch.cat([s1, adv, short]).contiguous()
    l = torch.cat([l1, torch.full((2,), L, dtype=torch.int32, device=DEV),
                   torch.full((2,), 65536, dtype=torch.int32, device=DEV)]).contiguous()
    l[2] = 9000   # direct path
    l[3] = 1500   # shorter than K
    with tk.execution(execution):
        tk.reset_stats()
        idx, val = tk.topk_exact_sorted(s, l, K=K)
        torch.cuda.synchronize()
        st = tk.get_stats()
        idx2, _ = tk.topk_exact_sorted(s, l, K=K, values=False)
        torch.cuda.synchronize()
    _check_sorted(s, l, idx, val, K, label=f"sorted, execution {execution}")
    _check_sorted(s, l, idx2, None, K, label=f"sorted indices only, execution {execution}")
    assert st["direct"] == 1 and st["sentinel"] == 1
    assert st["recover_under"] + st["recover_over"] >= 3


@pytest.mark.parametrize("execution", [tk.EXEC_ROW_PER_WG, tk.EXEC_PERSISTENT])
def test_sorted_output_with_rows_queued_for_recovery(execution):
    # 1M rows: the selector sorts the rows it completes, and the recovery finish kernel
    # sorts the rows handed to it (two underfilled rows, C(tau1) = 1028 < K).
    L = 1048576
    s1, l1 = _window_rows("c3a", [(0, 4)])
    adv = torch.from_numpy(np.stack([_adversarial_row(L, 1000, 950 + i) for i in range(2)])).to(DEV)
    s = torch.cat([s1, adv]).contiguous()
    l = torch.cat([l1, torch.full((2,), L, dtype=torch.int32, device=DEV)]).contiguous()
    with tk.execution(execution):
        tk.reset_stats()
        idx, val = tk.topk_exact_sorted(s, l, K=K)
        torch.cuda.synchronize()
        st = tk.get_stats()
    _check_sorted(s, l, idx, val, K, label=f"sorted with queued rows, execution {execution}")
    assert st["queued"] >= 2 and st["recover_under"] >= 2


def test_sorted_output_k4096_and_misaligned_values():
    s, l = _window_rows("c3a", [(8000, 3)])
    idx, val = tk.topk_exact_sorted(s, l, K=4096)
    torch.cuda.synchronize()
    _check_sorted(s, l, idx, val, 4096, label="1M rows, K 4096")
    buf = torch.empty(3 * 4096 + 1, dtype=torch.float32, device=DEV)
    code = tk.lib().topk_exact_sorted(s.data_ptr(), l.data_ptr(), 3, s.shape[1], 4096, idx.data_ptr(),
                                      buf.data_ptr() + 2, -1, torch.cuda.current_stream().cuda_stream)
    assert code == 7  # TOPK_ERR_BAD_ARG, nothing enqueued


@pytest.mark.parametrize("Kr", [512, 1000, 2048, 4096])
def test_sorted_output_in_selector_workgroups(Kr):
    # Few rows of 64K (bf16 ties; always recovered in place), one workgroup per row: each
    # workgroup sorts its own row once its selection is written (one to eight entries a
    # thread by K); values 4-byte but not 16-byte aligned take the scalar stores; the
    # short row is sorted from its scores.
    s, l = _window_rows("c4_n65536_m512", [(0, 5)])
    l[4] = 1500
    with tk.execution(tk.EXEC_ROW_PER_WG):
        idx, val = tk.topk_exact_sorted(s, l, K=Kr)
        torch.cuda.synchronize()
        _check_sorted(s, l, idx, val, Kr, label=f"sorted in the selector, K {Kr}")
        buf = torch.empty(5 * Kr + 1, dtype=torch.float32, device=DEV)
        idx2 = torch.empty((5, Kr), dtype=torch.int32, device=DEV)
        code = tk.lib().topk_exact_sorted(s.data_ptr(), l.data_ptr(), 5, s.shape[1], Kr, idx2.data_ptr(),
                                          buf.data_ptr() + 4, -1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    assert code == 0, tk.last_error()
    _check_sorted(s, l, idx2, buf[1:].view(5, Kr), Kr, label=f"sorted in the selector, offset values, K {Kr}")
