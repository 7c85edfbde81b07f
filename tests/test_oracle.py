"""Pins for the CPU oracle (no GPU).

The oracle is the plain definition of the exact Top-K set contract (page
"几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section
"什么叫精确，时间怎么量"). It is pinned here to things other than itself:
hand-derived golden cases, a literal IEEE totalOrder list, brute-force full
sorts in pure Python and numpy on tiny rows, closed forms (position-valued,
planted and short rows), and torch.topk's value multiset, the dense reference
that page names.
"""
import json
import math
import os
import random
import zlib

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "contract_cases.json")


def _f32(v):
    if isinstance(v, str):
        return np.float32(float(v))
    return np.float32(v)


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def test_golden_contract_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 10
    for c in cases:
        row = np.array([[_f32(v) for v in c["row"]]], dtype=np.float32)
        K, sentinel, L = c["K"], c["sentinel"], c["len"]
        out = oracle.topk(row, np.array([L], np.int32), K, sentinel)[0]
        if "expect_exact" in c:
            assert out.tolist() == c["expect_exact"], c["id"]
        elif "expect_set" in c:
            assert sorted(out.tolist()) == sorted(c["expect_set"]), c["id"]
        else:
            vals = sorted(float(row[0, i]) for i in out)
            assert vals == sorted(float(_f32(v)) for v in c["expect_values"]), c["id"]
            assert set(c["must_include"]) <= set(out.tolist()), c["id"]
            assert len(set(out.tolist())) == K and all(0 <= i < L for i in out), c["id"]
        n_bad, _ = oracle.check_contract(row, np.array([L], np.int32), K, sentinel, out[None, :])
        assert n_bad == 0, c["id"]


# IEEE-754 totalOrder, ascending, written out literally (not computed).
TOTAL_ORDER = [
    "-inf", -3.4028234663852886e38, -1.0, -1.1754943508222875e-38, -1.401298464324817e-45, "-0.0",
    0.0, 1.401298464324817e-45, 1.1754943508222875e-38, 1.0, 3.4028234663852886e38, "inf",
]


def test_total_order_literal():
    asc = np.array([_f32(v) for v in TOTAL_ORDER], dtype=np.float32)
    n = len(asc)
    rng = random.Random(7)
    for trial in range(20):
        perm = list(range(n))
        rng.shuffle(perm)
        row = asc[perm][None, :]
        for K in range(1, n):
            out = oracle.topk(row, np.array([n], np.int32), K)[0]
            got = sorted(_bits(row[0, out]).tolist())
            want = sorted(_bits(asc[n - K:]).tolist())
            assert got == want, (trial, K)


def _bruteforce_python(vals, L, K, sentinel):
    """Full sort in pure Python by (value descending, index ascending); no zeros/NaN."""
    if L <= K:
        return list(range(L)) + [sentinel] * (K - L)
    order = sorted(range(L), key=lambda i: (-float(vals[i]), i))
    return order[:K]


@pytest.mark.parametrize("dist", ["normal", "small_ints", "two_valued", "all_equal", "with_neg_inf",
                                  "denormal", "wide"])
def test_bruteforce_tiny_rows(dist):
    rng = np.random.default_rng(zlib.crc32(dist.encode()))
    N = 64
    for trial in range(150):
        M = 4
        if dist == "normal":
            x = rng.normal(30, 2.5, size=(M, N))
        elif dist == "small_ints":
            x = rng.integers(1, 6, size=(M, N)).astype(np.float64)
        elif dist == "two_valued":
            x = np.where(rng.random((M, N)) < 0.5, 3.0, -2.0)
        elif dist == "all_equal":
            x = np.full((M, N), 7.5)
        elif dist == "with_neg_inf":
            x = rng.normal(0, 1, size=(M, N))
            x[rng.random((M, N)) < 0.3] = -np.inf
        elif dist == "denormal":
            x = rng.integers(1, 200, size=(M, N)) * 1.401298464324817e-45 * rng.choice([-1, 1], (M, N))
        else:
            x = rng.normal(0, 1, size=(M, N)) * 10.0 ** rng.integers(-30, 30, size=(M, N))
        x = x.astype(np.float32)
        x[x == 0] = np.float32(1.0)  # zeros are covered by the totalOrder tests
        L = rng.integers(0, N + 1, size=M).astype(np.int32)
        K = int(rng.integers(1, 71))
        out = oracle.topk(x, L, K, sentinel=-1)
        for r in range(M):
            want = _bruteforce_python(x[r], int(L[r]), K, -1)
            if L[r] <= K:
                assert out[r].tolist() == want
            else:
                # Same tie-break (lower index first) on both sides: identical sets.
                assert sorted(out[r].tolist()) == sorted(want), (dist, trial, r, K, int(L[r]))


def test_numpy_stable_argsort_with_ties():
    rng = np.random.default_rng(11)
    M, N, K = 24, 3000, 700
    x = rng.integers(-20, 20, size=(M, N)).astype(np.float32)
    x[x == 0] = 0.5
    L = rng.integers(K + 1, N + 1, size=M).astype(np.int32)
    out = oracle.topk(x, L, K)
    for r in range(M):
        ref = np.argsort(-x[r, :L[r]], kind="stable")[:K]
        assert sorted(out[r].tolist()) == sorted(ref.tolist())


def test_signed_zero_boundary():
    # Half +0, half -0, K picks exactly the +0 entries first (totalOrder reading).
    row = np.array([[0.0, -0.0] * 20], dtype=np.float32)
    out = oracle.topk(row, np.array([40], np.int32), 20)[0]
    assert sorted(out.tolist()) == list(range(0, 40, 2))
    out = oracle.topk(row, np.array([40], np.int32), 25)[0]
    assert set(range(0, 40, 2)) <= set(out.tolist())


def test_position_valued_rows():
    # Closed form: if value == position, the top-K set is {L-K, ..., L-1}.
    N, K = 5000, 2048
    x = np.tile(np.arange(N, dtype=np.float32), (5, 1))
    L = np.array([N, 4096, 2049, 2048, 3000], np.int32)
    out = oracle.topk(x, L, K)
    for r in range(5):
        if L[r] > K:
            assert sorted(out[r].tolist()) == list(range(L[r] - K, L[r]))
        else:
            assert out[r].tolist() == list(range(L[r])) + [-1] * (K - L[r])
    # Reversed: value decreasing with position -> top-K set is {0..K-1}.
    y = np.ascontiguousarray(x[:, ::-1])
    out = oracle.topk(y, np.array([N] * 5, np.int32), K)
    for r in range(5):
        assert sorted(out[r].tolist()) == list(range(K))


def test_planted_rows_and_row_stride():
    rng = np.random.default_rng(3)
    M, N, K = 6, 20000, 2048
    x = (rng.random((M, N)) * 50).astype(np.float32)
    planted = []
    for r in range(M):
        pos = rng.choice(N, size=K, replace=False)
        x[r, pos] = (100 + np.arange(K) + r).astype(np.float32)
        planted.append(set(pos.tolist()))
    out = oracle.topk(x, np.full(M, N, np.int32), K)
    for r in range(M):
        assert set(out[r].tolist()) == planted[r]


def test_length_clamping_and_sentinel():
    x = np.arange(10, dtype=np.float32)[None, :].repeat(3, 0)
    out = oracle.topk(x, np.array([-5, 99, 0], np.int32), 4, sentinel=-9)
    assert out[0].tolist() == [-9] * 4          # negative length -> empty row
    assert sorted(out[1].tolist()) == [6, 7, 8, 9]  # length past N_alloc -> N_alloc
    assert out[2].tolist() == [-9] * 4


def test_torch_topk_value_multiset():
    # torch.topk(largest=True, sorted=False) is the dense reference the pages name.
    g = torch.Generator().manual_seed(5)
    M, N, K = 8, 40000, 2048
    x = torch.randn(M, N, generator=g) * 3 + 30
    x[x == 0] = 1.0
    L = torch.randint(K + 1, N + 1, (M,), generator=g, dtype=torch.int32)
    out = oracle.topk(x.numpy(), L.numpy(), K)
    for r in range(M):
        ref_vals = torch.topk(x[r, :int(L[r])], K, largest=True, sorted=False).values
        got = torch.from_numpy(x[r].numpy()[out[r]])
        assert torch.equal(torch.sort(got).values, torch.sort(ref_vals).values)


def test_threads_do_not_change_result():
    rng = np.random.default_rng(9)
    x = rng.integers(0, 50, size=(33, 5000)).astype(np.float32)
    L = rng.integers(0, 5001, size=33).astype(np.int32)
    a = oracle.topk(x, L, 300, n_threads=1)
    b = oracle.topk(x, L, 300, n_threads=8)
    assert np.array_equal(a, b)


def test_oracle_rows_are_sorted_descending():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, size=(4, 1000)).astype(np.float32)
    out = oracle.topk(x, np.full(4, 1000, np.int32), 100)
    for r in range(4):
        v = x[r, out[r]]
        assert np.all(v[:-1] >= v[1:])


# ---- sorted, value-returning output --------------------------------------------------------

def _py_key(v):
    u = int(np.asarray(v, dtype=np.float32).view(np.uint32))
    return (~u & 0xFFFFFFFF) if u & 0x80000000 else (u | 0x80000000)


def test_sorted_oracle_matches_python_sort_on_tiny_rows():
    rng = random.Random(7)
    pool = [0.0, -0.0, 1.0, -1.0, 2.5, float("inf"), float("-inf"), 1e-45, -1e-45, 3.0, 3.0]
    for _ in range(400):
        L = rng.randint(0, 24)
        N = max(L, 1) + rng.randint(0, 3)
        K = rng.randint(1, 30)
        row = np.array([rng.choice(pool) for _ in range(N)], dtype=np.float32)
        idx, val = oracle.topk_sorted(row[None, :], np.array([L], dtype=np.int32), K, -7)
        want = sorted(range(L), key=lambda j: (-_py_key(row[j]), j))[:min(K, L)]
        want_idx = want + [-7] * (K - len(want))
        assert idx[0].tolist() == want_idx
        want_val = np.array([row[j] for j in want] + [-np.inf] * (K - len(want)), dtype=np.float32)
        assert np.array_equal(val[0].view(np.uint32), want_val.view(np.uint32))


def test_sorted_oracle_closed_forms_and_agreement_with_topk():
    # Position-valued rows: the sorted output is L-1, L-2, ... with values equal to the indices.
    N, K = 100, 16
    s = np.tile(np.arange(N, dtype=np.float32), (3, 1))
    L = np.array([100, 40, 9], dtype=np.int32)
    idx, val = oracle.topk_sorted(s, L, K, -1)
    for r in range(3):
        n = min(K, int(L[r]))
        assert idx[r, :n].tolist() == list(range(int(L[r]) - 1, int(L[r]) - 1 - n, -1))
        assert np.array_equal(val[r, :n], idx[r, :n].astype(np.float32))
        assert (idx[r, n:] == -1).all() and np.isneginf(val[r, n:]).all()
    # Rows longer than K: the plain oracle's rows are already in this order.
    rng = np.random.default_rng(3)
    s = rng.integers(0, 6, size=(20, 300)).astype(np.float32)
    L = rng.integers(K + 1, 301, size=20).astype(np.int32)
    idx, val = oracle.topk_sorted(s, L, K, -1)
    assert np.array_equal(idx, oracle.topk(s, L, K, -1))
    assert np.array_equal(val, np.take_along_axis(s, idx.astype(np.int64), axis=1))
