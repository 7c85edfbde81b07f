"""Pins for the set-contract checker (no GPU): every injected fault is flagged.

The contract (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K",
section "什么叫精确，时间怎么量"): distinct indices inside the valid prefix;
exactly K of them with min(selected) >= max(unselected) when L > K, ties free,
order free; all valid indices plus the sentinel when L <= K.
"""
import numpy as np

import oracle
from oracle import (CHK_BAD_SENTINEL, CHK_BOUNDARY, CHK_DUPLICATE, CHK_MULTISET, CHK_OK,
                    CHK_OUT_OF_RANGE, CHK_SHORT_LAYOUT)

K = 8
S = -1


def _row(seed=0, n=64):
    rng = np.random.default_rng(seed)
    return rng.permutation(n).astype(np.float32)[None, :]  # distinct values 0..n-1


def _check(x, L, cand, ref=None):
    n, st = oracle.check_contract(x, np.array([L], np.int32), K, S, np.asarray(cand, np.int32)[None, :],
                                  None if ref is None else np.asarray(ref, np.int32)[None, :])
    return int(st[0])


def _topk_positions(x, L):
    return list(np.argsort(-x[0, :L], kind="stable")[:K])


def test_correct_output_passes():
    x = _row()
    good = _topk_positions(x, 64)
    assert _check(x, 64, good) == CHK_OK
    assert _check(x, 64, good[::-1]) == CHK_OK          # order is free
    assert _check(x, 64, good, ref=good) == CHK_OK


def test_injected_faults_are_flagged():
    x = _row()
    good = _topk_positions(x, 64)
    dup = good[:-1] + [good[0]]
    assert _check(x, 64, dup) == CHK_DUPLICATE
    oob = good[:-1] + [64]
    assert _check(x, 64, oob) == CHK_OUT_OF_RANGE
    neg = good[:-1] + [-5]
    assert _check(x, 64, neg) == CHK_OUT_OF_RANGE
    sent = good[:-1] + [S]
    assert _check(x, 64, sent) == CHK_BAD_SENTINEL
    # swap the smallest selected for a smaller unselected entry
    smallest_sel = min(good, key=lambda i: x[0, i])
    smaller = int(np.argsort(-x[0])[K])  # the (K+1)-th largest
    swapped = [smaller if i == smallest_sel else i for i in good]
    assert _check(x, 64, swapped) == CHK_BOUNDARY
    # index beyond the valid prefix, even though inside N_alloc
    L = 40
    good_l = _topk_positions(x, L)
    beyond = good_l[:-1] + [50]
    assert _check(x, L, beyond) == CHK_OUT_OF_RANGE


def test_reference_multiset_mismatch_is_flagged():
    x = _row()
    good = _topk_positions(x, 64)
    bad_ref = good[:-1] + [int(np.argsort(-x[0])[K + 3])]
    assert _check(x, 64, good, ref=bad_ref) == CHK_MULTISET


def test_signed_zero_boundary_is_flagged():
    # Under totalOrder +0 > -0: choosing -0 while leaving +0 out breaks the boundary.
    x = np.array([[5, 4, 3, 2, 1, 9, 8, -0.0, 0.0, -1.0]], dtype=np.float32)
    Kz = 8
    good = [0, 1, 2, 3, 4, 5, 6, 8]
    bad = [0, 1, 2, 3, 4, 5, 6, 7]
    n, st = oracle.check_contract(x, np.array([10], np.int32), Kz, S, np.array([good], np.int32))
    assert st[0] == CHK_OK
    n, st = oracle.check_contract(x, np.array([10], np.int32), Kz, S, np.array([bad], np.int32))
    assert st[0] == CHK_BOUNDARY


def test_boundary_ties_are_free():
    x = np.array([[9, 4, 4, 4, 1, 0.5, 0.25, 3, 2, 4]], dtype=np.float32)
    Kt = 3
    for choice in ([0, 1, 2], [0, 2, 3], [0, 9, 1], [3, 0, 9]):
        n, st = oracle.check_contract(x, np.array([10], np.int32), Kt, S, np.array([choice], np.int32),
                                      np.array([[0, 1, 2]], np.int32))
        assert st[0] == CHK_OK, choice


def test_short_row_layout():
    x = _row()
    L = 5
    good = [0, 1, 2, 3, 4, S, S, S]
    assert _check(x, L, good) == CHK_OK
    assert _check(x, L, [4, 3, 2, 1, 0, S, S, S]) == CHK_OK           # any order inside [0, L)
    assert _check(x, L, [0, 1, 2, 3, S, S, S, S]) == CHK_SHORT_LAYOUT  # missing index 4
    assert _check(x, L, [0, 1, 2, 3, 4, 5, S, S]) == CHK_SHORT_LAYOUT  # extra index past L
    assert _check(x, L, [0, 1, 2, 3, 3, S, S, S]) == CHK_DUPLICATE
    assert _check(x, 0, [S] * K) == CHK_OK
    assert _check(x, K, list(range(K))) == CHK_OK
    assert _check(x, K, list(range(K - 1)) + [S]) == CHK_SHORT_LAYOUT


def test_checker_agrees_with_oracle_on_random_rows():
    rng = np.random.default_rng(4)
    x = rng.integers(0, 30, size=(50, 900)).astype(np.float32)
    L = rng.integers(0, 901, size=50).astype(np.int32)
    ref = oracle.topk(x, L, 100)
    n, st = oracle.check_contract(x, L, 100, -1, ref, ref)
    assert n == 0
