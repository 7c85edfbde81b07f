"""CPU oracle for exact Top-K selection and the set-contract checker.

TEST INFRASTRUCTURE ONLY: imported by tests, the package smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library. The arithmetic lives in oracle_topk.cpp (plain definition:
per-row std::nth_element under key-descending, index-ascending order); this
module only marshals numpy arrays through ctypes.

Contract followed: page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K",
section "什么叫精确，时间怎么量" (exact set contract with sentinel padding).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_topk.so")
_lib = None

CHK_OK = 0
CHK_OUT_OF_RANGE = 1
CHK_DUPLICATE = 2
CHK_BAD_SENTINEL = 3
CHK_COUNT = 4
CHK_BOUNDARY = 5
CHK_MULTISET = 6
CHK_SHORT_LAYOUT = 7

CHK_NAMES = {
    CHK_OK: "ok",
    CHK_OUT_OF_RANGE: "out_of_range",
    CHK_DUPLICATE: "duplicate",
    CHK_BAD_SENTINEL: "bad_sentinel",
    CHK_COUNT: "count",
    CHK_BOUNDARY: "boundary",
    CHK_MULTISET: "multiset",
    CHK_SHORT_LAYOUT: "short_layout",
}


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing; build it with `python oracle/build.py`")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_topk.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int]
        L.oracle_topk_sorted.restype = ctypes.c_int
        L.oracle_topk_sorted.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int]
        L.oracle_check_contract.restype = ctypes.c_int64
        L.oracle_check_contract.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int]
        _lib = L
    return _lib


def _as_scores(scores):
    s = np.ascontiguousarray(scores, dtype=np.float32)
    if s.ndim != 2:
        raise ValueError("scores must be 2-D [M, N_alloc]")
    return s


def _as_lengths(row_len, M):
    r = np.ascontiguousarray(row_len, dtype=np.int32)
    if r.shape != (M,):
        raise ValueError("row_len must have shape [M]")
    return r


def topk(scores, row_len, K: int, sentinel: int = -1, n_threads: int = None) -> np.ndarray:
    """Exact Top-K indices per row, [M, K] int32 (rows with L > K sorted by key
    descending then index ascending; rows with L <= K are 0..L-1 then sentinel)."""
    s = _as_scores(scores)
    M, N = s.shape
    r = _as_lengths(row_len, M)
    out = np.empty((M, K), dtype=np.int32)
    rc = lib().oracle_topk(s.ctypes.data, r.ctypes.data, M, N, K, sentinel, out.ctypes.data,
                           n_threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_topk rejected its arguments (code {rc})")
    return out


def topk_sorted(scores, row_len, K: int, sentinel: int = -1, n_threads: int = None):
    """Sorted, value-returning Top-K: ([M, K] int32 indices, [M, K] float32 values). Every
    valid index of a row (K of them, or all L when L <= K) in (key descending, index
    ascending) order, then the sentinel; values are the scores, -inf in sentinel slots."""
    s = _as_scores(scores)
    M, N = s.shape
    r = _as_lengths(row_len, M)
    out = np.empty((M, K), dtype=np.int32)
    val = np.empty((M, K), dtype=np.float32)
    rc = lib().oracle_topk_sorted(s.ctypes.data, r.ctypes.data, M, N, K, sentinel, out.ctypes.data,
                                  val.ctypes.data, n_threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_topk_sorted rejected its arguments (code {rc})")
    return out, val


def check_contract(scores, row_len, K: int, sentinel: int, cand, ref=None, n_threads: int = None):
    """Returns (n_failing_rows, per-row CHK_* status array)."""
    s = _as_scores(scores)
    M, N = s.shape
    r = _as_lengths(row_len, M)
    c = np.ascontiguousarray(cand, dtype=np.int32)
    if c.shape != (M, K):
        raise ValueError("cand must have shape [M, K]")
    o = None
    if ref is not None:
        o = np.ascontiguousarray(ref, dtype=np.int32)
        if o.shape != (M, K):
            raise ValueError("ref must have shape [M, K]")
    status = np.empty((M,), dtype=np.int32)
    n = lib().oracle_check_contract(s.ctypes.data, r.ctypes.data, M, N, K, sentinel, c.ctypes.data,
                                    None if o is None else o.ctypes.data, status.ctypes.data,
                                    n_threads or default_threads())
    if n < 0:
        raise ValueError("oracle_check_contract rejected its arguments")
    return int(n), status
