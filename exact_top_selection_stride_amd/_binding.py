"""ctypes binding of libtopk_exact.so (include/topk_exact.h).

Argument marshalling only: shapes, dtypes and devices are checked, the raw device
pointers and the current HIP stream are handed to the C ABI, and every step of
the selection runs in the library's kernels. There is no CPU fallback: if the
library is missing the call raises.
"""
import contextlib
import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtopk_exact.so")

TOPK_OK = 0
TOPK_ERR_NULL_POINTER = 1
TOPK_ERR_BAD_SHAPE = 2
TOPK_ERR_BAD_K = 3
TOPK_ERR_BAD_SENTINEL = 4
TOPK_ERR_WORKSPACE = 5
TOPK_ERR_HIP = 6
TOPK_ERR_BAD_ARG = 7
TOPK_K_MAX = 4096

PATH_AUTO = 0
PATH_SAMPLED = 1
PATH_ROWSPLIT = 2
PATH_DIRECT = 3
PATH_RECOVERY = 4

EXEC_AUTO = 0
EXEC_PERSISTENT = 1
EXEC_ROW_PER_WG = 2
EXEC_ROWSPLIT = 3

STAT_NAMES = (
    "rows", "sentinel", "direct", "sampled", "tau0", "tau1", "recover_under", "recover_over",
    "rowsplit", "forced_recovery", "long_exact", "frontier_wide", "queued", "persistent", "row_per_wg",
    "recover_inplace", "inplace_certified", "inplace_full", "tau_a",
)
STAT_COUNT = 24

EXPORTED = (
    "topk_exact", "topk_exact_reserve", "topk_exact_get_stats", "topk_exact_reset_stats",
    "topk_exact_set_path_override", "topk_exact_last_error", "topk_stream_read_probe",
    "topk_exact_set_execution", "topk_exact_time_next_call", "topk_exact_set_proposal",
    "topk_indexer_scores", "topk_indexer_topk", "topk_exact_sorted", "topk_exact_noalloc",
    "topk_exact_record_phases", "topk_exact_set_admission",
)


class TopKError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed with status {code}: {last_error()}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Loads the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m exact_top_selection_stride_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.topk_exact.restype = ctypes.c_int
        L.topk_exact.argtypes = [vp, vp, i64, i64, i32, vp, i32, vp]
        L.topk_exact_noalloc.restype = ctypes.c_int
        L.topk_exact_noalloc.argtypes = [vp, vp, i64, i64, i32, vp, i32, vp]
        L.topk_exact_reserve.restype = ctypes.c_int
        L.topk_exact_reserve.argtypes = [i64, i64, i32]
        L.topk_exact_get_stats.restype = ctypes.c_int
        L.topk_exact_get_stats.argtypes = [vp, ctypes.c_int, vp]
        L.topk_exact_reset_stats.restype = ctypes.c_int
        L.topk_exact_reset_stats.argtypes = [vp]
        L.topk_exact_set_path_override.restype = ctypes.c_int
        L.topk_exact_set_path_override.argtypes = [ctypes.c_int]
        L.topk_exact_set_execution.restype = ctypes.c_int
        L.topk_exact_set_execution.argtypes = [ctypes.c_int]
        L.topk_exact_set_proposal.restype = ctypes.c_int
        L.topk_exact_set_proposal.argtypes = [i32, i32, i32]
        L.topk_exact_set_admission.restype = ctypes.c_int
        L.topk_exact_set_admission.argtypes = [i32]
        L.topk_exact_time_next_call.restype = ctypes.c_int
        L.topk_exact_time_next_call.argtypes = [vp, vp]
        L.topk_exact_record_phases.restype = ctypes.c_int
        L.topk_exact_record_phases.argtypes = [vp, i64, vp]
        L.topk_exact_last_error.restype = ctypes.c_char_p
        L.topk_exact_last_error.argtypes = []
        L.topk_stream_read_probe.restype = ctypes.c_int
        L.topk_stream_read_probe.argtypes = [vp, i64, vp, vp]
        L.topk_indexer_scores.restype = ctypes.c_int
        L.topk_indexer_scores.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, vp, vp]
        L.topk_exact_sorted.restype = ctypes.c_int
        L.topk_exact_sorted.argtypes = [vp, vp, i64, i64, i32, vp, vp, i32, vp]
        L.topk_indexer_topk.restype = ctypes.c_int
        L.topk_indexer_topk.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, vp, vp, i32, vp]
        _lib = L
    return _lib


def last_error() -> str:
    if _lib is None:
        return ""
    return (_lib.topk_exact_last_error() or b"").decode(errors="replace")


def _check(code: int, what: str):
    if code != TOPK_OK:
        raise TopKError(code, what)


def _stream_handle(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def topk_exact(scores: torch.Tensor, row_len: torch.Tensor, K: int = 2048, sentinel: int = -1,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Exact top-K indices of each ragged row; returns int32 [M, K] on the scores' device.

    scores: float32 [M, N_alloc] on a GPU, unit column stride and row stride N_alloc.
    row_len: int32 [M] on the same GPU. out (optional): int32 [M, K], contiguous.
    Enqueued on `stream` (default: the current stream); nothing synchronizes.
    """
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise ValueError("scores must be a 2-D float32 GPU tensor")
    M, N = scores.shape
    if scores.stride(1) != 1 or (M > 1 and scores.stride(0) != N):
        raise ValueError("scores must be row-major with row stride N_alloc")
    if row_len.dtype != torch.int32 or row_len.device != scores.device or tuple(row_len.shape) != (M,):
        raise ValueError("row_len must be an int32 [M] tensor on the scores' device")
    if not row_len.is_contiguous():
        raise ValueError("row_len must be contiguous")
    if out is None:
        out = torch.empty((M, K), dtype=torch.int32, device=scores.device)
    elif (out.dtype != torch.int32 or out.device != scores.device or tuple(out.shape) != (M, K)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [M, K] tensor on the scores' device")
    with torch.cuda.device(scores.device):
        code = lib().topk_exact(scores.data_ptr(), row_len.data_ptr(), M, N, K, out.data_ptr(),
                                sentinel, _stream_handle(scores.device, stream))
    _check(code, "topk_exact")
    return out


def topk_exact_noalloc(scores: torch.Tensor, row_len: torch.Tensor, K: int = 2048, sentinel: int = -1,
                       out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """topk_exact through the allocation-free entry point (the library's fixed scratch
    array instead of its workspace). `out` should be given where the caller cannot
    allocate; without it torch allocates the output here."""
    M, N = _check_scores(scores, row_len)
    if out is None:
        out = torch.empty((M, K), dtype=torch.int32, device=scores.device)
    elif (out.dtype != torch.int32 or out.device != scores.device or tuple(out.shape) != (M, K)
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous int32 [M, K] tensor on the scores' device")
    with torch.cuda.device(scores.device):
        code = lib().topk_exact_noalloc(scores.data_ptr(), row_len.data_ptr(), M, N, K, out.data_ptr(),
                                        sentinel, _stream_handle(scores.device, stream))
    _check(code, "topk_exact_noalloc")
    return out


def _check_scores(scores, row_len):
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise ValueError("scores must be a 2-D float32 GPU tensor")
    M, N = scores.shape
    if scores.stride(1) != 1 or (M > 1 and scores.stride(0) != N):
        raise ValueError("scores must be row-major with row stride N_alloc")
    if row_len.dtype != torch.int32 or row_len.device != scores.device or tuple(row_len.shape) != (M,) \
            or not row_len.is_contiguous():
        raise ValueError("row_len must be a contiguous int32 [M] tensor on the scores' device")
    return M, N


def topk_exact_sorted(scores: torch.Tensor, row_len: torch.Tensor, K: int = 2048, sentinel: int = -1,
                      values: bool = True, out: Optional[torch.Tensor] = None,
                      out_values: Optional[torch.Tensor] = None, stream=None):
    """Sorted, value-returning top-K: (indices int32 [M, K], values float32 [M, K] or None).

    Each row lists its selected indices by score descending (ties by index ascending),
    then the sentinel; values are the scores of the listed indices and -inf in sentinel
    slots. Same inputs and stream semantics as topk_exact.
    """
    if scores.dim() != 2 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise ValueError("scores must be a 2-D float32 GPU tensor")
    M, N = scores.shape
    if scores.stride(1) != 1 or (M > 1 and scores.stride(0) != N):
        raise ValueError("scores must be row-major with row stride N_alloc")
    if row_len.dtype != torch.int32 or row_len.device != scores.device or tuple(row_len.shape) != (M,) \
            or not row_len.is_contiguous():
        raise ValueError("row_len must be a contiguous int32 [M] tensor on the scores' device")
    dev = scores.device
    if out is None:
        out = torch.empty((M, K), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or out.device != dev or tuple(out.shape) != (M, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [M, K] tensor on the scores' device")
    if values and out_values is None:
        out_values = torch.empty((M, K), dtype=torch.float32, device=dev)
    if out_values is not None and (out_values.dtype != torch.float32 or out_values.device != dev
                                   or tuple(out_values.shape) != (M, K) or not out_values.is_contiguous()):
        raise ValueError("out_values must be a contiguous float32 [M, K] tensor on the scores' device")
    with torch.cuda.device(dev):
        code = lib().topk_exact_sorted(scores.data_ptr(), row_len.data_ptr(), M, N, K, out.data_ptr(),
                                       out_values.data_ptr() if out_values is not None else None,
                                       sentinel, _stream_handle(dev, stream))
    _check(code, "topk_exact_sorted")
    return out, out_values


def reserve(M_max: int, N_alloc_max: int, K: int = 2048, device=None):
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(lib().topk_exact_reserve(M_max, N_alloc_max, K), "topk_exact_reserve")


def get_stats(device=None, stream=None) -> dict:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    buf = (ctypes.c_uint64 * STAT_COUNT)()
    with torch.cuda.device(dev):
        _check(lib().topk_exact_get_stats(ctypes.addressof(buf), STAT_COUNT, _stream_handle(dev, stream)),
               "topk_exact_get_stats")
    return {name: int(buf[i]) for i, name in enumerate(STAT_NAMES)}


def reset_stats(device=None, stream=None):
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check(lib().topk_exact_reset_stats(_stream_handle(dev, stream)), "topk_exact_reset_stats")


def set_path_override(mode: int):
    _check(lib().topk_exact_set_path_override(int(mode)), "topk_exact_set_path_override")


@contextlib.contextmanager
def path_override(mode: int):
    set_path_override(mode)
    try:
        yield
    finally:
        set_path_override(PATH_AUTO)


def set_execution(mode: int):
    _check(lib().topk_exact_set_execution(int(mode)), "topk_exact_set_execution")


@contextlib.contextmanager
def execution(mode: int):
    set_execution(mode)
    try:
        yield
    finally:
        set_execution(EXEC_AUTO)


def set_proposal(stride: int = 128, rho0: float = 1.5, rho1: float = 1.75):
    """Sample stride and candidate targets (rho0*K, rho1*K) for later calls; the method's
    values are the defaults. Any setting gives an exact result."""
    _check(lib().topk_exact_set_proposal(int(stride), int(round(rho0 * 1000)), int(round(rho1 * 1000))),
           "topk_exact_set_proposal")


@contextlib.contextmanager
def proposal(stride: int = 128, rho0: float = 1.5, rho1: float = 1.75):
    set_proposal(stride, rho0, rho1)
    try:
        yield
    finally:
        _check(lib().topk_exact_set_proposal(0, 0, 0), "topk_exact_set_proposal")


def set_admission(rho_a: float = 2.25):
    """Admission target rho_a*K of rows sampled one element per period (0 turns the deeper
    admission off: every row admits at tau1). Any setting gives an exact result."""
    _check(lib().topk_exact_set_admission(int(round(rho_a * 1000))), "topk_exact_set_admission")


@contextlib.contextmanager
def admission(rho_a: float = 2.25):
    set_admission(rho_a)
    try:
        yield
    finally:
        _check(lib().topk_exact_set_admission(-1), "topk_exact_set_admission")


def time_next_call(start, stop):
    """Arms the one-shot selector timing of the next topk_exact call on this thread.

    start/stop: torch.cuda.Event(enable_timing=True) that have been recorded at least
    once (so the HIP events exist), or None for both to disarm. After the timed call
    completes, start.elapsed_time(stop) is the selector kernels' time in ms.
    """
    if (start is None) != (stop is None):
        raise ValueError("start and stop must both be events or both be None")
    h0 = start.cuda_event if start is not None else 0
    h1 = stop.cuda_event if stop is not None else 0
    if start is not None and (not h0 or not h1):
        raise ValueError("record both events once before arming the hook")
    _check(lib().topk_exact_time_next_call(h0 or None, h1 or None), "topk_exact_time_next_call")


PHASE_WORDS = 8
PHASE_NAMES = ("start", "sampled", "proposed", "passed", "end", "recovered", "where", "counts")
PATH_CODES = {1: "sentinel", 2: "direct", 3: "tau0", 4: "tau1", 5: "recover_inplace", 6: "recover_queued",
              7: "forced_recovery", 8: "tau_a"}


def record_phases(buf: Optional[torch.Tensor]) -> int:
    """Arms (buf: int64 [rows, 8] GPU tensor) or disarms (None) the per-row phase
    recording of later calls; returns the device wall-clock rate in kHz."""
    khz = ctypes.c_int64(0)
    if buf is None:
        _check(lib().topk_exact_record_phases(None, 0, ctypes.addressof(khz)), "topk_exact_record_phases")
    else:
        if buf.dtype != torch.int64 or not buf.is_cuda or buf.dim() != 2 or buf.shape[1] != PHASE_WORDS \
                or not buf.is_contiguous():
            raise ValueError("buf must be a contiguous int64 [rows, 8] GPU tensor")
        with torch.cuda.device(buf.device):
            _check(lib().topk_exact_record_phases(buf.data_ptr(), buf.shape[0], ctypes.addressof(khz)),
                   "topk_exact_record_phases")
    return int(khz.value)


def stream_read_probe(x: torch.Tensor, sink: torch.Tensor, stream=None):
    """Reads every element of x (a float32 GPU tensor) once; measurement only."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    if sink.dtype != torch.float32 or sink.device != x.device or sink.numel() < 4096:
        raise ValueError("sink must be a float32 tensor of >= 4096 elements on x's device")
    with torch.cuda.device(x.device):
        _check(lib().topk_stream_read_probe(x.data_ptr(), x.numel(), sink.data_ptr(),
                                            _stream_handle(x.device, stream)), "topk_stream_read_probe")


def _indexer_args(q, k, w, row_len):
    if q.dtype == torch.float8_e4m3fn:
        q = q.view(torch.uint8)
    if k.dtype == torch.float8_e4m3fn:
        k = k.view(torch.uint8)
    if q.dim() != 3 or q.dtype != torch.uint8 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous uint8 [T, H, D] GPU tensor")
    T, H, D = q.shape
    dev = q.device
    if k.dim() != 2 or k.dtype != torch.uint8 or k.device != dev or not k.is_contiguous() or k.shape[1] != D:
        raise ValueError("k must be a contiguous uint8 [S, D] tensor on q's device")
    if w.dtype != torch.float32 or w.device != dev or tuple(w.shape) != (T, H) or not w.is_contiguous():
        raise ValueError("w must be a contiguous float32 [T, H] tensor on q's device")
    if row_len.dtype != torch.int32 or row_len.device != dev or tuple(row_len.shape) != (T,) \
            or not row_len.is_contiguous():
        raise ValueError("row_len must be a contiguous int32 [T] tensor on q's device")
    return q, k, T, H, D, k.shape[0], dev


def _scores_buffer(out, T, S, dev):
    if out is None:
        return torch.empty((T, S), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.device != dev or tuple(out.shape) != (T, S) or not out.is_contiguous():
        raise ValueError("scores must be a contiguous float32 [T, S] tensor on q's device")
    return out


def indexer_scores(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, row_len: torch.Tensor,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """FP8 indexer scores I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . k[s]), -inf for s >= row_len[t].

    q: uint8 [T, H, D] holding OCP E4M3 codes (torch.float8_e4m3fn viewed as uint8 also
    accepted), k: uint8 [S, D] likewise, w: float32 [T, H], row_len: int32 [T], all
    contiguous on one GPU; H in {16, 32, 48, 64}, D = 128. Returns float32 [T, S]
    (or fills `out`). Enqueued on `stream` (default: the current stream).
    """
    q, k, T, H, D, S, dev = _indexer_args(q, k, w, row_len)
    out = _scores_buffer(out, T, S, dev)
    with torch.cuda.device(dev):
        code = lib().topk_indexer_scores(q.data_ptr(), k.data_ptr(), w.data_ptr(), row_len.data_ptr(),
                                         T, S, H, D, out.data_ptr(), _stream_handle(dev, stream))
    _check(code, "topk_indexer_scores")
    return out


def indexer_topk(q: torch.Tensor, k: torch.Tensor, w: torch.Tensor, row_len: torch.Tensor,
                 K: int = 2048, sentinel: int = -1, scores: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, stream=None):
    """The score + select chain (topk_indexer_topk): indexer scores, then the exact top-K of
    each ragged row, both enqueued on one stream (graph-capturable).
    Returns (scores [T, S] float32, idx [T, K] int32)."""
    q, k, T, H, D, S, dev = _indexer_args(q, k, w, row_len)
    scores = _scores_buffer(scores, T, S, dev)
    if out is None:
        out = torch.empty((T, K), dtype=torch.int32, device=dev)
    elif out.dtype != torch.int32 or out.device != dev or tuple(out.shape) != (T, K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 [T, K] tensor on q's device")
    with torch.cuda.device(dev):
        code = lib().topk_indexer_topk(q.data_ptr(), k.data_ptr(), w.data_ptr(), row_len.data_ptr(),
                                       T, S, H, D, K, scores.data_ptr(), out.data_ptr(), sentinel,
                                       _stream_handle(dev, stream))
    _check(code, "topk_indexer_topk")
    return scores, out
