"""The C-ABI library loads and exports every declared entry point; host-side
argument validation returns its documented codes without touching a GPU."""
import ctypes
import os
import re

import pytest

import exact_top_selection_stride_amd as tk
from exact_top_selection_stride_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "topk_exact.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(n for n in names if n.startswith("topk_")))


def test_header_declares_expected_entry_points():
    decl = _declared_functions()
    assert sorted(B.EXPORTED) == decl


def test_library_exports_every_declared_symbol():
    L = tk.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_argument_validation_without_gpu():
    L = tk.lib()
    fake = 0x1000  # never dereferenced: validation rejects the call first
    assert L.topk_exact(fake, fake, -1, 10, 4, fake, -1, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_exact(fake, fake, 2, 0, 4, fake, -1, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_exact(fake, fake, 2, 2**31, 4, fake, -1, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_exact(fake, fake, 2, 10, 0, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert L.topk_exact(fake, fake, 2, 10, B.TOPK_K_MAX + 1, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert L.topk_exact(fake, fake, 2, 10, 4, fake, 3, None) == B.TOPK_ERR_BAD_SENTINEL
    assert L.topk_exact(fake, fake, 2, 10, 4, fake, 0, None) == B.TOPK_ERR_BAD_SENTINEL
    assert L.topk_exact(None, fake, 2, 10, 4, fake, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact(fake, None, 2, 10, 4, fake, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact(fake, fake, 2, 10, 4, None, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert "null" in tk.last_error()
    # M == 0 is a successful no-op, even with null pointers.
    assert L.topk_exact(None, None, 0, 10, 4, None, -1, None) == B.TOPK_OK
    # A sentinel at or past N_alloc is allowed.
    assert L.topk_exact(fake, fake, 0, 10, 4, fake, 10, None) == B.TOPK_OK
    # The allocation-free entry point checks its arguments the same way, before any device work.
    assert L.topk_exact_noalloc(fake, fake, -1, 10, 4, fake, -1, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_exact_noalloc(fake, fake, 2, 10, B.TOPK_K_MAX + 1, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert L.topk_exact_noalloc(fake, fake, 2, 10, 4, fake, 5, None) == B.TOPK_ERR_BAD_SENTINEL
    assert L.topk_exact_noalloc(fake, None, 2, 10, 4, fake, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact_noalloc(None, None, 0, 10, 4, None, -1, None) == B.TOPK_OK
    assert L.topk_exact_record_phases(None, 5, None) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_record_phases(fake, 0, None) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_record_phases(None, 0, None) == B.TOPK_OK
    assert L.topk_exact_set_path_override(99) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_path_override(-1) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_get_stats(None, 4, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact_reserve(-1, 10, 4) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_exact_reserve(1, 10, 0) == B.TOPK_ERR_BAD_K
    assert L.topk_stream_read_probe(None, -1, None, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_stream_read_probe(None, 0, None, None) == B.TOPK_OK
    # Proposal parameters: stride in [1, 65536], 500 <= rho0 <= rho1 <= 4000 (thousandths).
    assert L.topk_exact_set_proposal(0, 1500, 1750) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_proposal(70000, 1500, 1750) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_proposal(128, 1750, 1500) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_proposal(128, 400, 1500) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_proposal(128, 1500, 4001) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_proposal(64, 1000, 1250) == B.TOPK_OK
    assert L.topk_exact_set_proposal(0, 0, 0) == B.TOPK_OK
    # Admission target: -1 (default), 0 (off) or 1000..8000 thousandths of K.
    assert L.topk_exact_set_admission(999) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_admission(8001) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_admission(-2) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_admission(0) == B.TOPK_OK
    assert L.topk_exact_set_admission(3000) == B.TOPK_OK
    assert L.topk_exact_set_admission(-1) == B.TOPK_OK
    # The timing hook takes both events or neither; (NULL, NULL) disarms it.
    assert L.topk_exact_time_next_call(fake, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact_time_next_call(None, fake) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_exact_time_next_call(None, None) == B.TOPK_OK
    # Indexer score producer: shape, head count, head dimension, alignment, null pointers.
    assert L.topk_indexer_scores(fake, fake, fake, fake, -1, 10, 64, 128, fake, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 0, 64, 128, fake, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 2**31, 64, 128, fake, None) == B.TOPK_ERR_BAD_SHAPE
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 10, 64, 64, fake, None) == B.TOPK_ERR_BAD_ARG
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 10, 8, 128, fake, None) == B.TOPK_ERR_BAD_ARG
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 10, 80, 128, fake, None) == B.TOPK_ERR_BAD_ARG
    assert L.topk_indexer_scores(fake + 4, fake, fake, fake, 2, 10, 64, 128, fake, None) == B.TOPK_ERR_BAD_ARG
    assert "aligned" in tk.last_error()
    assert L.topk_indexer_scores(None, fake, fake, fake, 2, 10, 64, 128, fake, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_indexer_scores(fake, fake, fake, fake, 2, 10, 64, 128, None, None) == B.TOPK_ERR_NULL_POINTER
    assert L.topk_indexer_scores(None, None, None, None, 0, 10, 64, 128, None, None) == B.TOPK_OK
    # Sorted variant: the selector's checks, and a misaligned value buffer, before enqueueing.
    so = L.topk_exact_sorted
    assert so(fake, fake, 2, 10, 0, fake, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert so(fake, fake, 2, 10, 4, fake, fake, 3, None) == B.TOPK_ERR_BAD_SENTINEL
    assert so(fake, fake, 2, 10, 4, None, fake, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert so(None, None, 0, 10, 4, None, None, -1, None) == B.TOPK_OK
    # Score + select chain: the checks of both steps run before anything is enqueued.
    ch = L.topk_indexer_topk
    assert ch(fake, fake, fake, fake, 2, 10, 64, 128, 0, fake, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert ch(fake, fake, fake, fake, 2, 10, 64, 128, B.TOPK_K_MAX + 1, fake, fake, -1, None) == B.TOPK_ERR_BAD_K
    assert ch(fake, fake, fake, fake, 2, 10, 64, 128, 4, fake, fake, 3, None) == B.TOPK_ERR_BAD_SENTINEL
    assert ch(fake, fake, fake, fake, 2, 10, 8, 128, 4, fake, fake, -1, None) == B.TOPK_ERR_BAD_ARG
    assert ch(fake, fake, fake, fake, 2, 10, 64, 128, 4, fake, None, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert ch(fake, fake, fake, fake, 2, 10, 64, 128, 4, None, fake, -1, None) == B.TOPK_ERR_NULL_POINTER
    assert ch(fake, fake, fake, fake, -1, 10, 64, 128, 4, fake, fake, -1, None) == B.TOPK_ERR_BAD_SHAPE
    assert ch(None, None, None, None, 0, 10, 64, 128, 4, None, None, -1, None) == B.TOPK_OK


def test_execution_mode_roundtrip():
    L = tk.lib()
    assert L.topk_exact_set_execution(7) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_execution(4) == B.TOPK_ERR_BAD_ARG
    assert L.topk_exact_set_execution(-1) == B.TOPK_ERR_BAD_ARG
    for mode in (B.EXEC_PERSISTENT, B.EXEC_ROW_PER_WG, B.EXEC_ROWSPLIT, B.EXEC_AUTO):
        tk.set_execution(mode)


def test_path_override_roundtrip():
    for mode in (B.PATH_SAMPLED, B.PATH_ROWSPLIT, B.PATH_DIRECT, B.PATH_RECOVERY, B.PATH_AUTO):
        tk.set_path_override(mode)
    with pytest.raises(tk.TopKError):
        tk.set_path_override(12)


def test_binding_rejects_bad_tensors_without_gpu():
    import torch
    with pytest.raises(ValueError):
        tk.topk_exact(torch.zeros(4, 8), torch.zeros(4, dtype=torch.int32), K=2)
