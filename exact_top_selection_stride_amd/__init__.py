"""MI355X-native sample-guided exact Top-K selection (HIP kernels for gfx950).

The selection runs in libtopk_exact.so (C ABI in include/topk_exact.h); this
package only marshals torch tensors to it. See `topk_exact`, and `indexer_scores`
/ `indexer_topk` for the FP8 indexer score producer and the score + select chain.
"""
from ._binding import (  # noqa: F401
    EXEC_AUTO, EXEC_PERSISTENT, EXEC_ROW_PER_WG, EXEC_ROWSPLIT, PATH_AUTO, PATH_DIRECT, PATH_RECOVERY,
    PATH_ROWSPLIT, PATH_SAMPLED, STAT_NAMES, TOPK_K_MAX, TopKError, execution, get_stats, last_error, lib,
    path_override, proposal, admission, set_admission, reserve, reset_stats, set_execution, set_path_override, set_proposal,
    stream_read_probe, time_next_call, record_phases, PATH_CODES, PHASE_NAMES, topk_exact, topk_exact_noalloc, topk_exact_sorted, indexer_scores,
    indexer_topk,
)

__all__ = [
    "topk_exact", "topk_exact_noalloc", "topk_exact_sorted", "indexer_scores", "indexer_topk", "reserve", "get_stats", "reset_stats", "set_path_override", "path_override",
    "stream_read_probe", "time_next_call", "record_phases", "PATH_CODES", "PHASE_NAMES", "set_proposal", "proposal", "set_admission", "admission", "last_error", "lib", "TopKError", "TOPK_K_MAX", "STAT_NAMES",
    "PATH_AUTO", "PATH_SAMPLED", "PATH_ROWSPLIT", "PATH_DIRECT", "PATH_RECOVERY",
    "EXEC_AUTO", "EXEC_PERSISTENT", "EXEC_ROW_PER_WG", "EXEC_ROWSPLIT", "set_execution", "execution",
]
