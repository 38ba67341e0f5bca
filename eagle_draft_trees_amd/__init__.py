"""MI355X (gfx950) EAGLE-2 draft round: HIP kernels behind a C ABI
(include/eagle_mi355x.h) with a thin ctypes binding."""
from . import _lib
from ._lib import (EagleError, eagle_draft_extend, eagle_draft_level, eagle_last_error,
                   eagle_rerank_build_tree, eagle_status_str, eagle_verify_greedy,
                   eagle_verify_relaxed,
                   eagle_workspace_bytes, eagle_workspace_init, eagle_ws_view)

__all__ = ["EagleError", "eagle_draft_extend", "eagle_draft_level", "eagle_last_error",
           "eagle_rerank_build_tree", "eagle_status_str", "eagle_verify_greedy",
           "eagle_verify_relaxed",
           "eagle_workspace_bytes", "eagle_workspace_init", "eagle_ws_view", "_lib"]
