"""Batched speculative-sampling verify step for MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/specverify.h`` (``libspecverify.so``); this package is its thin
Python binding.
"""

from ._lib import LIB_PATH, load_library, status_string  # noqa: F401
from .api import (  # noqa: F401
    FLAG_BAD_ID,
    FLAG_BAD_SPAN,
    FLAG_EOS,
    FLAG_NONFINITE,
    FLAG_Q_ZERO,
    FLAG_Z_DEGENERATE,
    accept_stats,
    accept_stats_draft_logits,
    draft_logits_workspace_size,
    verify_greedy,
    verify_greedy_ragged,
    verify_sample,
    verify_sample_draft_logits,
    verify_sample_lenient,
    verify_sample_noalloc,
    verify_sample_ragged,
    verify_sample_ragged_draft_logits,
    verify_sample_stats,
    verify_sample_stats_draft_logits,
    workspace_size,
)
