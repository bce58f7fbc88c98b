"""Plain fp64 CPU oracle for per-head causal local-window attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library.

Every function states the passage of "Asymmetric Attention Heads: Structured
Head-Wise Context Allocation for Transformer Attention" (AAH) that it follows.
All functions are pinned by tests that do not route through this package
(library routines, closed forms, invariants, finite differences, the pages'
printed worked example); no function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    window_allowed,
    kv_head,
    attn_fwd_ref,
    attn_fwd_rows_ref,
    attn_bwd_ref,
    pair_count_ref,
    acr_ref,
    acr_from_fractions_ref,
)
from .features import (  # noqa: F401
    N_FEATURES,
    attn_row_stats_ref,
    attn_row_stats_rows_ref,
    head_features_ref,
    features_ema_ref,
)
from .decode import (  # noqa: F401
    cache_rows_ref,
    decode_positions,
    decode_ref,
    cache_content_ref,
)
