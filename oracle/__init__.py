"""fp64 CPU oracle of the Sol-Attn sparse attention forward.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP implementation.
"""
from .oracle import (  # noqa: F401
    attend,
    attend_head,
    block_bounds,
    block_means,
    gauss_threshold,
    gauss_threshold_diag,
    proxy_scores,
    route,
    route_head,
    topk_mask,
    topp_mask,
)
