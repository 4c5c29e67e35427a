"""Plain, slow CPU oracle for adaptive block-sparse video attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code with the HIP library or its Python
binding, and computes everything in float64 with numpy.

Every function is pinned by CPU tests against something other than itself
(brute force over subsets, closed forms, dense softmax attention, torch SDPA
with an explicit mask, hand-derived index examples); see tests/test_oracle_*.py.
"""
from .abs_oracle import (  # noqa: F401
    Geometry,
    geometry,
    token_block_slot,
    block_members,
    pool,
    block_probabilities,
    select_row,
    route,
    slack_fill,
    dynamic_slack_fill,
    slack_budget,
    keep_to_csr,
    csr_to_keep,
    sparse_attention,
    dense_attention,
    schedule,
    row_exemptions,
    row_exemption_causes,
    split_units,
    partial_attention,
    merge_partials,
    frame_members,
    frame_pool,
    select_frames_row,
    route_frames,
    sparse_attention_frames,
)
