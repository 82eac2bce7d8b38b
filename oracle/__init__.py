"""CPU oracle for the co-activation-aware MoE dispatch path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the engine in
``co_activation_amd`` never does, and this package never imports it.
"""

from .coact import (  # noqa: F401
    OracleInputError,
    validate_routing,
    validate_placement,
    source_offsets,
    source_rank_of_tokens,
    coact_stats,
    ochiai,
    dispatch_plan,
    dispatch_plan_gathered,
    permute_rows,
    scatter_rows,
    combine,
    combine_unweighted,
    bf16_round,
    bf16_to_f32,
    shuffle_predict,
    two_layer_pipeline,
    shuffle_dispatch,
    expert_plan,
    partial_combine,
    moe_output,
    permute_scaled,
    row_dot,
    ema_update,
    colocated_coactivation,
    place_experts,
    shuffle_balanced,
)
