"""CPU oracle (float64, exact gate logits) -- TEST INFRASTRUCTURE ONLY.

Imported only by tests/, the package smoke check and the benchmark's CPU-baseline
leg.  It shares no code with the HIP library.
"""
from .moe_oracle import (  # noqa: F401
    e4m3_value,
    e8m0_value,
    E4M3_TABLE,
    E8M0_TABLE,
    mx_dequant,
    exact_logits,
    topk_ids,
    softmax_pick_renormalise,
    route,
    route_certified,
    route_replay,
    route_replay_filtered,
    validate_replay_ids,
    dispatch,
    silu,
    expert_ffn,
    layer,
    layer_dense,
    layer_backward,
    expert_backward,
    softmax_pick_grad,
    silu_grad,
    normwise_rel_err,
    e2m1_value,
    E2M1_TABLE,
    e2m1_rne_codes,
    e4m3_rne_codes,
    nvfp4_quantize,
    nvfp4_dequant,
    bf16_rne,
    expert_ffn_nvfp4,
    layer_nvfp4,
)
