"""Seeded synthetic inputs for the MoE-layer forward.

This module is the only code the CPU oracle and the HIP path have in common:
it draws the layer's inputs (activations, gate, expert weights, replayed IDs and
weights) from seeded generators and encodes them in the storage formats the
layer consumes (bf16, fp32, OCP MXFP8).  It computes none of the layer's own
arithmetic (no logits, no routing, no matmuls).
"""
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    make_layer_inputs,
    make_gate_inputs,
    zipf_replay_ids,
    dirichlet_weights,
    mxfp8_quantize,
    nvfp4_quantize,
    bf16_round,
)
