"""Seeded synthetic inputs for the EAGLE tree-verification path.

This package only *draws* inputs (query/key/value tensors, target and draft
logits, draft trees and their tokens).  It holds none of the verification
arithmetic: no attention, no acceptance rule, no residual.  Both the HIP path
and the CPU oracle consume the arrays it returns, bit for bit.
"""
from .inputs import (  # noqa: F401
    WorkloadSpec, Inputs, CONFIGS, config_spec, make_inputs, make_tree,
    to_bf16_bits, bf16_bits_to_f64, kv_head_block,
)
