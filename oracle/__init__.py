"""fp64 CPU oracle for the DeepSeekMoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__
and the CPU-baseline leg of bench.py may import anything from this package.
The HIP library never calls into it and it never calls into the HIP library;
the two share nothing except the seeded inputs from `synth`.

Every function is pinned by tests/test_oracle_pins.py (the layer) and
tests/test_oracle_stats_pins.py (routing statistics) and
tests/test_oracle_capacity_pins.py (capacity-limited dispatch) and
tests/test_oracle_decode_pins.py (bf16 storage decoding) against closed forms,
special cases and a pure-Python brute force (see tests/_brute.py).
"""
from .moe import (  # noqa: F401
    decode,
    dispatch,
    expert_ffn,
    ffn_of,
    relu_ffn,
    forward,
    gate_values,
    route,
    route_on,
    route_selection_bias,
    noisy_logits,
    selection_and_gate_logits,
    softplus,
    router_logits,
    select_topk,
    shared_ffn,
    silu,
    softmax,
)
from .gap import enforce_gap, topk_gap  # noqa: F401
from .stats import routing_stats  # noqa: F401
from .capacity import capacity_for, dispatch_capacity, keep_mask  # noqa: F401
