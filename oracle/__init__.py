"""fp64 CPU oracle of one small-batch MoE decode-layer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library (``moe_layer_skinny_amd``) and imports nothing
from it; both sides get their inputs from ``synth``.

See ``oracle.layer`` for the definitions and the passages they follow.
"""
from .layer import (  # noqa: F401
    LayerWeights,
    as_f64,
    chain_step,
    gates_for,
    layer_step,
    oproj_residual,
    rms_norm,
    round_to_bf16,
    round_to_f32,
    router_logits,
    routing_tables,
    selection_keys,
    sigmoid,
    silu,
    swiglu_expert,
    topk_gap,
    topk_sets,
)
