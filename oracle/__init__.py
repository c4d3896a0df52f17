"""CPU oracle of the decode-step MoE layer (test infrastructure only).

Plain, slow, float64 implementations of what the layer computes, written from
the vLLM API pages on the GLM-5.3-Flash specialized decode (module
``vllm.models.glm5next.nvidia.specialized_decode.runtime.decode``, class
``LayerStages``; module ``...runtime.draft``, class ``SpecializedDraft``).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package.  The product path (the HIP library and its
Python binding) never does, and shares no code with it.

Two independent versions live here:
  moe_oracle.py  NumPy, float64, the readable definition (small and sampled runs)
  moe_oracle.c   C, float64, OpenMP over output rows (full-size runs, CPU baseline)
"""

from .moe_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    e4m3_codes_to_f64,
    e8m0_bytes_to_f64,
    dequantize,
    router_logits,
    sigmoid,
    select_experts,
    route_weights,
    clamped_swiglu,
    expert_mlp,
    route_table,
    rms_norm,
    moe_layer,
    dense_layer,
    score_gaps,
)
