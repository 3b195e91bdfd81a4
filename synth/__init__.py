"""Seeded synthetic inputs for the segment-routed multi-adapter LoRA delta.

This package is shared by the CPU oracle side (tests) and the GPU side (tests, bench).
It only *draws* raw inputs:

* request lengths and per-request slot ids (-1 = base model),
* per-slot adapter ranks,
* unscaled per-projection adapter matrices in the PEFT layout
  (``lora_A`` [r, in], ``lora_B`` [out, r], fp32) and LoRA biases [out],
* activations ``x`` and base-layer outputs ``y``.

It performs none of the method's arithmetic: no scaling, padding, QKV fusion,
casting to the stack dtype, sorting or grouping.  For bf16 workloads the
activations are drawn in fp32 and their low 16 bits are cleared, so every value
is exactly a bf16 value and both sides read identical numbers.
"""

from .workloads import (  # noqa: F401
    MLP_PROJECTIONS,
    PROJECTIONS,
    WORKLOADS,
    Workload,
    bf16_bits,
    draw_activations,
    draw_adapter,
    draw_bias,
    draw_mlp_activations,
    draw_mlp_adapter,
    draw_ranks,
    draw_requests,
    get_workload,
)
