"""Seeded synthetic inputs for the sigmoid Top-K router and its expert-bias balancer.

This package turns a workload recipe into input bytes: hidden states, router weights,
the initial expert bias and momentum.  The CPU oracle and the GPU library both consume
exactly these bytes, so the package holds no routing or balancing arithmetic at all:
only random draws, the fp32 -> bf16 rounding of the inputs, and array layout.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    cluster_model,
    duplicate_rows,
    initial_bias,
    initial_momentum,
    router_weight,
    to_bf16_bits,
    tokens,
)
