"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package generates random tensors and holds the workload shape table.  It
contains none of the MoE layer's arithmetic (no routing, no dispatch, no
expert math): those live in ``oracle/`` (the CPU checker) and in the HIP
library, which never import each other.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits,
    bf16_bits_to_f32,
    round_bf16,
    make_workload,
    device_expert_weights,
    host_expert_weights,
    router_bias,
    zipf_bias,
)
