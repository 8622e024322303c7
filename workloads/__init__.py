"""Seeded synthetic inputs for the attention forward workloads.

This module is shared by the tests, the benchmark and the smoke check. It holds
no attention or quantisation arithmetic: it only draws random numbers, rounds
them once to bfloat16 or float16 (that rounding *is* the input definition) and builds the
block masks and sequence lengths. Both the HIP path and the oracle consume the
same bytes produced here.

Every random tensor is drawn per (config, tensor, head) from its own
``numpy.random.SeedSequence``, so any subset of heads can be regenerated
without drawing the others.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_block_keep,
    make_workload,
    random_bf16,
    random_f16,
    varlen_lengths,
)
