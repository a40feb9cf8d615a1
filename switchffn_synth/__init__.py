"""Seeded synthetic inputs for the SwitchFFN forward pass.

This module serves both the CPU oracle and the HIP path with the same bytes.
It holds none of the method's arithmetic: it only states the workload shapes
and draws the inputs (token states x, router weights Wr, expert weights and
biases) from a counter-based generator whose element definition is in
``csrc/synth_common.h``.  The host filler (C) and the device filler (HIP)
implement that one definition, so any slice of a tensor -- one expert's
weights, a sample of tokens -- can be regenerated on the CPU without moving
the device copy.
"""
from .workloads import WORKLOADS, Workload, workload  # noqa: F401
from .generate import (  # noqa: F401
    STREAMS,
    bf16_bits_to_f32,
    decode,
    device_inputs,
    expert_weights_host,
    host_array,
    host_rows,
    host_inputs,
    zipf_router_bias,
)
