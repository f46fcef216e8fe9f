"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This package holds no attention arithmetic: it only draws random tensors,
rounds them to the storage type and describes the workloads by shape.
"""
from .inputs import (  # noqa: F401
    DECODE_WORKLOADS,
    GQA_WORKLOADS,
    VARLEN_WORKLOADS,
    WORKLOADS,
    GqaWorkload,
    VarlenWorkload,
    Workload,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    decode_lengths,
    f32_to_bf16_bits,
    make_inputs,
    make_gqa_inputs,
    make_varlen_inputs,
    make_workload_inputs,
    varlen_lengths,
    spike_positions,
)
