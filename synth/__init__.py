"""Seeded synthetic inputs for the MapFlow hot path (compress + fused retrieve).

This package holds random draws only: normal vectors, unit vectors, hot key positions,
Dirichlet rows, sequence lengths and page permutations.  It contains no step of the method
itself, so both the fp64 oracle (``oracle/``) and the GPU path can consume its arrays without
sharing any of the method's arithmetic.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    cu_seqlens_of,
    make_dense_inputs,
    make_dense_inputs_torch,
    make_layer_inputs,
    make_layer_inputs_torch,
    make_page_table,
    make_receiver_inputs_torch,
    make_sender_inputs_torch,
    make_lengths,
    page_v,
    rng_for,
)
