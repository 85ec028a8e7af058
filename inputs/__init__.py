"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This package generates numbers only. It holds none of the MoE layer's arithmetic: no
routing, no softmax, no permutation, no matmul. Everything here is (seed -> array).
"""
from .generators import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    normal,
    uniform_open01,
    randint,
    permutation,
)
from .workloads import WORKLOADS, Workload, make_ep_share_inputs, make_layer_inputs, workload_inputs  # noqa: F401
