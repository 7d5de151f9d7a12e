"""Seeded synthetic inputs for the folded multi-branch verification layer.

This package is the only code shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It holds no step of the method itself: it draws
random weights, prefix KV caches, parent trees and hidden states, and it rounds
inputs to bfloat16.  Every draw is made with ``numpy.random.default_rng`` (PCG64)
seeded by ``[base_seed, step, layer, tensor_id]``, so any single tensor of any
workload can be regenerated on its own.
"""

from .inputs import (  # noqa: F401
    Shape,
    Workload,
    WORKLOADS,
    bf16_bits,
    bf16_round,
    bf16_bits_to_f32,
    child_hidden,
    device_layer,
    layer_weights,
    main_hidden,
    parent_tree,
    prefix_kv,
    step_inputs,
    step_tokens,
    tree_of,
)
