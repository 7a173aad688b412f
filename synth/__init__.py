"""Seeded synthetic inputs for the hybrid block-sparse + linear attention layer.

This module is shared by the tests, the CPU oracle's callers and the benchmark.
It only draws numbers: it holds none of the operator's arithmetic (no masks,
no softmax, no linear-attention state).  Everything it returns is plain NumPy.

The workloads stand in, by shape only, for the video-DiT layers the SALAD pages
measure on (Wan2.1 at roughly 30k and 100k tokens); no dataset, prompt or model
weight is involved.
"""

from .configs import CONFIGS, HeadSpec, LayerConfig, get_config
from .generate import LayerInputs, bf16_round, bf16_bits_to_f32, make_grad_output, make_inputs

__all__ = [
    "CONFIGS",
    "HeadSpec",
    "LayerConfig",
    "LayerInputs",
    "bf16_round",
    "bf16_bits_to_f32",
    "get_config",
    "make_grad_output",
    "make_inputs",
]
