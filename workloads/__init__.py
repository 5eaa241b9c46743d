"""Seeded synthetic inputs for multi-LoRA shrink/expand.

This package draws the batches (slot indices, activations, adapter weights,
scales, initial outputs) that both the fp64 oracle and the HIP library consume.
It holds none of the method's arithmetic: it only draws numbers and rounds
them to the storage dtype, so the two sides that are compared never share a
line of LoRA code.
"""

from .configs import CONFIGS, CONFIG_ORDER, describe
from .gen import (
    Problem,
    Workload,
    make_workload,
    random_problem,
    EmbeddingProblem,
    random_embedding_problem,
    round_to_dtype,
    bf16_bits_to_f32,
    STORAGE_NP,
)

__all__ = [
    "CONFIGS",
    "CONFIG_ORDER",
    "describe",
    "Problem",
    "Workload",
    "make_workload",
    "random_problem",
    "EmbeddingProblem",
    "random_embedding_problem",
    "round_to_dtype",
    "bf16_bits_to_f32",
    "STORAGE_NP",
]
