"""Seeded synthetic inputs for the tree-verification path.

This package only draws random numbers and lays them out in the shapes the
library expects (paged KV cache, block tables, parent arrays, logits, draft
distributions, draft tokens).  It holds none of the verification arithmetic:
both the CPU oracle and the GPU tests/bench take their inputs from here.
"""
from .gen import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_config,
    make_workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    sub_batch,
)
