"""Seeded synthetic workloads for the weight-only block-INT4 MatMul.

This package holds only shapes and seeded random inputs: it contains none of
the method's arithmetic (no packing, no dequantization, no matmul), so both the
CPU oracle's tests and the GPU path may draw their inputs from it.
"""

from .qwen3 import CONFIGS, Launch, Workload, workload  # noqa: F401
from .generate import ProjectionInputs, projection_inputs, seed_for  # noqa: F401
