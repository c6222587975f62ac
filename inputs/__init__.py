"""Seeded synthetic inputs shared by the CPU oracle and the HIP library's tests.

This package holds no attention arithmetic: it only draws random tensors and applies the
input constructions (duplicated key rows, an attention-sink key, a value grid, rows with a
repeated maximum of chosen sign) that the workloads and tests call for.
"""
from .gen import (CONFIGS, WorkloadConfig, make_inputs, randn_inputs, grid_inputs, rect_inputs,
                  tied_maxima_inputs, tensor_digest)

__all__ = ["CONFIGS", "WorkloadConfig", "make_inputs", "randn_inputs", "grid_inputs", "rect_inputs",
           "tied_maxima_inputs", "tensor_digest"]
