"""Seeded synthetic workloads for the sharded optimizer step.

This package is shared by the tests, the smoke check and the benchmark, on both the HIP side and
the oracle side. It holds only shapes, seeds and random draws: no partitioning, summation, Adam or
casting arithmetic lives here. Callers pass in the shard offset and size they computed themselves.

  shapes  parameter lists of the model shapes (GPT-2 small, Llama 7B/13B, GPT-3 175B), their flat
          element counts and the init kind of each flat range
  host    numpy generators (small workloads, fully on the CPU)
  device  torch generators on a GPU (the large workloads; bytes never leave HBM unless a test
          downloads a window to check it)
"""

from .shapes import (
    MODELS,
    WORKLOADS,
    Workload,
    flat_count,
    param_list,
    init_ranges,
    layer_ranges,
)

__all__ = ["MODELS", "WORKLOADS", "Workload", "flat_count", "param_list", "init_ranges", "layer_ranges"]
