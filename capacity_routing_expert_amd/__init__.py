"""Capacity-limited Mixture-of-Experts layer forward pass for AMD Instinct MI355X (gfx950).

The layer runs in libmoe (hand-written HIP, C interface in include/moe.h); `binding` is its
ctypes wrapper, `layer` a torch-side convenience for allocation, `workloads` the seeded
synthetic inputs.  Build the library with `python -m capacity_routing_expert_amd.build`.
"""
from . import workloads  # noqa: F401

__all__ = ["workloads", "binding", "layer", "build"]
