"""Seeded synthetic workloads for paged-KV chunk attention.

This package only draws inputs (shapes, value laws, page tables).  It holds
none of the attention arithmetic, so both the HIP library's tests and the
fp64 oracle can take their inputs from here without sharing any code of the
method itself.
"""
from .configs import CONFIGS, Config, get_config, mini_config  # noqa: F401
from .gen import ChunkInputs, Workload  # noqa: F401
