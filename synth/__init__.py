"""Seeded synthetic inputs and the workload table.

This module is shared by the oracle side (tests, the bench's CPU leg) and the
HIP side (tests, bench) and by nothing else.  It holds no arithmetic of the
attention method: it only draws Gaussian tensors and rounds them to the
storage dtype the kernels read, so that both sides see bit-identical inputs.
"""
from .workloads import CONFIGS, Workload, gen_block_mask, gen_head, gen_qkv, to_storage

__all__ = ["CONFIGS", "Workload", "gen_block_mask", "gen_head", "gen_qkv", "to_storage"]
