"""Seeded synthetic inputs and the named workloads.

This package holds no step of the attention method: only workload sizes and
parameters and seeded random tensors. Tests, the benchmark and the smoke check
call it, and pass what it returns both to the library and to the oracle.
"""
from .workloads import Workload, TINY, SMALL, HEADLINE, HEADLINE_B3, P1440, WORKLOADS
from .inputs import normal_qkv, planted_qkv, sample_indices, census_qkv

__all__ = ["Workload", "TINY", "SMALL", "HEADLINE", "HEADLINE_B3", "P1440", "WORKLOADS",
           "normal_qkv", "planted_qkv", "sample_indices", "census_qkv"]
