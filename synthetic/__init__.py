"""Seeded synthetic inputs for the paged-attention workloads.

This package draws random numbers and nothing else: sequence lengths,
initial free-list orders, pool contents, new K/V rows and queries.  It holds
none of the method's arithmetic (no block tables, slot mappings, attention or
quantisation); both the HIP path's harness and the CPU oracle take their
inputs from here and each builds everything else on its own.
"""
from .configs import (  # noqa: F401
    Workload, StepDraw, RequestStream, normal_f16, normal_bf16, round_bf16, config1, config2, config3, config4,
    config5, config6, CONFIGS, custom,
)
