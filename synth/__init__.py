"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package holds workload descriptions and random-input generation only:
none of the arithmetic of the method (shard bounds, packing, RoPE, attention)
lives here, so both the oracle and the GPU path may import it without sharing
any of the computation they are checked on.
"""
from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import (  # noqa: F401
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    gen_tensor,
    gen_gamma,
    gen_qkv,
    sample_rows,
)
