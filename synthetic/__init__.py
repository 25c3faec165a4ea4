"""Seeded synthetic inputs shared by the parity tests, the benchmark and the smoke check.

This module only draws random numbers and lays them out in memory. It holds none of the
method's arithmetic (no scores, no selection, no attention), so both the oracle side and
the HIP side can take their inputs from it without sharing any computation.

Workloads (shapes and value distributions) follow the dynamic-sparse attention setting of
the page "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理全解析" (ruibaoantu.com),
§2.2 (KV cache held in fixed-size blocks of contiguous tokens) and §2.4 (a vision prefix
that is always attended).
"""
from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .generate import (  # noqa: F401
    Inputs,
    make_inputs,
    bf16_bits,
)
