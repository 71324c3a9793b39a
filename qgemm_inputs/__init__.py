"""Seeded synthetic inputs for the int4 GPTQ and dense GEMM workloads.

This module is shared by the CPU oracle, the GPU tests and the benchmark.  It
produces raw storage bytes only (packed words, bf16/fp16 bit patterns) and holds
none of the arithmetic of the products themselves: no unpacking, no dequant, no
accumulation.  See `gen.py` for the generator definition and `configs.py` for
the workload shapes.
"""
from .gen import (  # noqa: F401
    SplitMix64,
    f32_to_bf16_bits,
    f64_to_fp16_bits,
    f64_to_fp32_bits,
    int4_inputs,
    dense_inputs,
    dense_batched_inputs,
    lora_inputs,
)
from .configs import (  # noqa: F401
    INT4_CONFIGS, DENSE_CONFIGS, ATTENTION_CONFIG, int4_cases, dense_cases, attention_cases,
)
