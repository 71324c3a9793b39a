"""CPU oracle for the int4 GPTQ and dense GEMMs -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The library itself never calls it, and it calls
nothing of the library: the two share no code.
"""
from .qgemm_oracle import (  # noqa: F401
    GROUP_SIZE,
    TOL_ABS,
    TOL_REL,
    fp16_value,
    bf16_value,
    fp32_value,
    unpack_qweight,
    unpack_qzeros,
    dequant,
    qgemm_int4,
    qgemm_int4_at,
    qgemm_int4_lora,
    qgemm_int4_lora_at,
    row_sumsq,
    row_sumsq_bound,
    dense,
    dense_at,
    dense_batched,
    dense_absdot,
    accept_fp32,
    compare_fp32,
    dense_batched_at,
    grid_bracket,
    round_to_grid,
    accept,
    compare,
)
