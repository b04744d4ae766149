"""CPU oracle for the sequence-parallel reduce + add + RMSNorm (+FP8) shard path.

TEST INFRASTRUCTURE ONLY.  The product package never imports this package;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may.  It shares no code with the HIP implementation.
"""

from .oracle import (  # noqa: F401
    ORC_BF16,
    ORC_E2M1,
    ORC_E4M3,
    ORC_F32,
    QUANT_DYNAMIC_TOKEN,
    QUANT_MX_BLOCK,
    QUANT_NONE,
    QUANT_STATIC_TENSOR,
    AbiProblem,
    OracleError,
    all_gather_unpad,
    bf16_from_double,
    bf16_from_double_array,
    bf16_to_double,
    build,
    dsacp_heads_to_tokens,
    e2m1_from_double,
    e2m1_from_double_array,
    e2m1_to_double,
    e4m3_from_double,
    e4m3_from_double_array,
    e4m3_to_double,
    fc2_batch_ids,
    fc2_regroup,
    matmul_scatter,
    reduce_add_rmsnorm,
    scaled_matmul_scatter,
    shard_geometry,
    sp_oracle_reduce_add_rmsnorm,
)
