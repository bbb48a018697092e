"""CPU oracle of the routed-expert MoE layer -- test infrastructure only.

Only tests, the smoke check and the bench's CPU-baseline leg may import this package.
The product path (the HIP library and its binding) never imports it.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    lib_path,
    fp16_to_double,
    bf16_to_double,
    dequant,
    group_pairs,
    moe_prefill,
    moe_workload,
    moe_block,
    default_threads,
    route,
)
