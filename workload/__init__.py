"""Seeded synthetic inputs shared by the CPU oracle, the HIP path, the tests and the bench.

This package only *creates* inputs: activations, routing decisions and packed expert
blobs.  It holds none of the routed-expert computation (no decode, no grouping, no FFN,
no combine).  The packers encode the two block formats; decoding them is done separately
by the oracle and by the HIP kernels, and the oracle's decoder is pinned by hand-packed
blocks that do not go through these packers.  The routing decisions of the layer workloads are
drawn here in numpy float64 as layer inputs; the router row itself (fp32 logits in, ids and
weights out) has its own oracle and kernel, which take only `gen_logits` from this package.
"""
from .gen import (  # noqa: F401
    QTYPE_Q2B,
    QTYPE_T1,
    BLOCK_VALUES,
    BLOCK_BYTES,
    DESC_DTYPE,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    gen_x,
    gen_logits,
    route_softmax_topk,
    zipf_bias,
    pack_q2b,
    pack_t1,
    pack_matrix,
    matrix_bytes,
    Experts,
    make_experts,
    Workload,
    make_workload,
    BlockWorkload,
    make_block_workload,
    CONFIGS,
)
