"""MI355X routed-expert MoE layer on 1.8-2.3-bit block-quantized experts.

A thin binding of the C ABI in include/rl_moe.h (librl_moe.so, HIP for gfx950).  Every
step of the layer runs in the library's kernels; this package only marshals arguments and
takes device memory and streams from PyTorch.  Importing it does not need a GPU; calling it
needs the built library and fails loudly without it.
"""
from ._binding import (  # noqa: F401
    RL_OK,
    RL_QTYPE_Q2B,
    RL_QTYPE_T1,
    RL_DEC_STRIP,
    RL_DEC_MFMA_GATEUP,
    RL_DEC_MFMA_DOWN,
    RL_DEC_ROWS_GATEUP,
    RL_DEC_ROWS_DOWN,
    t1_splits_h,
    RlError,
    DeviceExperts,
    lib,
    lib_path,
    exported_symbols,
    workspace_bytes,
    alloc_workspace,
    prefill,
    prefill_timed,
    prefill_noalloc,
    prefill_block,
    decode_block,
    prefill_from_logits,
    ExpertCache,
    CachedExperts,
    noalloc_status,
    NOALLOC_SCRATCH_BYTES,
    TIMED_EVENTS,
    decode,
    gate_up,
    group_pairs,
    dequant,
    route,
    status,
    strerror,
)
