"""MI355X-native blockwise causal attention for one sequence-parallel rank.

Python binding of the gfx950 HIP library ``libea_attn.so`` (C ABI in
include/ea_attn.h): forward with LSE, recompute-based backward, LSE merge of
ring-step partials, zigzag position helpers, rotary position embedding by global
position (also fused into the attention calls), and the fused cross-entropy of
the training step.  PyTorch supplies
device memory and streams only.
"""
from ._lib import (  # noqa: F401
    EA_BF16, EA_F32, EA_MASK_CAUSAL, EA_MASK_FULL, EaError, EXPORTS, KERNELS, LIB_PATH, ea_attn_bwd,
    ea_attn_bwd_rope, ea_attn_fwd, ea_attn_fwd_merge, ea_attn_fwd_rope,
    ea_kernel_name, ea_lse_merge, ea_profile_begin, ea_profile_end, ea_profile_query, ea_ring_source, ea_rope,
    ea_version, ea_xent_fwd_bwd, ea_zigzag_segments, lib, strerror,
)
from .ring import (  # noqa: F401
    DenseCausal, ZigzagRingRank, capture_step, ulysses_shard, ulysses_unshard, zigzag_shard, zigzag_unshard,
)
