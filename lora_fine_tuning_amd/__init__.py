"""MI355X (gfx950) LoRA linear layer: Y = XW + alpha * (dropout(X) A) B, forward
and backward, single-adapter and mixed-adapter batches.

The compute lives in liblora_fused.so (hand-written HIP kernels behind the C ABI
declared in include/lora_fused.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, LoraAdapter, LoraError, adapter_table, load, lora_check_bubble_lemma,
    lora_dora_norm, lora_dora_norm_workspace_size, lora_dropout_mask, lora_microbatch_segments,
    lora_pack_greedy,
    lora_frozen_bwd, lora_frozen_fwd, lora_linear_bwd, lora_linear_bwd_noalloc,
    lora_linear_bwd_noalloc_max_scratch, lora_linear_bwd_workspace_size,
    lora_linear_fwd, lora_linear_fwd_concat, lora_linear_fwd_workspace_size, lora_profiling_enable,
    lora_profiling_query, lora_profiling_reset, multi_lora_bwd_workspace_size,
    multi_lora_check_segments, multi_lora_fwd_workspace_size, multi_lora_linear_bwd,
    multi_lora_linear_fwd,
)
from .autograd import (  # noqa: F401,E402
    LoraLinear, LoraLinearFunction, MultiLoraLinearFunction, lora_linear, multi_lora_linear,
)
