"""MI355X (gfx950) hybrid-window GQA decode attention block.

The compute path is ``libgqa.so`` (hand-written HIP kernels behind the C ABI
in ``include/gqa.h``); this package is its thin Python binding.  PyTorch only
provides device memory and streams.
"""
from .binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    Arch,
    GqaError,
    KvSeq,
    PreparedBlock,
    PreparedLayer,
    PreparedMlp,
    PreparedStack,
    StackLayer,
    attention_block_chunk,
    attention_block_decode,
    attention_block_decode_noalloc,
    attention_gated,
    attention_layer_decode,
    attention_partials,
    attention_stack_decode,
    embed_tokens,
    kv_slot,
    kv_window,
    library_path,
    lm_head,
    lm_head_workspace_size,
    mlp_decode,
    mlp_workspace_size,
    o_proj_gemv,
    qkv_rope_kv,
    residual_add,
    rms_norm_bf16w,
    rope_params_for,
    split_plan,
    workspace_size,
)
