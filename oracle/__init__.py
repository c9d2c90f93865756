"""fp64 CPU oracle of the hybrid-window GQA decode attention block.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the library or its binding.
It shares no code with the HIP path.  See ``oracle/block.py`` for the
definitions, their sources on the pages, and the readings taken where the pages
are silent.
"""
from .block import (  # noqa: F401
    AttentionStepResult,
    BlockResult,
    ChunkResult,
    MlpResult,
    OracleSeq,
    StackResult,
    attention_decode,
    attention_step,
    bf16_bits_to_f64,
    block_chunk,
    block_decode,
    decoder_stack_decode,
    embed_gather,
    gelu_erf,
    gemv,
    head_gate,
    kv_slot,
    kv_window,
    lm_head,
    mlp_decode,
    physical_rows,
    rms_norm,
    rope_neox,
    rope_params_for,
    sigmoid,
    split_qkv,
    stack_decode,
    to_fp16,
)
