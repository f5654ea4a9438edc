"""Tensor-parallel transformer shards on AMD Instinct MI355X (gfx950).

The compute lives in ``libtpshard.so`` (HIP kernels behind the C ABI in
``include/tpshard.h``); ``binding`` exposes the same entry points to Python
for torch tensors.  Importing the package loads the library and raises if it
has not been built.
"""

from .binding import (  # noqa: F401
    TPS_BF16, TPS_F32, TpsError, LIB_PATH, lib,
    tps_partition, tps_version,
    tp_mlp_fwd, tp_mlp_bwd, tp_mlp_bwd_workspace,
    tp_attn_fwd, tp_attn_fwd_workspace, tp_attn_bwd, tp_attn_bwd_workspace,
    shard_reduce, shard_reduce_add,
    vocab_embed_fwd, vocab_embed_bwd, vocab_embed_bwd_workspace,
    vocab_embed_bwd_noalloc, vocab_embed_bwd_noalloc_max_tokens,
    tied_logits, tied_logits_bwd,
    vocab_ce_stats, vocab_ce_combine, vocab_ce_bwd,
    column_linear_fwd, column_linear_bwd, row_linear_fwd, row_linear_bwd, shard_reduce_bias,
    shard_reduce_scatter, shard_all_gather, embedding_fwd, dropout_apply,
    layernorm_fwd, layernorm_bwd, layernorm_bwd_workspace, layernorm_bwd_residual,
    trace_start, trace_stop, trace_records, trace_clear,
)
