"""One GPU's share of Ulysses sequence parallelism on MI355X (gfx950).

The hot path (layout swaps around the all-to-all, causal GQA attention
forward and backward, dense or packed documents) runs in libulysses.so,
hand-written HIP for gfx950; this package is its thin Python binding. The
same attention calls plus a merge of per-block results and a sum of
per-block gradients also serve ring attention, the variant the pages
contrast with Ulysses; the shifted-label loss and its weighted aggregation
over the SP ranks close the step; TiledMLP runs the model's MLP over token
tiles.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    STATUS,
    CODE,
    NOALLOC_SCRATCH_BYTES,
    UlyssesError,
    attn_bwd,
    attn_bwd_dkdv,
    attn_bwd_dq,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fwd_noalloc,
    attn_fwd_workspace_bytes,
    attn_lse_merge,
    raw,
    ring_grad_sum,
    shifted_ce_bwd,
    shifted_ce_fwd,
    sp_loss_aggregate,
    status_string,
    tiled_mlp_bwd,
    tiled_mlp_fwd,
    tiled_mlp_workspace_bytes,
    ulysses_check_cu_seqlens,
    ulysses_head_to_seq,
    ulysses_seq_to_head,
    ulysses_shard_len,
)
