"""One decode step of one layer through the library: copy-on-write block copies, the new tokens'
slot-mapped write, then paged attention over every sequence.

The order follows the pages: a block still shared by another sequence is copied before a token is
written into it ("PagedAttention", Ultralytics glossary, section "シーケンス間でのブロック共有"),
the new token's K/V go into their slots (same page, "ページングの仕組み"), and the query then
attends all cached tokens including its own (the podcast transcript's paragraph on decode: each new
token reads the keys and values of every earlier token).
"""

from __future__ import annotations

from . import lib


def decode_step(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new, slot_mapping,
                cow_pairs, scale: float, k_scale=None, v_scale=None, partition_tokens: int = 0,
                variant: int = lib.PA_VARIANT_AUTO, workspace=None, stream=None,
                flags: int = 0, fused: bool = True) -> None:
    """All tensors on the GPU; ``cow_pairs`` is int32 [n][2] (n may be 0). ``flags`` as for
    ``pa_decode`` (PA_DECODE_SHARED_BLOCKS when sequences of the batch share blocks). With
    ``fused`` the slot write rides along with the attention (pa_decode_append: one launch fewer,
    the new token taken from k_new / v_new); otherwise pa_write_kv then pa_decode."""
    if cow_pairs is not None and cow_pairs.shape[0] > 0:
        lib.pa_copy_blocks(k_cache, v_cache, cow_pairs, k_scale, v_scale, stream=stream)
    if fused:
        lib.pa_decode_append(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                             slot_mapping, scale, k_scale, v_scale,
                             partition_tokens=partition_tokens, variant=variant,
                             workspace=workspace, stream=stream, flags=flags)
        return
    lib.pa_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=stream)
    lib.pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                  partition_tokens=partition_tokens, variant=variant, workspace=workspace,
                  stream=stream, flags=flags)


def workspace_for(q, k_cache, block_tables, block_size: int, partition_tokens: int = 0):
    """A uint8 GPU tensor sized for pa_decode (None when no workspace is needed); ``k_cache`` is the
    key pool [num_blocks][num_kv_heads][block_size][head_dim]."""
    import torch
    S, Hq, D = q.shape
    n = lib.pa_decode_workspace_bytes(S, Hq, k_cache.shape[1], D, block_tables.shape[1], block_size,
                                      partition_tokens)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=q.device)


def grouped_workspace_for(q, block_tables, block_size: int, partition_tokens: int = 0):
    """A uint8 GPU tensor sized for pa_decode_grouped."""
    import torch
    S, Hq, D = q.shape
    n = lib.pa_decode_grouped_workspace_bytes(S, Hq, D, block_tables.shape[1], block_size,
                                              partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def decode_step_grouped(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                        slot_mapping, cow_pairs, group_start, prefix_blocks, max_group_size: int,
                        scale: float, k_scale=None, v_scale=None, partition_tokens: int = 0,
                        workspace=None, stream=None, flags: int = 0, fused: bool = True) -> None:
    """The decode step of a batch whose sequences share prefix blocks (``group_start`` /
    ``prefix_blocks`` as ``blocks.shared_prefix_groups`` returns them, on the GPU): copies, then
    pa_decode_grouped, which reads each shared block once per group, with the slot write taken
    along (``fused``: pa_decode_grouped_append) or as pa_write_kv before it."""
    if cow_pairs is not None and cow_pairs.shape[0] > 0:
        lib.pa_copy_blocks(k_cache, v_cache, cow_pairs, k_scale, v_scale, stream=stream)
    if workspace is None:
        workspace = grouped_workspace_for(q, block_tables, k_cache.shape[2], partition_tokens)
    if fused:
        lib.pa_decode_grouped_append(out, q, k_cache, v_cache, block_tables, context_lens, k_new,
                                     v_new, slot_mapping, group_start, prefix_blocks,
                                     max_group_size, scale, k_scale, v_scale,
                                     partition_tokens=partition_tokens, workspace=workspace,
                                     stream=stream, flags=flags)
        return
    lib.pa_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=stream)
    lib.pa_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                          prefix_blocks, max_group_size, scale, k_scale, v_scale,
                          partition_tokens=partition_tokens, workspace=workspace, stream=stream,
                          flags=flags)
