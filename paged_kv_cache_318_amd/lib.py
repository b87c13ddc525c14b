"""ctypes binding of ``libpagedattn.so`` (declared in ``include/pa.h``).

Argument marshalling only: each function takes torch tensors on the GPU, checks dtype / device /
contiguity / shape consistency, and passes raw pointers, sizes and the current HIP stream to the
C entry point of the same name. Every step of the computation runs in the library's HIP kernels;
if the library is missing this module raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_VARIANT_AUTO, PA_VARIANT_VALU, PA_VARIANT_MFMA = 0, 1, 2
PA_DECODE_SHARED_BLOCKS = 1
PA_KERNEL_DECODE_PARTITION, PA_KERNEL_DECODE_MERGE, PA_KERNEL_WRITE_KV, PA_KERNEL_COPY_BLOCKS, \
    PA_KERNEL_GATHER_KV, PA_KERNEL_SWAP_BLOCKS, PA_KERNEL_PREFILL = range(7)
PA_SWAP_OUT, PA_SWAP_IN = 0, 1
STATUS = {0: "PA_OK", -1: "PA_ERR_INVALID_ARG", -2: "PA_ERR_UNSUPPORTED", -3: "PA_ERR_WORKSPACE",
          -4: "PA_ERR_HIP"}

LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

_lib: Optional[ctypes.CDLL] = None

_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "pa_status_string": ([_i32], ctypes.c_char_p),
    "pa_version": ([], _i32),
    "pa_write_kv": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                     _vp], _i32),
    "pa_copy_blocks": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp], _i32),
    "pa_gather_kv": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                      _vp], _i32),
    "pa_decode_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "pa_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                   _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp], _i32),
    "pa_decode_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp,
                          _sz, _vp], _i32),
    "pa_decode_noalloc": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                           _f32, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "pa_decode_grouped_workspace_bytes": ([_i32, _i32, _i32, _i32, _i32, _i32], _sz),
    "pa_decode_grouped": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                           _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32, _vp, _vp, _i32, _i32,
                           _vp, _sz, _vp], _i32),
    "pa_decode_grouped_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                  _i32, _vp, _vp, _i32, _i32, _vp, _sz, _vp], _i32),
    "pa_prefill": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                    _i32, _i32, _f32, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "pa_swap_blocks": ([_vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                        _i32, _i32, _i32, _vp], _i32),
    "pa_diag_read_bandwidth": ([_vp, _sz, _vp, _i32, _i32, _vp, _vp], _i32),
    "pa_profile_enable": ([_i32], _i32),
    "pa_profile_read": ([_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong)],
                        _i32),
}


class PagedAttnError(RuntimeError):
    """A libpagedattn entry point returned a non-zero pa_status."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Open the library once (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m paged_kv_cache_318_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedAttnError(fn, status)


def dtype_code(t) -> int:
    import torch
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
         torch.uint8: PA_FP8_E4M3, torch.float8_e4m3fn: PA_FP8_E4M3}
    if t.dtype not in m:
        raise ValueError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libpagedattn must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpagedattn must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def pa_status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def pa_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None,
                stream=None) -> None:
    """k_new/v_new [T][Hkv][D]; k_cache [NB][Hkv][B][D]; v_cache [NB][Hkv][D][B]; slots int32 [T]."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    T = slot_mapping.shape[0]
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(tuple(k_new.shape) == (T, Hkv, D) and tuple(v_new.shape) == (T, Hkv, D),
          "k_new/v_new must be [T][Hkv][D]")
    _need(slot_mapping.dtype == torch.int32, "slot_mapping must be int32")
    _check("pa_write_kv", load().pa_write_kv(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv, D, B,
        NB, dtype_code(k_new), dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, k_scale=None, v_scale=None, stream=None) -> None:
    """block_pairs int32 [n][2] = (src, dst)."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    _need(block_pairs.dtype == torch.int32 and block_pairs.dim() == 2 and block_pairs.shape[1] == 2,
          "block_pairs must be int32 [n][2]")
    n = block_pairs.shape[0]
    _check("pa_copy_blocks", load().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_pairs) if n else None, n, Hkv, D, B, NB, dtype_code(k_cache), _stream(stream)))


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
               max_query_len: int, k_scale=None, v_scale=None, stream=None) -> None:
    """``q``/``out`` [T][Hq][D]; ``query_start`` int32 [S+1] (sequence s owns rows
    query_start[s] .. query_start[s+1]-1); ``context_lens`` counts each sequence's cached tokens
    including its new ones; ``max_query_len`` >= every sequence's number of rows."""
    import torch
    T, Hq, D = q.shape
    NB, Hkv, B, Dk = k_cache.shape
    S, MB = block_tables.shape
    _need(Dk == D and tuple(v_cache.shape) == (NB, Hkv, D, B), "cache shapes do not match q")
    _need(tuple(out.shape) == (T, Hq, D), "out must be [T][Hq][D]")
    _need(tuple(query_start.shape) == (S + 1,) and query_start.dtype == torch.int32,
          "query_start must be int32 [S+1]")
    _need(tuple(context_lens.shape) == (S,) and context_lens.dtype == torch.int32,
          "context_lens must be int32 [S]")
    _need(block_tables.dtype == torch.int32, "block_tables must be int32")
    _check("pa_prefill", load().pa_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start), S, T, int(max_query_len), Hq, Hkv, D, B, MB, NB, float(scale),
        dtype_code(q), dtype_code(k_cache), dtype_code(out), _ptr(k_scale), _ptr(v_scale),
        _stream(stream)))


def _host_ptr(t) -> Optional[int]:
    if t is None:
        return None
    if t.is_cuda or not t.is_pinned():
        raise ValueError("host pools passed to pa_swap_blocks must be pinned host tensors")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpagedattn must be contiguous")
    return t.data_ptr()


def pa_swap_blocks(k_cache, v_cache, host_k, host_v, block_pairs, direction: int, k_scale=None,
                   v_scale=None, host_k_scale=None, host_v_scale=None, stream=None) -> None:
    """Device pool <-> pinned host pool of the same block shape. ``block_pairs`` int32 [n][2] =
    (src, dst) on the GPU or in pinned host memory; PA_SWAP_OUT copies device block src to host
    block dst, PA_SWAP_IN host block src to device block dst."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    NH = host_k.shape[0]
    _need(tuple(host_k.shape[1:]) == (Hkv, B, D) and tuple(host_v.shape) == (NH, Hkv, D, B),
          "host pools must be keys [num_host_blocks][Hkv][B][D], values [num_host_blocks][Hkv][D][B]")
    _need(host_k.dtype == k_cache.dtype and host_v.dtype == v_cache.dtype, "host pool dtype differs")
    _need(block_pairs.dtype == torch.int32 and block_pairs.dim() == 2 and block_pairs.shape[1] == 2,
          "block_pairs must be int32 [n][2]")
    n = block_pairs.shape[0]
    pairs = None
    if n:
        pairs = _ptr(block_pairs) if block_pairs.is_cuda else _host_ptr(block_pairs)
    _check("pa_swap_blocks", load().pa_swap_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), NB, _host_ptr(host_k),
        _host_ptr(host_v), _host_ptr(host_k_scale), _host_ptr(host_v_scale), NH, pairs, n,
        direction, Hkv, D, B, dtype_code(k_cache), _stream(stream)))


def pa_gather_kv(k_out, v_out, k_cache, v_cache, block_tables, context_lens, stream=None) -> None:
    """k_out/v_out [S][max_tokens][Hkv][D] in the cache dtype."""
    NB, Hkv, B, D = k_cache.shape
    S, MB = block_tables.shape
    max_tokens = k_out.shape[1]
    _need(tuple(k_out.shape) == (S, max_tokens, Hkv, D) and k_out.shape == v_out.shape,
          "k_out/v_out must be [S][max_tokens][Hkv][D]")
    _check("pa_gather_kv", load().pa_gather_kv(
        _ptr(k_out), _ptr(v_out), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), S, Hkv, D, B, MB, NB, max_tokens, dtype_code(k_cache), _stream(stream)))


def pa_decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                              max_blocks_per_seq: int, block_size: int,
                              partition_tokens: int = 0) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                max_blocks_per_seq, block_size, partition_tokens))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, k_scale=None,
              v_scale=None, partition_tokens: int = 0, variant: int = PA_VARIANT_AUTO,
              workspace=None, stream=None, flags: int = 0) -> None:
    """out/q [S][Hq][D]; caches as in pa_write_kv; block_tables int32 [S][MB]; lens int32 [S].
    ``workspace``: a uint8 GPU tensor of at least ``pa_decode_workspace_bytes`` bytes."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    S, Hq, Dq = q.shape
    MB = block_tables.shape[1]
    _need(Dq == D and tuple(out.shape) == (S, Hq, D), "q/out must be [S][Hq][D]")
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables / context_lens must be int32")
    _need(block_tables.shape[0] == S and context_lens.shape[0] == S, "one table row / length per sequence")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", load().pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        S, Hq, Hkv, D, B, MB, NB, float(scale), dtype_code(q), dtype_code(k_cache), dtype_code(out),
        _ptr(k_scale), _ptr(v_scale), int(partition_tokens), int(variant), int(flags),
        _ptr(workspace), ws_bytes, _stream(stream)))


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      k_scale=None, v_scale=None, partition_tokens: int = 0,
                      variant: int = PA_VARIANT_AUTO, stream=None, flags: int = 0) -> None:
    """pa_decode with the partial results in the library's own fixed device array (no workspace
    argument, nothing allocated); raises PagedAttnError(PA_ERR_WORKSPACE) when the plan needs more
    than PA_NOALLOC_SCRATCH_BYTES."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    S, Hq, Dq = q.shape
    MB = block_tables.shape[1]
    _need(Dq == D and tuple(out.shape) == (S, Hq, D), "q/out must be [S][Hq][D]")
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables / context_lens must be int32")
    _need(block_tables.shape[0] == S and context_lens.shape[0] == S, "one table row / length per sequence")
    _check("pa_decode_noalloc", load().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        S, Hq, Hkv, D, B, MB, NB, float(scale), dtype_code(q), dtype_code(k_cache), dtype_code(out),
        _ptr(k_scale), _ptr(v_scale), int(partition_tokens), int(variant), int(flags),
        _stream(stream)))


PA_NOALLOC_SCRATCH_BYTES = 32 << 20


def pa_decode_grouped_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int,
                                      max_blocks_per_seq: int, block_size: int,
                                      partition_tokens: int = 0) -> int:
    return int(load().pa_decode_grouped_workspace_bytes(num_seqs, num_heads, head_dim,
                                                        max_blocks_per_seq, block_size,
                                                        partition_tokens))


def pa_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                      prefix_blocks, max_group_size: int, scale: float, k_scale=None,
                      v_scale=None, partition_tokens: int = 0, workspace=None, stream=None,
                      flags: int = 0) -> None:
    """pa_decode with the prefix blocks a group of sequences shares read once for the group:
    ``group_start`` int32 [groups + 1] (consecutive sequences), ``prefix_blocks`` int32 [S]."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    S, Hq, Dq = q.shape
    MB = block_tables.shape[1]
    _need(Dq == D and tuple(out.shape) == (S, Hq, D), "q/out must be [S][Hq][D]")
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(all(t.dtype == torch.int32 for t in (block_tables, context_lens, group_start, prefix_blocks)),
          "block_tables / context_lens / group_start / prefix_blocks must be int32")
    _need(block_tables.shape[0] == S and context_lens.shape[0] == S and prefix_blocks.shape[0] == S,
          "one table row / length / prefix per sequence")
    _need(group_start.dim() == 1 and group_start.shape[0] >= 2, "group_start must be [groups + 1]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_grouped", load().pa_decode_grouped(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(group_start), _ptr(prefix_blocks), group_start.shape[0] - 1, int(max_group_size), S, Hq,
        Hkv, D, B, MB, NB, float(scale), dtype_code(q), dtype_code(k_cache), dtype_code(out),
        _ptr(k_scale), _ptr(v_scale), int(partition_tokens), int(flags), _ptr(workspace), ws_bytes,
        _stream(stream)))


def pa_decode_grouped_append(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                             slot_mapping, group_start, prefix_blocks, max_group_size: int,
                             scale: float, k_scale=None, v_scale=None, partition_tokens: int = 0,
                             workspace=None, stream=None, flags: int = 0) -> None:
    """pa_write_kv of one new token per sequence (as pa_decode_append) and pa_decode_grouped in
    one pass."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    S, Hq, Dq = q.shape
    MB = block_tables.shape[1]
    _need(Dq == D and tuple(out.shape) == (S, Hq, D), "q/out must be [S][Hq][D]")
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(tuple(k_new.shape) == (S, Hkv, D) and k_new.shape == v_new.shape,
          "k_new/v_new must be [S][Hkv][D]")
    _need(all(t.dtype == torch.int32 for t in (block_tables, context_lens, slot_mapping,
                                                 group_start, prefix_blocks)),
          "block_tables / context_lens / slot_mapping / group_start / prefix_blocks must be int32")
    _need(block_tables.shape[0] == S and context_lens.shape[0] == S and slot_mapping.shape[0] == S
          and prefix_blocks.shape[0] == S, "one table row / length / slot / prefix per sequence")
    _need(group_start.dim() == 1 and group_start.shape[0] >= 2, "group_start must be [groups + 1]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_grouped_append", load().pa_decode_grouped_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), dtype_code(k_new), _ptr(group_start),
        _ptr(prefix_blocks), group_start.shape[0] - 1, int(max_group_size), S, Hq, Hkv, D, B, MB, NB,
        float(scale), dtype_code(q), dtype_code(k_cache), dtype_code(out), _ptr(k_scale),
        _ptr(v_scale), int(partition_tokens), int(flags), _ptr(workspace), ws_bytes,
        _stream(stream)))


def pa_decode_append(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                     slot_mapping, scale: float, k_scale=None, v_scale=None,
                     partition_tokens: int = 0, variant: int = PA_VARIANT_AUTO, workspace=None,
                     stream=None, flags: int = 0) -> None:
    """pa_write_kv of one new token per sequence (``k_new``/``v_new`` [S][Hkv][D], ``slot_mapping``
    int32 [S], each the slot of position context_lens[s]-1) and pa_decode in one pass."""
    import torch
    NB, Hkv, B, D = k_cache.shape
    S, Hq, Dq = q.shape
    MB = block_tables.shape[1]
    _need(Dq == D and tuple(out.shape) == (S, Hq, D), "q/out must be [S][Hq][D]")
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache must be [NB][Hkv][D][B]")
    _need(tuple(k_new.shape) == (S, Hkv, D) and k_new.shape == v_new.shape,
          "k_new/v_new must be [S][Hkv][D]")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32 and
          slot_mapping.dtype == torch.int32, "block_tables / context_lens / slot_mapping must be int32")
    _need(block_tables.shape[0] == S and context_lens.shape[0] == S and slot_mapping.shape[0] == S,
          "one table row / length / slot per sequence")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_append", load().pa_decode_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), dtype_code(k_new), S, Hq, Hkv, D, B, MB, NB,
        float(scale), dtype_code(q), dtype_code(k_cache), dtype_code(out), _ptr(k_scale),
        _ptr(v_scale), int(partition_tokens), int(variant), int(flags), _ptr(workspace), ws_bytes,
        _stream(stream)))


def pa_diag_read_bandwidth(buf, tile_bytes: int, num_tiles: int, tile_order=None, sink=None,
                           stream=None) -> None:
    """Diagnostic read of ``num_tiles`` tiles of ``buf`` (a GPU tensor), in address order or in
    the order of the int32 tensor ``tile_order``."""
    import torch
    if sink is None:
        sink = torch.empty(64 * 1024, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check("pa_diag_read_bandwidth", load().pa_diag_read_bandwidth(
        _ptr(buf), nbytes // tile_bytes, _ptr(tile_order), int(num_tiles), int(tile_bytes),
        _ptr(sink), _stream(stream)))


def pa_profile_enable(on: bool = True) -> None:
    _check("pa_profile_enable", load().pa_profile_enable(1 if on else 0))


def pa_profile_read(kernel_kind: int):
    """(total device milliseconds, launches) of one kernel kind since the last enable."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_longlong(0)
    _check("pa_profile_read", load().pa_profile_read(kernel_kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
