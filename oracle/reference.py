"""Reference (oracle) implementation of the paged decode path, in float64 on the CPU.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this module. It shares no code, headers, tables or helpers with the HIP library.

Sources, cited by page title and section:

* [Ultralytics] "PagedAttention", Ultralytics glossary (Japanese). Section "ページングの仕組み"
  (how paging works) holds a PyTorch key-pool example: a pool of 64 blocks of 16 slots of 64
  dims, free blocks 41, 7, 19, 2, 33 taken from the front; the key at position pos lands at slot
  pos mod B of the block the table lists at index pos div B, and the request is read back by
  indexing the pool with its table and keeping the first L rows. Section "シーケンス間でのブロック共有"
  (sharing blocks between sequences) gives refcounts and block-level copy-on-write. Section
  "関連手法" (related methods) names grouped-query attention and the 8-bit (FP8) KV cache.
* [Wikipedia] "PagedAttention", Wikipedia article (Russian mirror). Section "Математическая
  формулировка" (mathematical formulation): the causal attention equation for a query token i
  (weights a_ij over t = 1..i, output o_i = sum_j a_ij v_j, scaling by 1/sqrt(d)); the block
  definitions K_j, V_j of B consecutive keys/values; and the blockwise equation A_ij, o_i summed
  over the blocks j = 1..ceil(i/B), which the page states preserves causal attention.
* [Transcript] "vLLM и PagedAttention: виртуальная память для инференса LLM" (podcast
  transcript), the paragraph on OPT-13B memory (about 800 KB of KV per token, about 1.6 GB for
  2048 tokens).

Data layout (the interface both sides agree on; see ``include/pa.h``):

* ``k_pool[num_blocks][num_kv_heads][block_size][head_dim]`` -- the key of slot ``o`` of physical
  block ``b`` for kv head ``g`` is ``k_pool[b, g, o, :]`` (the glossary example's
  ``[block, slot, dim]`` pool with a head axis added).
* ``v_pool[num_blocks][num_kv_heads][head_dim][block_size]`` -- the value of that slot is
  ``v_pool[b, g, :, o]`` (values are stored dim-major inside a block).
* 16-bit storage: fp16 as ``numpy.float16``; bf16 as its raw ``uint16`` bit pattern. fp8 storage:
  OCP E4M3 codes as ``uint8`` with fp32 scales ``k_scale, v_scale [num_blocks][num_kv_heads]``;
  the real value of a code is ``e4m3(code) * scale``.

Readings of points the pages leave open (each also listed in the design notes):

* Only slots ``t < L`` of a sequence count; the tail of the last block is excluded, so the
  blockwise equation equals causal attention as the Wikipedia section asserts.
* The blockwise denominator (a sum of a vector of exponentials) is read as the sum of all entries.
* Query head ``h`` reads kv head ``h // (Hq / Hkv)`` (contiguous groups).
* ``L == 0`` gives a zero output.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "E4M3_VALUES", "e4m3_decode", "e4m3_encode", "fp8_quantize",
    "to_f64", "write_kv", "copy_blocks", "swap_blocks", "gather_sequence", "sequence_kv",
    "attention_contiguous", "attention_blockwise", "attention_split",
    "decode", "decode_blockwise", "decode_split", "prefill",
    "kv_bytes_per_token", "unused_slots",
]

# --------------------------------------------------------------------------------------------
# OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities;
# S.1111.111 is NaN; exponent field 0 encodes subnormals m/8 * 2^-6. The glossary's "関連手法"
# section names an 8-bit KV cache without fixing the format; this is the format's definition.
# --------------------------------------------------------------------------------------------


def _e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


#: float64 value of every one of the 256 codes (NaN for 0x7F and 0xFF).
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS_VALUES = E4M3_VALUES[:0x7F]          # codes 0x00..0x7E: 0, subnormals, normals up to 448
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Exact float64 value of each E4M3 code (table lookup)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(y) -> np.ndarray:
    """Round float32 values to E4M3 codes: nearest representable value, ties to the code whose
    mantissa LSB is 0, magnitudes at or above 448 saturate to 448, NaN stays NaN (0x7F with the
    input's sign bit). The sign bit of the code is the sign bit of the input (so -0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y).astype(np.uint8) << 7
    isnan = np.isnan(y)
    a = np.where(isnan, 0.0, np.abs(y).astype(np.float64))
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # _POS_VALUES[hi-1] < a <= _POS_VALUES[hi]
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code).astype(np.uint8)
    code = np.where(isnan, 0x7F, code).astype(np.uint8)
    return (code | sign).astype(np.uint8)


def fp8_quantize(x, scale) -> np.ndarray:
    """E4M3 code of ``x / scale`` for a positive scale: the division is one IEEE float32 divide
    (round to nearest even), the magnitude is rounded by ``e4m3_encode`` and the code's sign bit is
    the sign bit of ``x`` (so a NaN input keeps its sign whatever the divide does to it)."""
    x = np.asarray(x, dtype=np.float32)
    y = (x / np.asarray(scale, dtype=np.float32)).astype(np.float32)
    mag = e4m3_encode(np.abs(y)) & np.uint8(0x7F)
    return (mag | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


# --------------------------------------------------------------------------------------------
# storage -> float64
# --------------------------------------------------------------------------------------------


def to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements. ``dtype`` is one of 'f32', 'f16', 'bf16' (uint16
    bit patterns), 'fp8' (E4M3 codes, scale not applied)."""
    a = np.asarray(a)
    if dtype in ("f32", "f16"):
        return a.astype(np.float64)
    if dtype == "bf16":
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_decode(a)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------------------------
# Slot-mapped write and block copy (glossary, "ページングの仕組み" example and "シーケンス間での
# ブロック共有" copy-on-write). These work on host copies of the pools, in place.
# --------------------------------------------------------------------------------------------


def write_kv(k_pool, v_pool, k_new, v_new, slots, block_size, cache_dtype=None,
             k_scale=None, v_scale=None, in_dtype=None):
    """Token ``t`` with ``slots[t] >= 0`` goes to block ``slots[t] // B`` at offset
    ``slots[t] % B`` (the glossary example's slot arithmetic), for every kv head. With an fp8
    cache the stored code is ``fp8_quantize(x, scale[block, head])`` of the new token's real
    value ``x`` (its storage dtype ``in_dtype`` converted exactly to float32); otherwise the stored
    bits are the new token's bits."""
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        b, o = divmod(slot, block_size)
        if cache_dtype == "fp8":
            if in_dtype not in ("f32", "f16", "bf16"):
                raise ValueError("an fp8 write needs the new tokens' dtype (in_dtype)")
            kx = to_f64(k_new[t], in_dtype).astype(np.float32)
            vx = to_f64(v_new[t], in_dtype).astype(np.float32)
            k_pool[b, :, o, :] = fp8_quantize(kx, k_scale[b][:, None])
            v_pool[b, :, :, o] = fp8_quantize(vx, v_scale[b][:, None])
        else:
            k_pool[b, :, o, :] = k_new[t]
            v_pool[b, :, :, o] = v_new[t]


def copy_blocks(k_pool, v_pool, pairs, k_scale=None, v_scale=None):
    """For each (src, dst) pair, in order: the whole block -- every head's keys and values, and the
    fp8 scales when given -- becomes a copy of the source block."""
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        k_pool[dst] = k_pool[src].copy()
        v_pool[dst] = v_pool[src].copy()
        if k_scale is not None:
            k_scale[dst] = k_scale[src].copy()
            v_scale[dst] = v_scale[src].copy()


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, src_ks=None, src_vs=None, dst_ks=None,
                dst_vs=None):
    """Preemption by swapping ([Transcript], the paragraph on preemption: a group's KV data moves
    to CPU memory and later comes back): for each (src, dst) pair, block ``dst`` of the destination
    pool becomes a copy of block ``src`` of the source pool -- every head's keys and values, and
    the fp8 scales when given. A pair naming a block outside its pool is skipped (the library's
    contract for unvalidated device contents)."""
    for src, dst in np.asarray(pairs).reshape(-1, 2).tolist():
        if not (0 <= src < src_k.shape[0] and 0 <= dst < dst_k.shape[0]):
            continue
        dst_k[dst] = src_k[src]
        dst_v[dst] = src_v[src]
        if src_ks is not None:
            dst_ks[dst] = src_ks[src]
            dst_vs[dst] = src_vs[src]


# --------------------------------------------------------------------------------------------
# Block-table gather (glossary example: the kernel reads keys back through the table)
# --------------------------------------------------------------------------------------------


def gather_sequence(k_pool, v_pool, table_row, L, block_size):
    """Stored keys and values of one sequence in logical order, ``[L][Hkv][D]`` each, read token by
    token through its block table. No conversion: the stored bits come back as they are."""
    _, hkv, _, d = k_pool.shape
    K = np.empty((L, hkv, d), dtype=k_pool.dtype)
    V = np.empty((L, hkv, d), dtype=v_pool.dtype)
    for t in range(L):
        b = int(table_row[t // block_size])
        o = t % block_size
        K[t] = k_pool[b, :, o, :]
        V[t] = v_pool[b, :, :, o]
    return K, V


def sequence_kv(k_pool, v_pool, table_row, L, block_size, dtype, k_scale=None, v_scale=None):
    """Real (dequantised) keys and values of one sequence as float64 ``[L][Hkv][D]``."""
    K, V = gather_sequence(k_pool, v_pool, table_row, L, block_size)
    K = to_f64(K, dtype)
    V = to_f64(V, dtype)
    if dtype == "fp8":
        blocks = np.asarray([table_row[t // block_size] for t in range(L)], dtype=np.int64)
        K = K * np.asarray(k_scale, np.float64)[blocks][:, :, None]
        V = V * np.asarray(v_scale, np.float64)[blocks][:, :, None]
    return K, V


# --------------------------------------------------------------------------------------------
# Attention for the decode query (the newest token, position i = L) -- Wikipedia,
# "Математическая формулировка".
# --------------------------------------------------------------------------------------------


def attention_contiguous(q, K, V, scale):
    """Standard causal attention of one query over the gathered contiguous keys/values ``[L][D]``:
    weights exp(scale q.k_t) normalised over t = 1..L, output sum_t a_t v_t. The maximum score is
    subtracted before exponentiating (a shift that cancels exactly in the ratio)."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def attention_blockwise(q, key_blocks, value_blocks, L, block_size, scale):
    """The blockwise equation taken literally: for blocks j = 1..ceil(L/B) the score vector
    A_j = exp(scale q^T K_j) (slots at or beyond L excluded), the denominator is the sum of all
    blocks' scores, and o = sum_j V_j A_j^T / denominator. ``key_blocks[j]`` is ``[B][D]``;
    ``value_blocks[j]`` is ``[D][B]`` (columns are the block's values, as V_j is written). A common
    shift c (the largest valid score) is subtracted inside every exponential."""
    nb = len(key_blocks)
    if L == 0 or nb == 0:
        return np.zeros(value_blocks[0].shape[0] if nb else 0, dtype=np.float64)
    valid = [np.arange(j * block_size, (j + 1) * block_size) < L for j in range(nb)]
    scores = [scale * (key_blocks[j] @ q) for j in range(nb)]
    c = max(scores[j][valid[j]].max() for j in range(nb))
    A = [np.exp(scores[j][valid[j]] - c) for j in range(nb)]          # excluded slots dropped
    den = sum(a.sum() for a in A)
    num = sum(value_blocks[j][:, valid[j]] @ A[j] for j in range(nb))
    return num / den


def attention_split(q, K, V, scale, part_tokens):
    """Causal attention computed over consecutive partitions of ``part_tokens`` tokens and then
    combined: partition k yields its own max m_k, sum l_k = sum exp(z - m_k) and normalised output
    o_k; the result is sum_k w_k o_k / sum_k w_k with w_k = l_k exp(m_k - max_k m_k). This is the
    blockwise equation's single global denominator regrouped by partition."""
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    ms, ls, os_ = [], [], []
    for s in range(0, L, part_tokens):
        z = scale * (K[s:s + part_tokens] @ q)
        m = z.max()
        e = np.exp(z - m)
        ms.append(m)
        ls.append(e.sum())
        os_.append((e @ V[s:s + part_tokens]) / e.sum())
    M = max(ms)
    w = np.array([l * math.exp(m - M) for m, l in zip(ms, ls)])
    return (w[:, None] * np.array(os_)).sum(axis=0) / w.sum()


def _heads(q):
    return q.shape[0]


def decode(q, k_pool, v_pool, tables, lens, block_size, scale, dtype, q_dtype=None,
           k_scale=None, v_scale=None, seqs=None, heads=None):
    """Decode-step paged attention for every (sequence, query head): gather each sequence through
    its table, then ``attention_contiguous``. Returns float64 ``[S][Hq][D]`` (rows not in ``seqs``
    / ``heads`` are left zero when a subset is asked for)."""
    q64 = to_f64(q, q_dtype or dtype)
    S, Hq, D = q64.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(lens[s])
        K, V = sequence_kv(k_pool, v_pool, tables[s], L, block_size, dtype, k_scale, v_scale)
        for h in (range(Hq) if heads is None else heads):
            g = h // G
            out[s, h] = attention_contiguous(q64[s, h], K[:, g, :], V[:, g, :], scale)
    return out


def decode_blockwise(q, k_pool, v_pool, tables, lens, block_size, scale, dtype, q_dtype=None,
                     k_scale=None, v_scale=None):
    """Same result as ``decode`` by the second, independent route: blocks are read one at a time
    through the table (no gather) and combined with ``attention_blockwise``."""
    q64 = to_f64(q, q_dtype or dtype)
    S, Hq, D = q64.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        nb = -(-L // block_size)
        for h in range(Hq):
            g = h // G
            kb, vb = [], []
            for j in range(nb):
                b = int(tables[s][j])
                Kj = to_f64(k_pool[b, g], dtype)          # [B][D]
                Vj = to_f64(v_pool[b, g], dtype)          # [D][B]
                if dtype == "fp8":
                    Kj = Kj * float(k_scale[b, g])
                    Vj = Vj * float(v_scale[b, g])
                kb.append(Kj)
                vb.append(Vj)
            out[s, h] = attention_blockwise(q64[s, h], kb, vb, L, block_size, scale) if nb else 0.0
    return out


def decode_split(q, k_pool, v_pool, tables, lens, block_size, scale, dtype, part_tokens,
                 q_dtype=None, k_scale=None, v_scale=None):
    """``decode`` with every sequence split into partitions of ``part_tokens`` (``attention_split``)."""
    q64 = to_f64(q, q_dtype or dtype)
    S, Hq, D = q64.shape
    G = Hq // k_pool.shape[1]
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        K, V = sequence_kv(k_pool, v_pool, tables[s], L, block_size, dtype, k_scale, v_scale)
        for h in range(Hq):
            out[s, h] = attention_split(q64[s, h], K[:, h // G], V[:, h // G], scale, part_tokens)
    return out


# --------------------------------------------------------------------------------------------
# Memory arithmetic: transcript paragraph on OPT-13B (≈800 KB per token, ≈1.6 GB per 2048
# tokens); glossary "ページングの仕組み" (only the last block of a sequence is partly empty).
# --------------------------------------------------------------------------------------------


# --------------------------------------------------------------------------------------------
# Several new query tokens per sequence (prefill of a chunk over the cached context) --
# Wikipedia, "Математическая формулировка": the equations hold for any query position i, each
# query attending the keys up to and including its own position.
# --------------------------------------------------------------------------------------------


def prefill(q, k_pool, v_pool, tables, lens, query_start, block_size, scale, dtype, q_dtype=None,
            k_scale=None, v_scale=None, tokens=None):
    """Causal paged attention of a chunk of new tokens per sequence. Sequence s owns query rows
    ``query_start[s] .. query_start[s+1]-1`` (n_s of them) and attends ``lens[s]`` cached tokens,
    the last n_s of which are its new tokens; query k (0-based) sits at position
    ``p = lens[s] - n_s + k`` and attends positions 0..p through the table
    (``attention_contiguous`` over the first p+1 gathered tokens). Returns float64 ``[T][Hq][D]``;
    with ``tokens`` only those rows are computed (the rest stay zero)."""
    q64 = to_f64(q, q_dtype or dtype)
    T, Hq, D = q64.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    want = None if tokens is None else set(int(t) for t in tokens)
    for s in range(qs.shape[0] - 1):
        n = int(qs[s + 1] - qs[s])
        if n == 0 or (want is not None and not any(qs[s] <= t < qs[s + 1] for t in want)):
            continue
        L = int(lens[s])
        K, V = sequence_kv(k_pool, v_pool, tables[s], L, block_size, dtype, k_scale, v_scale)
        for k in range(n):
            t = int(qs[s]) + k
            if want is not None and t not in want:
                continue
            p = L - n + k
            for h in range(Hq):
                g = h // G
                out[t, h] = attention_contiguous(q64[t, h], K[:p + 1, g, :], V[:p + 1, g, :], scale)
    return out


def kv_bytes_per_token(layers, heads, head_dim, elem_bytes):
    """Bytes of K and V cached for one token across all layers."""
    return 2 * layers * heads * head_dim * elem_bytes


def unused_slots(num_tokens, block_size):
    """Empty slots of a paged sequence: the unused tail of its last block."""
    return -(-num_tokens // block_size) * block_size - num_tokens
