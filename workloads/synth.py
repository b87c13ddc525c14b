"""Seeded synthetic decode-step workloads shaped like the pages' examples.

Every workload is one decode step of one layer: each sequence already holds ``L - 1`` tokens in a
scattered block pool, gets one new token (its slot comes from the host block manager, possibly
with a copy-on-write pair), and attends ``L`` tokens. Shapes follow the pages: block size 16 (the
Ultralytics glossary, section on how paging works), OPT-13B / LLaMA-13B-like caches of 40 heads x
128 dims (the podcast transcript's OPT-13B paragraph puts about 800 KB of KV per token on that
model), grouped-query heads and an 8-bit cache (the glossary's section on related methods).

Recipe (fixed draw order from ``numpy.random.default_rng(seed)``, PCG64): context lengths ->
(shared prefix: prompt lengths, decoded counts) -> permutation of physical block ids (the free
list, consumed from the front) -> q -> K -> V -> the new token's K and V. Values are N(0, 1) drawn
in float32 and rounded to the storage dtype with round-to-nearest-even; fp8 tiles get one fp32
scale per (block, kv head) = amax of the tile's stored tokens / 448 (1.0 for an all-zero tile)
and codes from PyTorch's float32 -> float8_e4m3fn cast. Unused slots, free blocks and the
new token's slot hold poison; table padding is -1.

No attention, softmax, write or copy arithmetic lives here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from paged_kv_cache_318_amd.blocks import BlockPool

__all__ = ["Workload", "STORAGE", "ELEM_BYTES", "round_to", "make_workload", "make_shared_prefix",
           "config", "config_lens", "CONFIG_NAMES", "PrefillWorkload", "make_prefill"]

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}

CONFIG_NAMES = {
    1: "tiny fp32 MHA decode (4 seqs, L={1,17,40,100}, 2 heads, D=64, 64-block pool)",
    2: "OPT-13B-shaped MHA decode (64 seqs, 40 heads, D=128, fp16, L~U[128,2048])",
    3: "GQA long-context decode (128 seqs, 32/8 heads, D=128, bf16, L log-normal median 1024)",
    4: "shared-prefix sampling (16 prompts x 4 samples, 40 heads, D=128, bf16)",
    5: "fp8 KV decode (16 seqs, 32/8 heads, D=128, e4m3 K/V, bf16 q, L~U[16384,32768])",
}


def round_to(x, dtype: str) -> np.ndarray:
    """float32 -> storage dtype with round-to-nearest-even (bf16 as uint16 bit patterns)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        bits = x.view(np.uint32).astype(np.uint64)
        rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
        out = rounded.astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            out[nan] = 0x7FC0
        return out
    raise ValueError(f"round_to: unsupported dtype {dtype!r}")


def _fp8_codes(y) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _poison_fill(arr: np.ndarray, dtype: str, poison: str, rng: np.random.Generator) -> None:
    """Fill ``arr`` (a storage array) with the chosen poison."""
    if poison == "nan":
        val = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0),
               "fp8": np.uint8(0x7F)}[dtype]
        arr[...] = val
    elif poison == "big":
        val = {"f32": np.float32(3.0e38), "f16": np.float16(60000.0), "bf16": np.uint16(0x7F7F),
               "fp8": np.uint8(0x7E)}[dtype]
        arr[...] = val
    elif poison == "random":
        if dtype == "fp8":
            arr[...] = rng.integers(0, 256, size=arr.shape, dtype=np.uint8)
        else:
            arr[...] = round_to(rng.standard_normal(arr.shape, dtype=np.float32) * 50.0, dtype)
    elif poison == "zero":
        arr[...] = 0
    else:
        raise ValueError(f"unknown poison {poison!r}")


@dataclass
class Workload:
    """Host arrays of one decode step. Pools are the state *before* the step's copies and writes."""
    name: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str                       # cache storage dtype: f32 | f16 | bf16 | fp8
    q_dtype: str                     # query / new-token dtype (== dtype unless the cache is fp8)
    scale: float
    q: np.ndarray                    # [S][Hq][D]
    k_pool: np.ndarray               # [NB][Hkv][B][D]
    v_pool: np.ndarray               # [NB][Hkv][D][B]
    k_scale: Optional[np.ndarray]    # fp32 [NB][Hkv] (fp8 caches only)
    v_scale: Optional[np.ndarray]
    tables: np.ndarray               # int32 [S][W], padded with -1 (after the step's append)
    lens: np.ndarray                 # int32 [S], attended tokens including the new one
    k_new: np.ndarray                # [S][Hkv][D] in new_dtype
    v_new: np.ndarray
    slots: np.ndarray                # int32 [S]
    cow: np.ndarray                  # int32 [n][2] (src, dst)
    unique_tokens: int               # tokens stored once in the pool after the step
    meta: Dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.lens.shape[0])

    @property
    def new_dtype(self) -> str:
        return self.q_dtype if self.dtype == "fp8" else self.dtype

    @property
    def attended_tokens(self) -> int:
        return int(self.lens.astype(np.int64).sum())

    def kv_bytes(self, unique: bool = False) -> int:
        """Algorithmic K+V bytes one decode call must read (valid tokens only; fp8 adds the two
        fp32 scales per (block, kv head) a sequence touches)."""
        tok = self.unique_tokens if unique else self.attended_tokens
        b = tok * 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.dtype]
        if self.dtype == "fp8":
            blocks = int(sum(-(-int(L) // self.block_size) for L in self.lens))
            b += blocks * 2 * self.num_kv_heads * 4
        return b

    def decode_bytes(self, unique: bool = False) -> int:
        """All algorithmic bytes of one decode call: K/V (+scales), q, output, tables, lengths."""
        S = self.num_seqs
        qo = 2 * S * self.num_heads * self.head_dim * ELEM_BYTES[self.q_dtype]
        nb = int(sum(-(-int(L) // self.block_size) for L in self.lens))
        return self.kv_bytes(unique) + qo + 4 * nb + 4 * S

    def write_bytes(self) -> int:
        """Bytes the slot write moves: read the new K/V, write them into the cache."""
        n = int((self.slots >= 0).sum())
        per = self.num_kv_heads * self.head_dim
        return n * 2 * per * (ELEM_BYTES[self.new_dtype] + ELEM_BYTES[self.dtype]) + 4 * self.num_seqs

    def copy_bytes(self) -> int:
        blk = self.num_kv_heads * self.block_size * self.head_dim * ELEM_BYTES[self.dtype] * 2
        if self.dtype == "fp8":
            blk += 2 * self.num_kv_heads * 4
        return int(self.cow.shape[0]) * 2 * blk


@dataclass
class PrefillWorkload(Workload):
    """Host arrays of one chunked-prefill step: every sequence appends a chunk of new tokens to
    its cached context and attends causally. ``q``, ``k_new``, ``v_new`` and ``slots`` have one
    row per new token (T in all), sequence s owning rows ``query_start[s] .. query_start[s+1]-1``;
    ``lens`` counts the context plus the chunk."""
    query_start: Optional[np.ndarray] = None     # int32 [S+1]

    @property
    def new_tokens(self) -> int:
        return int(self.query_start[-1])

    def query_positions(self) -> np.ndarray:
        """Absolute position of every query row (its own cache position)."""
        pos = np.empty(self.new_tokens, dtype=np.int64)
        for s in range(self.num_seqs):
            a, b = int(self.query_start[s]), int(self.query_start[s + 1])
            pos[a:b] = int(self.lens[s]) - (b - a) + np.arange(b - a)
        return pos

    def attended_pairs(self) -> int:
        """(query, key) pairs the causal mask keeps: sum over query rows of position + 1."""
        return int((self.query_positions() + 1).sum())

    def prefill_flops(self) -> float:
        """Algorithmic flops: 2 D per pair for the scores and 2 D for the weighted values, per
        query head."""
        return 4.0 * self.head_dim * self.num_heads * self.attended_pairs()

    def prefill_bytes(self) -> int:
        """Algorithmic bytes: every cached K/V element read once, q in and out once each."""
        qo = 2 * self.new_tokens * self.num_heads * self.head_dim * ELEM_BYTES[self.q_dtype]
        nb = int(sum(-(-int(L) // self.block_size) for L in self.lens))
        return self.kv_bytes() + qo + 4 * nb + 8 * self.num_seqs


def make_prefill(context_lens, new_lens, *, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int = 16, dtype: str = "bf16", q_dtype: Optional[str] = None,
                 seed: int = 0, free_fraction: float = 0.2, poison: str = "nan",
                 name: str = "prefill") -> PrefillWorkload:
    """Sequences with ``context_lens[s]`` cached tokens each receive ``new_lens[s]`` new tokens
    (their slots reserved token by token through the block manager, blocks handed out in a seeded
    random order). fp8 caches: a block opened by the chunk gets its scales from the amax of the
    chunk's tokens that land in it; a block already holding context keeps its scales."""
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in context_lens]
    new = [int(x) for x in new_lens]
    if len(ctx) != len(new) or min(ctx + new, default=0) < 0:
        raise ValueError("context_lens and new_lens must be equally long and non-negative")
    S, B, Hq, Hkv, D = len(ctx), block_size, num_heads, num_kv_heads, head_dim
    q_dtype = q_dtype or (dtype if dtype != "fp8" else "bf16")
    new_dtype = q_dtype if dtype == "fp8" else dtype
    lens = np.array([c + n for c, n in zip(ctx, new)], dtype=np.int64)
    used = int(sum(-(-int(L) // B) for L in lens))
    NB = max(1, math.ceil((1.0 + free_fraction) * used))
    pool = BlockPool(NB, B, free_order=rng.permutation(NB).tolist())
    T = int(sum(new))
    slots = np.empty(T, dtype=np.int32)
    qs = np.zeros(S + 1, dtype=np.int32)
    t = 0
    for s in range(S):
        pool.add_sequence(s, ctx[s])
        for _ in range(new[s]):
            slots[t], cow = pool.append_slot(s)
            assert cow is None
            t += 1
        qs[s + 1] = t
    W = max(max((len(pool.tables[s]) for s in range(S)), default=1), 1)
    tables = pool.block_table(list(range(S)), width=W)

    q = round_to(rng.standard_normal((T, Hq, D), dtype=np.float32), q_dtype)
    C = int(sum(ctx))
    Kf = rng.standard_normal((C, Hkv, D), dtype=np.float32)
    Vf = rng.standard_normal((C, Hkv, D), dtype=np.float32)
    kn_f = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    vn_f = rng.standard_normal((T, Hkv, D), dtype=np.float32)

    st = STORAGE[dtype]
    k_pool = np.empty((NB, Hkv, B, D), dtype=st)
    v_pool = np.empty((NB, Hkv, D, B), dtype=st)
    _poison_fill(k_pool, dtype, poison, rng)
    _poison_fill(v_pool, dtype, poison, rng)
    k_scale = v_scale = None
    if dtype == "fp8":
        k_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
        v_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
    off = 0
    for s in range(S):
        n = ctx[s]
        Ks, Vs = Kf[off:off + n], Vf[off:off + n]
        off += n
        if n == 0:
            continue
        if dtype == "fp8":
            nb = -(-n // B)
            kc, ksc = _quantize_sequence(Ks, nb, B)
            vc, vsc = _quantize_sequence(Vs, nb, B)
            _place(k_pool, v_pool, pool.tables[s], kc, vc, B)
            for j in range(nb):
                k_scale[pool.tables[s][j]] = ksc[j]
                v_scale[pool.tables[s][j]] = vsc[j]
        else:
            _place(k_pool, v_pool, pool.tables[s], round_to(Ks, dtype), round_to(Vs, dtype), B)
    k_new = round_to(kn_f, new_dtype)
    v_new = round_to(vn_f, new_dtype)
    if dtype == "fp8":
        from_bits = lambda a: (a.astype(np.uint32) << 16).view(np.float32) if new_dtype == "bf16" \
            else a.astype(np.float32)
        kx, vx = from_bits(k_new), from_bits(v_new)
        opened = {}
        for t in range(T):
            b = int(slots[t]) // B
            if np.isnan(k_scale[b, 0]) or b in opened:
                opened.setdefault(b, []).append(t)
        for b, rows in opened.items():
            for arr, x in ((k_scale, kx), (v_scale, vx)):
                a = np.abs(x[rows]).max(axis=(0, 2)) / np.float32(448.0)
                a[a == 0] = 1.0
                arr[b] = a.astype(np.float32)
    return PrefillWorkload(name=name, num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                           num_blocks=NB, dtype=dtype, q_dtype=q_dtype,
                           scale=float(1.0 / math.sqrt(D)), q=q, k_pool=k_pool, v_pool=v_pool,
                           k_scale=k_scale, v_scale=v_scale, tables=tables,
                           lens=lens.astype(np.int32), k_new=k_new, v_new=v_new, slots=slots,
                           cow=np.zeros((0, 2), dtype=np.int32), unique_tokens=int(lens.sum()),
                           meta={"seed": seed, "poison": poison}, query_start=qs)


def _quantize_sequence(Kf: np.ndarray, nb: int, B: int):
    """fp8 codes and per-(logical block, head) scales of one sequence's float32 tokens [n][H][D]."""
    n, H, D = Kf.shape
    pad = np.zeros((nb * B, H, D), dtype=np.float32)
    pad[:n] = Kf
    amax = np.abs(pad.reshape(nb, B, H, D)).max(axis=(1, 3))            # [nb][H]
    sc = (amax / np.float32(448.0)).astype(np.float32)
    sc[sc == 0] = np.float32(1.0)
    per_tok = np.repeat(sc, B, axis=0)[:n]                               # [n][H]
    codes = _fp8_codes(Kf / per_tok[:, :, None])
    return codes, sc


def _place(pool_k, pool_v, table: Sequence[int], Kseq: np.ndarray, Vseq: np.ndarray, B: int) -> None:
    """Put tokens 0..n-1 of one sequence into its blocks (keys slot-major, values dim-major)."""
    n = Kseq.shape[0]
    for j in range(-(-n // B)):
        lo, hi = j * B, min(n, (j + 1) * B)
        b = int(table[j])
        pool_k[b, :, : hi - lo, :] = Kseq[lo:hi].transpose(1, 0, 2)
        pool_v[b, :, :, : hi - lo] = Vseq[lo:hi].transpose(1, 2, 0)


def _new_block_scales(k_scale, v_scale, slots, B, k_new_f, v_new_f):
    """A new token that opens a fresh block sets that block's scales from its own amax."""
    for t, slot in enumerate(slots):
        if slot >= 0 and slot % B == 0:
            b = slot // B
            for arr, x in ((k_scale, k_new_f[t]), (v_scale, v_new_f[t])):
                a = np.abs(x).max(axis=1) / np.float32(448.0)
                a[a == 0] = 1.0
                arr[b] = a.astype(np.float32)


def make_workload(lens, *, num_heads: int, num_kv_heads: int, head_dim: int, block_size: int = 16,
                  dtype: str = "f16", q_dtype: Optional[str] = None, seed: int = 0,
                  num_blocks: Optional[int] = None, free_fraction: float = 0.2,
                  poison: str = "nan", table_width: Optional[int] = None,
                  scale: Optional[float] = None, name: str = "custom",
                  lens_rng: Optional[np.random.Generator] = None,
                  placement_seed: Optional[int] = None, placement: str = "scattered") -> Workload:
    """Independent sequences with the given attended lengths (each >= 0; a length-0 sequence gets
    no new token). The pool holds ``num_blocks`` blocks (default: blocks in use + ``free_fraction``)
    handed out in a seeded random order. ``placement_seed`` draws that order from its own generator,
    so two workloads differing only in it hold the same logical data at different physical blocks.
    ``placement="contiguous"`` hands the blocks out in address order instead (every sequence's
    blocks consecutive, sequences one after another: the layout of a contiguous cache, still read
    through the tables); the random order is drawn all the same, so the data is the same."""
    if placement not in ("scattered", "contiguous"):
        raise ValueError(f"placement must be 'scattered' or 'contiguous', not {placement!r}")
    rng = lens_rng if lens_rng is not None else np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    S = lens.shape[0]
    B = block_size
    Hkv, Hq, D = num_kv_heads, num_heads, head_dim
    q_dtype = q_dtype or (dtype if dtype != "fp8" else "bf16")
    new_dtype = q_dtype if dtype == "fp8" else dtype
    used = int(sum(-(-int(L) // B) for L in lens))
    NB = num_blocks if num_blocks is not None else max(1, math.ceil((1.0 + free_fraction) * used))
    if NB < used:
        raise ValueError(f"pool of {NB} blocks cannot hold {used} blocks")
    perm = (rng if placement_seed is None else np.random.default_rng(placement_seed)).permutation(NB)
    if placement == "contiguous":
        perm = np.arange(NB)
    pool = BlockPool(NB, B, free_order=perm.tolist())
    slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        L = int(lens[s])
        pool.add_sequence(s, max(L - 1, 0))
        if L > 0:
            slots[s], cow = pool.append_slot(s)
            assert cow is None
    W = max(table_width or 0, max((len(pool.tables[s]) for s in range(S)), default=1), 1)
    tables = pool.block_table(list(range(S)), width=W)

    q = round_to(rng.standard_normal((S, Hq, D), dtype=np.float32), q_dtype)
    prev = [max(int(L) - 1, 0) for L in lens]
    T = int(sum(prev))
    Kf = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    Vf = rng.standard_normal((T, Hkv, D), dtype=np.float32)
    kn_f = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    vn_f = rng.standard_normal((S, Hkv, D), dtype=np.float32)

    st = STORAGE[dtype]
    k_pool = np.empty((NB, Hkv, B, D), dtype=st)
    v_pool = np.empty((NB, Hkv, D, B), dtype=st)
    _poison_fill(k_pool, dtype, poison, rng)
    _poison_fill(v_pool, dtype, poison, rng)
    k_scale = v_scale = None
    if dtype == "fp8":
        k_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
        v_scale = np.full((NB, Hkv), np.nan, dtype=np.float32)
    off = 0
    for s in range(S):
        n = prev[s]
        Ks, Vs = Kf[off:off + n], Vf[off:off + n]
        off += n
        if n == 0:
            continue
        if dtype == "fp8":
            nb = -(-n // B)
            kc, ksc = _quantize_sequence(Ks, nb, B)
            vc, vsc = _quantize_sequence(Vs, nb, B)
            _place(k_pool, v_pool, pool.tables[s], kc, vc, B)
            for j in range(nb):
                k_scale[pool.tables[s][j]] = ksc[j]
                v_scale[pool.tables[s][j]] = vsc[j]
        else:
            _place(k_pool, v_pool, pool.tables[s], round_to(Ks, dtype), round_to(Vs, dtype), B)
    k_new = round_to(kn_f, new_dtype)
    v_new = round_to(vn_f, new_dtype)
    if dtype == "fp8":
        from_bits = lambda a: (a.astype(np.uint32) << 16).view(np.float32) if new_dtype == "bf16" \
            else a.astype(np.float32)
        _new_block_scales(k_scale, v_scale, slots.tolist(), B, from_bits(k_new), from_bits(v_new))
    return Workload(name=name, num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                    num_blocks=NB, dtype=dtype, q_dtype=q_dtype,
                    scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
                    q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
                    tables=tables, lens=lens.astype(np.int32), k_new=k_new, v_new=v_new,
                    slots=slots, cow=np.zeros((0, 2), dtype=np.int32),
                    unique_tokens=int(lens.sum()), meta={"seed": seed, "poison": poison})


def make_shared_prefix(*, seed: int = 4, num_prompts: int = 16, samples: int = 4,
                       prompt_range=(256, 1024), decoded_range=(0, 200), first_step: bool = False,
                       num_heads: int = 40, head_dim: int = 128, block_size: int = 16,
                       dtype: str = "bf16", free_fraction: float = 0.2, poison: str = "nan",
                       name: str = "shared-prefix") -> Workload:
    """Parallel sampling: each prompt's ``samples`` sequences share its blocks by reference count
    (forks of the prompt), then each decodes its own ``d`` tokens step by step through the block
    manager (copy-on-write of a shared, partly filled last block happens there), then the measured
    step appends one token to every sample. With ``first_step`` every ``d`` is 0, so the measured
    step itself performs the copies: for a partly filled prompt block held by n samples, n-1 copy
    and the last writes in place."""
    rng = np.random.default_rng(seed)
    B = block_size
    P = rng.integers(prompt_range[0], prompt_range[1], endpoint=True, size=num_prompts)
    if first_step:
        d = np.zeros((num_prompts, samples), dtype=np.int64)
    else:
        d = rng.integers(decoded_range[0], decoded_range[1], endpoint=True, size=(num_prompts, samples))
    S = num_prompts * samples
    dflat = d.reshape(-1)

    def simulate(bp: BlockPool):
        for p in range(num_prompts):
            bp.add_sequence(p * samples, int(P[p]))
            for i in range(1, samples):
                bp.fork(p * samples, p * samples + i)
        for k in range(int(dflat.max(initial=0))):
            for s in range(S):
                if dflat[s] > k:
                    bp.append_slot(s)
        pre = {s: list(bp.tables[s]) for s in range(S)}
        slots, cows = [], []
        for s in range(S):
            slot, cow = bp.append_slot(s)
            slots.append(slot)
            if cow is not None:
                cows.append(cow)
        return pre, slots, cows

    big = int(sum(-(-int(p) // B) for p in P) + S * (-(-int(dflat.max(initial=0) + 1) // B) + 2))
    probe = BlockPool(big, B)
    simulate(probe)
    used = probe.blocks_in_use()
    NB = max(1, math.ceil((1.0 + free_fraction) * used))
    perm = rng.permutation(NB)
    bp = BlockPool(NB, B, free_order=perm.tolist())
    pre, slots, cows = simulate(bp)
    bp.check()
    lens = bp.context_lens(list(range(S)))
    tables = bp.block_table(list(range(S)))

    Hq = Hkv = num_heads
    D = head_dim
    q = round_to(rng.standard_normal((S, Hq, D), dtype=np.float32), dtype)
    Tp, Td = int(P.sum()), int(dflat.sum())
    Kp = rng.standard_normal((Tp + Td, Hkv, D), dtype=np.float32)
    Vp = rng.standard_normal((Tp + Td, Hkv, D), dtype=np.float32)
    kn = round_to(rng.standard_normal((S, Hkv, D), dtype=np.float32), dtype)
    vn = round_to(rng.standard_normal((S, Hkv, D), dtype=np.float32), dtype)
    Kp, Vp = round_to(Kp, dtype), round_to(Vp, dtype)
    p_off = np.concatenate([[0], np.cumsum(P)])
    d_off = Tp + np.concatenate([[0], np.cumsum(dflat)])

    st = STORAGE[dtype]
    k_pool = np.empty((NB, Hkv, B, D), dtype=st)
    v_pool = np.empty((NB, Hkv, D, B), dtype=st)
    _poison_fill(k_pool, dtype, poison, rng)
    _poison_fill(v_pool, dtype, poison, rng)
    for s in range(S):
        p = s // samples
        idx = np.concatenate([np.arange(p_off[p], p_off[p + 1]), np.arange(d_off[s], d_off[s + 1])])
        _place(k_pool, v_pool, pre[s], Kp[idx], Vp[idx], B)
    unique = int(P.sum() + dflat.sum() + S)
    return Workload(name=name, num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=B,
                    num_blocks=NB, dtype=dtype, q_dtype=dtype, scale=1.0 / math.sqrt(D),
                    q=q, k_pool=k_pool, v_pool=v_pool, k_scale=None, v_scale=None,
                    tables=tables, lens=lens, k_new=kn, v_new=vn,
                    slots=np.asarray(slots, dtype=np.int32),
                    cow=np.asarray(cows, dtype=np.int32).reshape(-1, 2), unique_tokens=unique,
                    meta={"seed": seed, "poison": poison, "prompts": P.tolist(),
                          "decoded": d.tolist(), "samples": samples})


def _draw_lens(n: int, rng: np.random.Generator, over: dict) -> np.ndarray:
    """Context lengths of configurations 2, 3 and 5 (the first draws of their generators)."""
    if n == 2:
        S = over.pop("num_seqs", 64)
        return rng.integers(over.pop("min_len", 128), over.pop("max_len", 2048), endpoint=True, size=S)
    if n == 3:
        S = over.pop("num_seqs", 128)
        lo, hi = over.pop("clip", (64, 8192))
        return np.clip(np.round(np.exp(rng.normal(math.log(1024.0), 1.0, size=S))), lo, hi).astype(np.int64)
    if n == 5:
        S = over.pop("num_seqs", 16)
        return rng.integers(over.pop("min_len", 16384), over.pop("max_len", 32768), endpoint=True, size=S)
    raise ValueError(f"config {n} has no drawn lengths")


def config_lens(n: int) -> dict:
    """Shape of configuration 2, 3 or 5 without its data: the same lengths ``config(n)`` draws,
    head counts, head size, cache dtype and name (for timing inputs generated elsewhere)."""
    lens = _draw_lens(n, np.random.default_rng(n), {})
    shape = {2: (40, 40, "f16", "cfg2-opt13b-mha-f16"), 3: (32, 8, "bf16", "cfg3-gqa-long-bf16"),
             5: (32, 8, "fp8", "cfg5-fp8-kv")}[n]
    return {"lens": [int(x) for x in lens], "num_heads": shape[0], "num_kv_heads": shape[1],
            "head_dim": 128, "dtype": shape[2], "name": shape[3]}


def config(n: int, **over) -> Workload:
    """The five decode-step configurations (full size by default; keyword overrides shrink them
    for quick tests, e.g. ``num_seqs=8``)."""
    poison = over.pop("poison", "nan")
    if n == 1:
        return make_workload(over.pop("lens", [1, 17, 40, 100]), num_heads=2, num_kv_heads=2,
                             head_dim=64, block_size=16, dtype=over.pop("dtype", "f32"),
                             seed=over.pop("seed", 1), num_blocks=64, poison=poison,
                             name="cfg1-tiny-fp32", **over)
    if n == 2:
        seed = over.pop("seed", 2)
        rng = np.random.default_rng(seed)
        lens = _draw_lens(2, rng, over)
        dt = over.pop("dtype", "f16")
        return make_workload(lens, num_heads=40, num_kv_heads=40, head_dim=128,
                             block_size=over.pop("block_size", 16), dtype=dt, seed=seed,
                             poison=poison, lens_rng=rng, name=f"cfg2-opt13b-mha-{dt}", **over)
    if n == 3:
        seed = over.pop("seed", 3)
        rng = np.random.default_rng(seed)
        lens = _draw_lens(3, rng, over)
        return make_workload(lens, num_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=over.pop("block_size", 16), dtype=over.pop("dtype", "bf16"),
                             seed=seed, poison=poison, lens_rng=rng, name="cfg3-gqa-long-bf16", **over)
    if n == 4:
        return make_shared_prefix(seed=over.pop("seed", 4), poison=poison,
                                  name="cfg4-shared-prefix-bf16" + ("-first-step" if over.get("first_step") else ""),
                                  **over)
    if n == 5:
        seed = over.pop("seed", 5)
        rng = np.random.default_rng(seed)
        lens = _draw_lens(5, rng, over)
        return make_workload(lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                             dtype="fp8", q_dtype=over.pop("q_dtype", "bf16"), seed=seed,
                             poison=poison, lens_rng=rng, name="cfg5-fp8-kv", **over)
    raise ValueError(f"no config {n}")
