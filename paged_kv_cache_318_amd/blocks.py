"""Host-side block manager: free pool, per-sequence block tables, refcounts and copy-on-write.

This is the bookkeeping that produces the device inputs of the paged path -- block tables,
context lengths, the slot of each new token and the (src, dst) pairs a copy-on-write needs. It
runs on the host and never touches device memory.

Rules, by page title and section:

* "PagedAttention", Ultralytics glossary, section "ページングの仕組み" (how paging works): a
  sequence takes a new block from the free pool only once its previous block is full; the table
  records the order of its blocks; only the tail of the last block is ever unused. The section's
  example takes free blocks from the front of the free list -- ``BlockPool`` does the same.
* Same page, section "シーケンス間でのブロック共有" (sharing blocks between sequences) and
  section "関連手法" (continuous batching): several tables may name one physical block, counted
  by a per-block reference count; a write into a block that another sequence also uses first
  copies the block (copy-on-write); a finished sequence's blocks go straight back to the pool.
* "vLLM и PagedAttention" (podcast transcript), paragraph on shared prefixes: the check is on the
  reference count at the moment a sequence wants to add a token to a shared, partly filled block;
  full shared blocks stay shared.
* "Paged Attention" study notes, section "块分配策略" (block allocation): allocation fails with
  an out-of-memory error when the free list is too short. Unlike those notes, ``free`` here
  honours reference counts, and allocation never needs contiguous blocks.
* "vLLM и PagedAttention" (podcast transcript), paragraph on preemption: when running sequences
  need blocks and none are free, a whole group is suspended -- the next attention step needs every
  block of a sequence, so eviction is all-or-nothing per group -- and its KV data either moves to
  CPU memory and comes back later, or is dropped and recomputed. ``swap_out`` / ``swap_in`` keep
  the host side of the first option: a second pool of host blocks with its own free list.

Readings where the pages are open: the sequence that triggers a copy gets the copy and the source
block's count drops by one; the last remaining holder (count 1) writes in place; within one decode
step sequences append in the order they are given. A swapped group must own its blocks outright
(no block shared with a sequence outside the group); blocks shared inside the group stay shared
on the host and after the swap back (one host block per distinct device block, and back).
"""

from __future__ import annotations

import hashlib
from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["OutOfBlocks", "BlockPool", "CachingBlockPool", "block_hash", "shared_prefix_groups"]


class OutOfBlocks(RuntimeError):
    """The free pool cannot satisfy an allocation; the pool state is left unchanged."""


class BlockPool:
    """Free list + reference counts + per-sequence tables for one pool of ``num_blocks`` blocks of
    ``block_size`` token slots.

    ``free_order`` gives the initial free list (front = next block handed out); by default it is
    ``0 .. num_blocks-1``.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None,
                 num_host_blocks: int = 0):
        if num_blocks <= 0 or block_size <= 0 or num_host_blocks < 0:
            raise ValueError("num_blocks and block_size must be positive, num_host_blocks >= 0")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != sorted(set(order)) or any(b < 0 or b >= num_blocks for b in order):
            raise ValueError("free_order must list distinct block ids in [0, num_blocks)")
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        # host pool for swapped-out groups: free list, refcounts, and the swapped sequences'
        # tables of host block ids
        self.num_host_blocks = int(num_host_blocks)
        self.host_free: deque = deque(range(self.num_host_blocks))
        self.host_ref: List[int] = [0] * self.num_host_blocks
        self.swapped: Dict[int, List[int]] = {}

    # -- allocation ---------------------------------------------------------------------------
    def _take(self, n: int) -> List[int]:
        if n > len(self.free):
            raise OutOfBlocks(f"need {n} free blocks, have {len(self.free)}")
        out = [self.free.popleft() for _ in range(n)]
        for b in out:
            self.ref[b] = 1
        return out

    def blocks_needed(self, num_tokens: int) -> int:
        return -(-int(num_tokens) // self.block_size)

    def add_sequence(self, seq_id: int, num_tokens: int) -> List[int]:
        """Give a new sequence enough blocks for ``num_tokens`` tokens (its prompt)."""
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} already exists")
        blocks = self._take(self.blocks_needed(num_tokens))
        self.tables[seq_id] = blocks
        self.lengths[seq_id] = int(num_tokens)
        return list(blocks)

    def fork(self, parent: int, child: int) -> None:
        """``child`` starts as a copy of ``parent``'s table; every block gains one reference."""
        if child in self.tables:
            raise ValueError(f"sequence {child} already exists")
        blocks = list(self.tables[parent])
        for b in blocks:
            self.ref[b] += 1
        self.tables[child] = blocks
        self.lengths[child] = self.lengths[parent]

    def append_slot(self, seq_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow)`` where ``slot = block * block_size + offset`` and ``cow`` is a
        ``(src, dst)`` pair when the token lands in a block shared with another sequence (that
        block must be copied to ``dst`` before the token is written), else ``None``. On
        ``OutOfBlocks`` the state is unchanged.
        """
        table = self.tables[seq_id]
        pos = self.lengths[seq_id]
        j, off = divmod(pos, self.block_size)
        cow = None
        if j == len(table):                       # previous block full (or none yet): new block
            table.append(self._take(1)[0])
        elif self.ref[table[j]] > 1:              # partly filled block shared with others: copy it
            src = table[j]
            dst = self._take(1)[0]
            self.ref[src] -= 1
            table[j] = dst
            cow = (src, dst)
        self.lengths[seq_id] = pos + 1
        return table[j] * self.block_size + off, cow

    def free_sequence(self, seq_id: int) -> None:
        """Drop a finished (or swapped-out) sequence; blocks whose count reaches zero return to
        their pool's free list."""
        if seq_id in self.swapped:
            for h in self.swapped.pop(seq_id):
                self.host_ref[h] -= 1
                if self.host_ref[h] == 0:
                    self.host_free.append(h)
        else:
            for b in self.tables.pop(seq_id):
                self.ref[b] -= 1
                if self.ref[b] == 0:
                    self.free.append(b)
        del self.lengths[seq_id]

    # -- preemption by swapping --------------------------------------------------------------------
    @staticmethod
    def _distinct(tables: Iterable[List[int]]) -> List[int]:
        seen: Dict[int, None] = {}
        for t in tables:
            for b in t:
                seen.setdefault(b, None)
        return list(seen)

    def swap_out(self, seq_ids: Sequence[int]) -> List[Tuple[int, int]]:
        """Move a group's blocks to the host pool. Returns the ``(device block, host block)`` pairs
        to copy (``pa_swap_blocks`` with PA_SWAP_OUT) before the freed device blocks are reused.
        Raises ``ValueError`` if a block is also used outside the group, ``OutOfBlocks`` if the
        host pool is short; the state is then unchanged."""
        group = list(dict.fromkeys(seq_ids))
        for s in group:
            if s not in self.tables:
                raise ValueError(f"sequence {s} is not resident")
        dev = self._distinct(self.tables[s] for s in group)
        inside: Dict[int, int] = {}
        for s in group:
            for b in self.tables[s]:
                inside[b] = inside.get(b, 0) + 1
        if any(self.ref[b] != inside[b] for b in dev):
            raise ValueError("a block of the group is shared with a sequence outside it")
        if len(dev) > len(self.host_free):
            raise OutOfBlocks(f"need {len(dev)} free host blocks, have {len(self.host_free)}")
        to_host = {b: self.host_free.popleft() for b in dev}
        for b in dev:
            self.host_ref[to_host[b]] = self.ref[b]
            self.ref[b] = 0
            self.free.append(b)
        for s in group:
            self.swapped[s] = [to_host[b] for b in self.tables.pop(s)]
        return [(b, to_host[b]) for b in dev]

    def swap_in(self, seq_ids: Sequence[int]) -> List[Tuple[int, int]]:
        """Bring a swapped-out group back into device blocks (taken from the front of the free
        list). Returns the ``(host block, device block)`` pairs to copy (PA_SWAP_IN) before the
        group runs again. The group must hold every reference to its host blocks; raises
        ``OutOfBlocks`` if the device pool is short, leaving the state unchanged."""
        group = list(dict.fromkeys(seq_ids))
        for s in group:
            if s not in self.swapped:
                raise ValueError(f"sequence {s} is not swapped out")
        host = self._distinct(self.swapped[s] for s in group)
        inside: Dict[int, int] = {}
        for s in group:
            for h in self.swapped[s]:
                inside[h] = inside.get(h, 0) + 1
        if any(self.host_ref[h] != inside[h] for h in host):
            raise ValueError("a host block of the group is shared with a sequence outside it")
        dev = self._take(len(host))
        to_dev = dict(zip(host, dev))
        for h in host:
            self.ref[to_dev[h]] = self.host_ref[h]
            self.host_ref[h] = 0
            self.host_free.append(h)
        for s in group:
            self.tables[s] = [to_dev[h] for h in self.swapped.pop(s)]
        return [(h, to_dev[h]) for h in host]

    # -- views ----------------------------------------------------------------------------------
    def block_table(self, seq_ids: Sequence[int], width: Optional[int] = None) -> np.ndarray:
        """``int32 [len(seq_ids)][width]`` tables, padded with -1."""
        w = max((len(self.tables[s]) for s in seq_ids), default=0) if width is None else int(width)
        out = np.full((len(seq_ids), max(w, 1)), -1, dtype=np.int32)
        for i, s in enumerate(seq_ids):
            t = self.tables[s]
            if len(t) > out.shape[1]:
                raise ValueError("width smaller than a table")
            out[i, :len(t)] = t
        return out

    def context_lens(self, seq_ids: Sequence[int]) -> np.ndarray:
        return np.array([self.lengths[s] for s in seq_ids], dtype=np.int32)

    def blocks_in_use(self) -> int:
        return self.num_blocks - len(self.free)

    # -- invariants -----------------------------------------------------------------------------
    def check(self) -> None:
        """Raise AssertionError if any bookkeeping invariant is broken."""
        refs = [0] * self.num_blocks
        for s, t in self.tables.items():
            assert len(t) == self.blocks_needed(self.lengths[s]), f"seq {s}: table/length mismatch"
            for b in t:
                refs[b] += 1
        assert refs == self.ref, "reference counts differ from the number of table entries"
        free = set(self.free)
        assert len(free) == len(self.free), "a block appears twice in the free list"
        used = {b for b in range(self.num_blocks) if self.ref[b] > 0}
        assert not (free & used), "a referenced block is on the free list"
        assert free | used == set(range(self.num_blocks)), "a block is neither free nor referenced"
        href = [0] * self.num_host_blocks
        for s, t in self.swapped.items():
            assert s not in self.tables, f"seq {s} is both resident and swapped out"
            assert len(t) == self.blocks_needed(self.lengths[s]), f"seq {s}: host table/length mismatch"
            for h in t:
                href[h] += 1
        assert href == self.host_ref, "host reference counts differ from the swapped tables"
        hfree = set(self.host_free)
        assert len(hfree) == len(self.host_free), "a host block appears twice in the free list"
        hused = {h for h in range(self.num_host_blocks) if self.host_ref[h] > 0}
        assert not (hfree & hused) and hfree | hused == set(range(self.num_host_blocks)), \
            "host pool: a block is both free and used, or neither"


# ------------------------------------------------------------------------------------------------
# Groups of sequences sharing prefix blocks (input of pa_decode_grouped)
# ------------------------------------------------------------------------------------------------

def shared_prefix_groups(tables, lens, block_size: int,
                         max_group_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Groups of consecutive sequences whose tables begin with the same physical blocks -- the
    parallel samples of one prompt, which share its blocks by reference count ("PagedAttention",
    Ultralytics glossary, section "シーケンス間でのブロック共有"). Greedy, in batch order: a
    sequence joins the open group while the group has fewer than ``max_group_size`` members and
    the sequence's table starts with at least one of the group's shared whole blocks.

    Returns ``group_start`` (int32 [groups + 1]) and ``prefix_blocks`` (int32 [S]): the leading
    table entries every member of the group shares, counting only blocks every member attends in
    full (``len // block_size``); 0 for a sequence alone in its group."""
    tables = np.asarray(tables)
    lens = np.asarray(lens, dtype=np.int64)
    S = int(lens.shape[0])
    if max_group_size < 1:
        raise ValueError("max_group_size must be at least 1")
    full = np.maximum(lens, 0) // block_size
    starts, prefix = [0], np.zeros(S, dtype=np.int32)
    s = 0
    while s < S:
        common, e = int(full[s]), s + 1
        while e < S and e - s < max_group_size:
            n = min(common, int(full[e]))
            same = np.flatnonzero(tables[e, :n] != tables[s, :n])
            k = int(same[0]) if same.size else n
            if k == 0:
                break
            common, e = k, e + 1
        if e - s > 1:
            prefix[s:e] = common
        starts.append(e)
        s = e
    return np.asarray(starts, dtype=np.int32), prefix


# ------------------------------------------------------------------------------------------------
# Prefix caching across requests
# ------------------------------------------------------------------------------------------------

def block_hash(parent: bytes, tokens: Sequence[int]) -> bytes:
    """Digest of one full block: SHA-256 over the parent block's digest and the block's token ids
    (int64 little-endian). Chained this way a block's digest stands for the whole prefix that ends
    with it, so equal digests mean equal prefixes, not just equal blocks."""
    h = hashlib.sha256()
    h.update(parent)
    h.update(np.asarray(tokens, dtype="<i8").tobytes())
    return h.digest()


class CachingBlockPool(BlockPool):
    """``BlockPool`` whose full blocks are also indexed by the hash of the prefix they end, so a
    new request whose prompt starts with an already cached prefix reuses those blocks (one more
    reference each) instead of recomputing and storing them.

    Rules, by page title and section:

    * "PagedAttention", Ultralytics glossary, section "シーケンス間でのブロック共有": hashing whole
      blocks extends block sharing from the sequences of one request to different requests.
    * "Paged Attention" study notes, section "Prefix Caching机制": a prefix is looked up by its
      hash, a hit is confirmed by checking that the cached tokens really match the prompt, and
      cached blocks carry reference counts.

    Readings where the pages are open: only full blocks are hashed (a partly filled block still
    changes); the hash chains the parent block's digest (a block stands for its whole prefix);
    a hit is confirmed token by token (a digest collision never hands out wrong data); a cached
    block whose last reference goes away stays cached and goes to the back of the free list, so
    the least recently released cached block is the first one a new allocation reclaims (and
    its hash entry is dropped then). Sharing a cached block never needs copy-on-write: only
    partly filled blocks are ever written.
    """

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Iterable[int]] = None,
                 num_host_blocks: int = 0):
        super().__init__(num_blocks, block_size, free_order, num_host_blocks)
        self.by_hash: Dict[bytes, int] = {}
        self.block_key: Dict[int, Tuple[bytes, Tuple[int, ...]]] = {}  # block -> (hash, tokens)
        self.hits = 0
        self.lookups = 0

    def _take(self, n: int) -> List[int]:
        out = super()._take(n)
        for b in out:                      # reclaiming a released cached block drops its entry
            key = self.block_key.pop(b, None)
            if key is not None:
                del self.by_hash[key[0]]
        return out

    def _hashes(self, tokens: Sequence[int]) -> List[Tuple[bytes, Tuple[int, ...]]]:
        B = self.block_size
        out, parent = [], b""
        for j in range(len(tokens) // B):
            blk = tuple(int(t) for t in tokens[j * B:(j + 1) * B])
            parent = block_hash(parent, blk)
            out.append((parent, blk))
        return out

    def cached_prefix(self, tokens: Sequence[int]) -> List[int]:
        """Physical blocks holding the longest cached prefix of ``tokens`` (full blocks only,
        confirmed token by token); nothing is reserved."""
        blocks = []
        for h, blk in self._hashes(tokens):
            b = self.by_hash.get(h)
            if b is None or self.block_key[b][1] != blk:
                break
            blocks.append(b)
        return blocks

    def add_sequence_cached(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Start a sequence for the prompt ``tokens``: reuse the blocks of its longest cached
        prefix, allocate the rest. Returns the number of prompt tokens already cached; the caller
        computes and writes only tokens from there on (a chunked prefill whose context is the
        cached prefix). On ``OutOfBlocks`` the state is unchanged. The caller must leave at least
        one token to compute, so a fully cached prompt reuses all but its last block."""
        if seq_id in self.tables or seq_id in self.swapped:
            raise ValueError(f"sequence {seq_id} already exists")
        n = len(tokens)
        hit = self.cached_prefix(tokens)
        if hit and len(hit) * self.block_size >= n:   # keep the last token to compute
            hit = hit[:-1]
        need = self.blocks_needed(n) - len(hit)
        revive = [b for b in hit if self.ref[b] == 0]
        if need > len(self.free) - len(revive):
            raise OutOfBlocks(f"need {need} free blocks, have {len(self.free) - len(revive)}")
        for b in revive:                   # released but still cached: back in use
            self.free.remove(b)
        for b in hit:
            self.ref[b] += 1
        self.tables[seq_id] = list(hit) + self._take(need)
        self.lengths[seq_id] = n
        self.lookups += 1
        self.hits += 1 if hit else 0
        return len(hit) * self.block_size

    def register(self, seq_id: int, tokens: Sequence[int]) -> int:
        """Index the sequence's full blocks (whose keys and values are written) under their
        prefix hashes, so later prompts can reuse them. ``tokens`` are the sequence's token ids
        so far. A prefix that is already cached under another block keeps that block. Returns
        the number of blocks newly indexed."""
        table = self.tables[seq_id]
        added = 0
        for j, (h, blk) in enumerate(self._hashes(tokens[: self.lengths[seq_id]])):
            b = table[j]
            if h in self.by_hash or b in self.block_key:
                continue
            self.by_hash[h] = b
            self.block_key[b] = (h, blk)
            added += 1
        return added

    def check(self) -> None:
        super().check()
        assert len(self.by_hash) == len(self.block_key), "hash index and block keys differ"
        for h, b in self.by_hash.items():
            assert self.block_key[b][0] == h, "hash index points at a block with another key"
