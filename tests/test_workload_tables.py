"""The shared-prefix batch's tables, slots and copy-on-write pairs against closed forms (CPU only).

The generator takes its tables and copy pairs from the host block manager, and both the oracle and
the kernels consume them, so a wrong copy-on-write decision would pass every parity test. These
checks derive what the pages' rule implies without the block manager ("PagedAttention", Ultralytics
glossary, section "シーケンス間でのブロック共有": samples of a prompt share its blocks by reference
count, and a block still shared is copied before a write lands in it; the podcast transcript's
paragraph on shared prefixes: the count is checked, the writer gets the copy):

* at the first decode step every sample of a prompt writes position P. If P is a multiple of B,
  the last prompt block is full and each sample opens a block of its own, with no copy. Otherwise
  the partly filled last block is held by all n samples: the first n - 1 (in batch order) each
  copy it, and the last, then its only holder, writes in place. So there are exactly n - 1 pairs
  per such prompt, all with that block as source;
* after any number of private decode steps, only whole prompt blocks are shared (identical leading
  entries across a prompt's samples); every other block belongs to one sequence; each sequence
  attends P + d + 1 tokens, and its new token's slot is offset (L - 1) mod B of its own last block.
"""

import numpy as np
import pytest

from workloads import make_shared_prefix


def _used(w, s):
    return [int(b) for b in w.tables[s, : -(-int(w.lens[s]) // w.block_size)]]


@pytest.mark.parametrize("B,seed", [(4, 11), (16, 4), (8, 23), (16, 31)])
def test_first_step_copies_follow_the_refcount_rule(B, seed):
    n = 4
    w = make_shared_prefix(num_prompts=12, samples=n, prompt_range=(5, 90), decoded_range=(0, 0),
                           first_step=True, num_heads=2, head_dim=4, block_size=B, dtype="bf16",
                           seed=seed)
    P = w.meta["prompts"]
    pairs = [tuple(int(x) for x in p) for p in w.cow]
    partial = [p for p in range(len(P)) if P[p] % B != 0]
    assert len(pairs) == (n - 1) * len(partial)
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts)                       # every copy gets its own block
    k = 0
    for p in range(len(P)):
        sam = list(range(p * n, (p + 1) * n))
        j = P[p] // B                                         # logical block of position P
        full = [_used(w, s)[:j] for s in sam]
        assert all(t == full[0] for t in full)                # whole prompt blocks shared as they are
        last = [_used(w, s)[j] for s in sam]
        if P[p] % B == 0:                                     # each sample opens its own block
            assert len(set(last)) == n and not set(last) & set(full[0])
            continue
        src = last[-1]                                        # the last sample writes in place
        for s_i, s in enumerate(sam[:-1]):                    # the others, in order, copy it
            assert pairs[k] == (src, last[s_i])
            k += 1
        assert len(set(last)) == n
    assert k == len(pairs)
    for s in range(w.num_seqs):                               # slot = own last block, offset P mod B
        L = int(w.lens[s])
        assert L == P[s // n] + 1
        assert int(w.slots[s]) == _used(w, s)[(L - 1) // B] * B + (L - 1) % B


@pytest.mark.parametrize("B,seed", [(4, 5), (16, 4), (8, 9)])
def test_after_private_steps_only_whole_prompt_blocks_are_shared(B, seed):
    n = 4
    w = make_shared_prefix(num_prompts=10, samples=n, prompt_range=(3, 70), decoded_range=(0, 40),
                           num_heads=2, head_dim=4, block_size=B, dtype="bf16", seed=seed)
    P, d = w.meta["prompts"], np.asarray(w.meta["decoded"]).reshape(-1)
    owners = {}
    for s in range(w.num_seqs):
        L = int(w.lens[s])
        assert L == P[s // n] + int(d[s]) + 1
        t = _used(w, s)
        assert len(t) == -(-L // B) and len(set(t)) == len(t)
        for j, b in enumerate(t):
            owners.setdefault(b, set()).add((s // n, j))
        assert int(w.slots[s]) == t[(L - 1) // B] * B + (L - 1) % B
    for b, who in owners.items():
        refs = sum(b in _used(w, s) for s in range(w.num_seqs))
        if refs > 1:                                  # shared: one prompt, one position, whole block
            assert len(who) == 1
            (p, j), = who
            assert (j + 1) * B <= P[p]
            assert refs == sum(1 for s in range(p * n, (p + 1) * n) if _used(w, s)[j] == b)
    # the block holding each new token is held by that sequence alone
    for s in range(w.num_seqs):
        b = int(w.slots[s]) // B
        assert sum(b in _used(w, x) for x in range(w.num_seqs)) == 1
