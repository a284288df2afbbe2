"""Reference for the block-table builder -- TEST INFRASTRUCTURE ONLY.

The library's host-side builder deals each sequence its own pages from a
shared pool.  The pool is first shuffled; the result is integer work, so the
library must match this reference bit for bit.

Specification (the pages give the table's meaning -- "kern manifest v7"
schema, $defs.Domain: a paged KV block table indexes pages of `stride` token
slots; $defs.HostTensor: the page count is the host's choice -- but no
dealing rule, so this one is the plainest that gives non-overlapping random
pages):

1. perm = [0, 1, ..., pool_pages-1], shuffled by Durstenfeld's Fisher-Yates:
   for i = pool_pages-1 down to 1, j = next() mod (i+1), swap perm[i], perm[j];
   next() is Vigna's splitmix64 generator seeded with ``seed``.
2. Sequence s (in order) takes the next ceil(ctx_lens[s] / page_size) entries
   of perm.  Columns past that are -1.
3. Optional slot mapping: for every sequence in order and every position t
   of it, slot = table[s][t // page_size] * page_size + t % page_size.
"""
from __future__ import annotations

import numpy as np

_MASK = (1 << 64) - 1


class SplitMix64:
    """Vigna's splitmix64: a Weyl sequence with step 0x9E3779B97F4A7C15
    passed through two xor-shift-multiply rounds and a final xor-shift."""

    def __init__(self, seed: int):
        self.state = seed & _MASK

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _MASK
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        return z ^ (z >> 31)


def build_block_table(ctx_lens, page_size: int, pool_pages: int, seed: int,
                      max_pages_per_seq: int, want_slots: bool = False):
    ctx = [int(c) for c in ctx_lens]
    need = [(c + page_size - 1) // page_size for c in ctx]
    if any(c < 0 for c in ctx) or any(n > max_pages_per_seq for n in need):
        raise ValueError("context longer than the table row")
    if sum(need) > pool_pages:
        raise ValueError("pool too small")
    perm = list(range(pool_pages))
    rng = SplitMix64(seed)
    for i in range(pool_pages - 1, 0, -1):
        j = rng.next() % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    table = np.full((len(ctx), max_pages_per_seq), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    if not want_slots:
        return table
    slots = []
    for s, c in enumerate(ctx):
        t = np.arange(c, dtype=np.int64)
        slots.append(table[s, t // page_size].astype(np.int64) * page_size + t % page_size)
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return table, slots.astype(np.int32)
