"""Host bookkeeping for one iteration that admits new prompts through the
allocator's automatic prefix caching (pa_alloc_add_seq_tokens): which rows the
iteration must compute, where their K / V go, and the block tables.

A prompt whose leading full blocks are found in the prefix table reuses them
(zhy-blog.vercel.app vLLM post, section 2.2 (5)); only the positions after
them are computed: their K / V are written (pa_reshape_and_cache) and their
queries attend over the whole context through the block table, the chunked
prefill of section 4.2 of the same post (pa_prefill).  A prompt found whole
still needs its last position's query (the next token's logits): that row is
computed, and its slot is -1 so that its K / V, already cached, is not
written again.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Admission:
    seq_ids: np.ndarray      # int64 [B]
    lens: np.ndarray         # int32 [B] prompt lengths
    cached: np.ndarray       # int32 [B] leading tokens whose K / V was reused
    query_start: np.ndarray  # int32 [B + 1] rows to compute, sequence by sequence
    row_seq: np.ndarray      # int64 [T] index (0 .. B-1) of each row's sequence
    row_pos: np.ndarray      # int64 [T] position of each row in its prompt
    slots: np.ndarray        # int64 [T] slot to write, -1 = already cached
    tables: np.ndarray       # int32 [B][max_blocks], -1 padded

    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start).max(initial=0))


def admit(alloc, seq_ids, prompts, salt: int = 0, max_blocks: int | None = None) -> Admission:
    """Add every prompt (int token arrays) as a new sequence of ``alloc`` (a
    BlockAllocator), reusing cached prefix blocks; all prompts are admitted
    in the given order, so a later prompt reuses blocks an earlier one of the
    same call filled (its K / V is written by this iteration's
    pa_reshape_and_cache, before the attention reads it).

    All or nothing: if a prompt cannot be admitted (e.g. OutOfBlocks), the
    prompts admitted before it in this call are discarded again, newest
    first, together with the prefix-table entries they created -- their K / V
    will never be written -- and the error is re-raised.  (Evictions made on
    their behalf are not undone.)"""
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    B = len(seq_ids)
    lens = np.array([len(p) for p in prompts], dtype=np.int32)
    cached = np.zeros(B, dtype=np.int32)
    done = 0
    try:
        for i, (s, p) in enumerate(zip(seq_ids, prompts)):
            cached[i] = alloc.add_seq_tokens(int(s), p, salt)
            done = i + 1
    except Exception:
        for s in reversed(seq_ids[:done]):
            alloc.discard_seq(int(s))
        raise
    bs = alloc.block_size
    if max_blocks is None:
        max_blocks = max(1, int(-(-lens.max(initial=0) // bs)))
    tables, _ = alloc.block_tables(seq_ids, max_blocks)
    first = np.where(lens > 0, np.minimum(cached, lens - 1), 0).astype(np.int64)
    nrows = lens.astype(np.int64) - first
    query_start = np.concatenate([[0], np.cumsum(nrows)]).astype(np.int32)
    row_seq = np.repeat(np.arange(B, dtype=np.int64), nrows)
    row_pos = np.arange(int(nrows.sum()), dtype=np.int64) - np.repeat(query_start[:-1], nrows) \
        + np.repeat(first, nrows)
    blk = tables[row_seq, row_pos // bs].astype(np.int64)
    slots = np.where(row_pos >= cached[row_seq], blk * bs + row_pos % bs, -1)
    return Admission(seq_ids, lens, cached, query_start, row_seq, row_pos, slots, tables)
