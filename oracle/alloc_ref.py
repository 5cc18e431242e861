"""Reference block manager -- TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

A plain Python model of the ref-counted KV block pool, written from:

* deepinsea.top "PagedAttention 内存管理深度解析", section "分页机制设计": a free
  list taken from the end, the number of blocks of a request is
  ceil(tokens / block_size), and allocation checks the free count first and
  fails without taking anything;
* wq-win.github.io "079 | vLLM 与 PagedAttention", section 二 ("共享与写时复制",
  "一次分叉什么时候真的要复制缓存块") and section 三: a block carries a
  reference count, a fork shares every block, writing into a tail block that
  someone else still references first copies it and remaps only the writer,
  releasing drops references and a block returns to the pool only at zero,
  a new block is taken only when the next token crosses a block boundary.

Readings where the pages are silent: the pool is shuffled once from a seed and
then used LIFO; a failed request changes nothing (all-or-nothing).
"""
from __future__ import annotations

import random


class OutOfBlocks(Exception):
    pass


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, shuffle_seed: int | None = None):
        self.block_size = block_size
        self.free = list(range(num_blocks))
        if shuffle_seed is not None:
            random.Random(shuffle_seed).shuffle(self.free)
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # blocks a request of n tokens occupies: ceil(n / block_size)
    def blocks_for(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def _take(self) -> int:
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def add_seq(self, seq: int, n_tokens: int) -> None:
        need = self.blocks_for(n_tokens)
        if seq in self.tables:
            raise KeyError(seq)
        if need > len(self.free):
            raise OutOfBlocks(seq)
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = n_tokens

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append(self, seq: int, n_tokens: int):
        """Reserve slots for the next ``n_tokens`` tokens of ``seq``.

        Returns (slots, cow_pairs).  Before the first write into a tail block
        with ref > 1 the block is copied; the pair (old, new) is reported."""
        table, L, bs = self.tables[seq], self.lens[seq], self.block_size
        need_new = self.blocks_for(L + n_tokens) - len(table)
        cow = n_tokens > 0 and L % bs != 0 and self.ref[table[-1]] > 1
        if need_new + (1 if cow else 0) > len(self.free):
            raise OutOfBlocks(seq)
        pairs = []
        if cow:
            old = table[-1]
            new = self._take()
            self._drop(old)
            table[-1] = new
            pairs.append((old, new))
        slots = []
        for pos in range(L, L + n_tokens):
            if pos // bs == len(table):
                table.append(self._take())
            slots.append(table[pos // bs] * bs + pos % bs)
        self.lens[seq] = L + n_tokens
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]

    def num_free(self) -> int:
        return len(self.free)

    def slots_reserved(self, seq: int) -> int:
        return len(self.tables[seq]) * self.block_size

    def tail_waste(self, seq: int) -> int:
        return self.slots_reserved(seq) - self.lens[seq]
