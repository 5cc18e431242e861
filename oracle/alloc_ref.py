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
then used LIFO; a failed request changes nothing (all-or-nothing); releasing a
sequence drops its blocks from the last to the first.

``PrefixCachingPool`` adds automatic prefix caching, written from the
zhy-blog.vercel.app vLLM post, section 2.2 (5) ("自动前缀缓存"): every cached
block sits in one table under a key made of its own tokens and all the tokens
before it, and a new request looks its blocks up there and reuses the ones it
finds; and from the wq-win page's self-test ("自测：从内存图推导服务行为"),
question 2: KV may be reused only for the same prefix under the same
conditions, equal tokens at one place are not enough.  Readings where the pages are silent (the plainest ones the rest
supports):

* only full blocks are cached (a partially filled block is still written, the
  wq-win page's section 二 shares only blocks that are full and no longer
  rewritten); a block enters the table when it becomes full;
* the key of block i is (salt, every token of positions 0 .. (i+1)*BS - 1);
  the salt stands for "the same conditions" (model, adapter, ...);
* a request reuses the longest run of its leading full blocks that are in the
  table, and stops at the first one that is not;
* a cached block whose count drops to 0 stays in the table, evictable; free
  blocks are taken first, and only when none is left is the evictable block
  released longest ago evicted (least recently used); a block that fills with
  a key already in the table stays private to its sequence.
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

    def num_free(self) -> int:
        return len(self.free)

    def add_seq(self, seq: int, n_tokens: int) -> None:
        need = self.blocks_for(n_tokens)
        if seq in self.tables:
            raise KeyError(seq)
        if need > self.num_free():
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
        if need_new + (1 if cow else 0) > self.num_free():
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
        for b in reversed(self.tables.pop(seq)):
            self._drop(b)
        del self.lens[seq]

    def slots_reserved(self, seq: int) -> int:
        return len(self.tables[seq]) * self.block_size

    def tail_waste(self, seq: int) -> int:
        return self.slots_reserved(seq) - self.lens[seq]


class PrefixCachingPool(BlockPool):
    """BlockPool with automatic prefix caching (see the module docstring)."""

    def __init__(self, num_blocks: int, block_size: int, shuffle_seed: int | None = None):
        super().__init__(num_blocks, block_size, shuffle_seed)
        self.cached: dict[tuple, int] = {}   # key -> block holding that prefix
        self.key_of: dict[int, tuple] = {}   # block -> its key, for table entries
        self.evictable: list[int] = []       # table entries at count 0, oldest first
        self.tokens: dict[int, list | None] = {}  # None: tokens unknown, not cached
        self.salt: dict[int, int] = {}
        self.entered: dict[int, list] = {}   # seq -> blocks it entered into the table

    def key(self, salt: int, tokens, i: int) -> tuple:
        """Key of block i: the salt and every token up to the end of block i."""
        return (salt, tuple(tokens[:(i + 1) * self.block_size]))

    def num_free(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        else:  # evict the entry released longest ago
            b = self.evictable.pop(0)
            del self.cached[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            (self.evictable if b in self.key_of else self.free).append(b)

    def _revive(self, b: int) -> None:
        """A request reuses table entry b: one more reference; an entry at
        count 0 leaves the evictable list."""
        if self.ref[b] == 0:
            self.evictable.remove(b)
        self.ref[b] += 1

    def _register(self, key: tuple, b: int, seq: int) -> None:
        if key not in self.cached:
            self.cached[key] = b
            self.key_of[b] = key
            self.entered.setdefault(seq, []).append(b)

    def add_seq(self, seq: int, n_tokens: int) -> None:
        super().add_seq(seq, n_tokens)
        self.tokens[seq] = None

    def add_seq_tokens(self, seq: int, tokens, salt: int = 0) -> int:
        """New sequence whose prompt is ``tokens``.  Returns how many leading
        tokens already have their K / V in reused blocks (a multiple of BS)."""
        if seq in self.tables:
            raise KeyError(seq)
        tokens = list(tokens)
        bs, n = self.block_size, len(tokens)
        hits = []
        for i in range(n // bs):
            b = self.cached.get(self.key(salt, tokens, i))
            if b is None:
                break
            hits.append(b)
        need = self.blocks_for(n) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need > self.num_free() - revived:
            raise OutOfBlocks(seq)
        for b in hits:
            self._revive(b)
        table = list(hits)
        for i in range(len(hits), self.blocks_for(n)):
            b = self._take()
            table.append(b)
            if (i + 1) * bs <= n:
                self._register(self.key(salt, tokens, i), b, seq)
        self.tables[seq] = table
        self.lens[seq] = n
        self.tokens[seq] = tokens
        self.salt[seq] = salt
        return len(hits) * bs

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        t = self.tokens[parent]
        self.tokens[child] = None if t is None else list(t)
        self.salt[child] = self.salt.get(parent, 0)

    def append(self, seq: int, n_tokens: int):
        """Append without tokens: the sequence's later blocks are not cached."""
        out = super().append(seq, n_tokens)
        self.tokens[seq] = None
        return out

    def append_tokens(self, seq: int, tokens):
        """Append known tokens; every block they fill enters the table."""
        tokens = list(tokens)
        L = self.lens[seq]
        slots, pairs = super().append(seq, len(tokens))
        if self.tokens[seq] is not None:
            self.tokens[seq].extend(tokens)
            bs = self.block_size
            for p in range(L, L + len(tokens)):
                if (p + 1) % bs == 0:
                    i = p // bs
                    self._register(self.key(self.salt[seq], self.tokens[seq], i),
                                   self.tables[seq][i], seq)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        super().free_seq(seq)
        del self.tokens[seq]
        self.salt.pop(seq, None)
        self.entered.pop(seq, None)

    def discard_seq(self, seq: int) -> None:
        """Release a sequence whose reserved slots never received their K / V:
        the table entries it created are forgotten first (their blocks then
        go to the free list), so no later request can reuse them."""
        for b in self.entered.get(seq, []):
            if b in self.key_of:
                del self.cached[self.key_of.pop(b)]
        self.free_seq(seq)

    def reset_cache(self) -> None:
        """Forget every table entry; evictable blocks become free (oldest
        release first onto the free list)."""
        self.free.extend(self.evictable)
        self.evictable = []
        self.cached.clear()
        self.key_of.clear()
