"""Pins for automatic prefix caching (zhy-blog.vercel.app vLLM post, section
2.2 (5): cached blocks live in one table keyed by their tokens and every token
before them, and a new request reuses what it finds; wq-win.github.io "079 |
vLLM 与 PagedAttention", self-test question 2: only the same prefix under the
same conditions may reuse K/V).

The pins run on any pool behind the small adapter interface below, so they
check the reference pool (``oracle.alloc_ref.PrefixCachingPool``) and libpa's
allocator alike.  Each returns None when it holds, or a short message.

* ``pin_content`` drives random requests, appends, forks and releases and
  plays the caller: it writes, per slot, the (salt, prefix) that defines the
  K/V of that position (K/V at position p is a function of the salt and
  tokens 0 .. p), and copies a block's contents when the pool reports a
  copy-on-write pair.  After every step every live sequence must read, through
  its block table, exactly the K/V of its own tokens: a reused or evicted
  block holding anything else shows up at once.
* ``pin_maximal_reuse``: in a pool too large to evict, a request reuses
  exactly as many leading full blocks as the longest run of its full-block
  prefixes that some earlier request or append has completed (brute force
  over the history).
* the scenario pins follow the stated eviction rules on tiny pools, with the
  expected tables derived by hand in their docstrings.
"""
from __future__ import annotations

import numpy as np


# ------------------------------------------------------------------ adapters
class OracleAdapter:
    def __init__(self, pool):
        from oracle.alloc_ref import OutOfBlocks
        self.p, self._oom, self.bs = pool, OutOfBlocks, pool.block_size

    def add(self, seq, tokens, salt=0):
        try:
            return self.p.add_seq_tokens(seq, tokens, salt)
        except self._oom:
            return None

    def append(self, seq, tokens):
        try:
            return self.p.append_tokens(seq, tokens)
        except self._oom:
            return None

    def append_plain(self, seq, n):
        try:
            return self.p.append(seq, n)
        except self._oom:
            return None

    def fork(self, parent, child):
        self.p.fork(parent, child)

    def free(self, seq):
        self.p.free_seq(seq)

    def table(self, seq):
        return list(self.p.tables[seq])

    def num_free(self):
        return self.p.num_free()

    def refcount(self, b):
        return self.p.ref[b]

    def num_evictable(self):
        return len(self.p.evictable)

    def num_cached(self):
        return len(self.p.cached)

    def reset(self):
        self.p.reset_cache()


def oracle_factory(cls=None):
    from oracle.alloc_ref import PrefixCachingPool
    cls = cls or PrefixCachingPool
    return lambda nb, bs, seed=None: OracleAdapter(cls(nb, bs, shuffle_seed=seed))


# ----------------------------------------------------------- content check
class ContentSim:
    """Plays the caller: what K/V each slot holds, per the writes it made."""

    def __init__(self, pool):
        self.pool, self.bs = pool, pool.bs
        self.slot: dict[int, tuple] = {}
        self.seqs: dict[int, tuple[int, list]] = {}

    def _slot(self, table, p):
        return table[p // self.bs] * self.bs + p % self.bs

    def add(self, seq, tokens, salt):
        n_cached = self.pool.add(seq, tokens, salt)
        if n_cached is None:
            return None
        t = self.pool.table(seq)
        for p in range(n_cached, len(tokens)):
            self.slot[self._slot(t, p)] = (salt, tuple(tokens[:p + 1]))
        self.seqs[seq] = (salt, list(tokens))
        return n_cached

    def append(self, seq, tokens):
        r = self.pool.append(seq, tokens)
        if r is None:
            return None
        slots, pairs = r
        for src, dst in pairs:
            for o in range(self.bs):
                if src * self.bs + o in self.slot:
                    self.slot[dst * self.bs + o] = self.slot[src * self.bs + o]
        salt, toks = self.seqs[seq]
        for s, tok in zip(slots, tokens):
            toks.append(int(tok))
            self.slot[int(s)] = (salt, tuple(toks))
        return r

    def fork(self, parent, child):
        self.pool.fork(parent, child)
        salt, toks = self.seqs[parent]
        self.seqs[child] = (salt, list(toks))

    def free(self, seq):
        self.pool.free(seq)
        del self.seqs[seq]

    def check(self):
        for seq, (salt, toks) in self.seqs.items():
            t = self.pool.table(seq)
            if len(t) != -(-len(toks) // self.bs):
                return f"seq {seq}: {len(t)} blocks for {len(toks)} tokens"
            for p in range(len(toks)):
                if self.slot.get(self._slot(t, p)) != (salt, tuple(toks[:p + 1])):
                    return f"seq {seq} position {p} reads K/V of another prefix"
        return None


def _prompt(rng, prefixes, vocab):
    """A prompt: one of a few shared prefixes (cut at a random length) and a
    random tail, so that requests overlap at every depth."""
    base = prefixes[int(rng.integers(len(prefixes)))]
    cut = int(rng.integers(0, len(base) + 1))
    tail = rng.integers(0, vocab, size=int(rng.integers(0, 12))).tolist()
    return base[:cut] + tail


def random_ops(sim, rng, steps, salts=(0, 1), vocab=3, plain_append=False):
    """Random script of requests, appends, forks and releases on a ContentSim;
    returns the first failure message or None."""
    prefixes = [rng.integers(0, vocab, size=40).tolist() for _ in range(3)]
    live, nxt = [], 0
    for step in range(steps):
        op = int(rng.integers(0, 10))
        if op < 4 or not live:
            sim.add(nxt, _prompt(rng, prefixes, vocab), int(rng.choice(salts)))
            if nxt in sim.seqs:
                live.append(nxt)
            nxt += 1
        elif op < 7:
            s = live[int(rng.integers(len(live)))]
            toks = rng.integers(0, vocab, size=int(rng.integers(1, 6))).tolist()
            if plain_append and op == 6:
                if sim.pool.append_plain(s, len(toks)) is not None:
                    live.remove(s)
                    sim.free(s)  # its K/V is unknown from here on
                continue
            sim.append(s, toks)
        elif op < 8:
            sim.fork(live[int(rng.integers(len(live)))], nxt)
            live.append(nxt)
            nxt += 1
        else:
            sim.free(live.pop(int(rng.integers(len(live)))))
        msg = sim.check()
        if msg:
            return f"step {step}: {msg}"
    return None


def pin_content(make, seeds=(0, 1, 2), nb=48, bs=4, steps=400):
    """Small pools (constant eviction): every sequence reads its own K/V."""
    for seed in seeds:
        rng = np.random.default_rng(seed)
        msg = random_ops(ContentSim(make(nb, bs, None)), rng, steps)
        if msg:
            return f"seed {seed}: {msg}"
    return None


def pin_maximal_reuse(make, seed=3, bs=4, steps=300):
    """Nothing is ever evicted: the number of reused tokens is the longest run
    of the request's full-block prefixes already completed (brute force)."""
    rng = np.random.default_rng(seed)
    sim = ContentSim(make(100000, bs, None))
    prefixes = [rng.integers(0, 3, size=40).tolist() for _ in range(3)]
    done: set[tuple] = set()  # (salt, prefix) of every full block completed

    def complete(salt, toks):
        for i in range(len(toks) // bs):
            done.add((salt, tuple(toks[:(i + 1) * bs])))

    live, nxt = [], 0
    for step in range(steps):
        op = int(rng.integers(0, 4))
        if op < 2 or not live:
            toks, salt = _prompt(rng, prefixes, 3), int(rng.integers(0, 2))
            want = 0
            while want < len(toks) // bs and (salt, tuple(toks[:(want + 1) * bs])) in done:
                want += 1
            got = sim.add(nxt, toks, salt)
            if got != want * bs:
                return f"step {step}: reused {got} tokens, longest completed run is {want * bs}"
            complete(salt, toks)
            live.append(nxt)
            nxt += 1
        elif op == 2:
            s = live[int(rng.integers(len(live)))]
            sim.append(s, rng.integers(0, 3, size=int(rng.integers(1, 6))).tolist())
            complete(*sim.seqs[s])
        else:
            sim.free(live.pop(int(rng.integers(len(live)))))
    return None


# ------------------------------------------------------------ scenarios
def pin_lru_and_release_order(make):
    """Pool of 4 blocks of 2 tokens, ids in order (taken from the top: 3, 2, ..).

    A = [1,2,3,4] takes 3 (key ..2) and 2 (key ..4); releasing A drops 2 then 3,
    so the evictable list is [2, 3].  B = [5..9] needs 3 blocks: 1 and 0 from
    the free list, then evicts 2 (released longest ago), keeping key ..2 in 3.
    C = [1,2,3,4] would reuse 3 and need 1 more block, but the only free block
    is 3 itself: out of blocks, and 3 stays evictable at count 0.  Releasing B
    drops 2 (private: free), 0 and 1 (entries: evictable).  C then reuses 3
    and takes 2: table [3, 2], 2 tokens reused."""
    p = make(4, 2, None)
    if p.add(0, [1, 2, 3, 4]) != 0 or p.table(0) != [3, 2]:
        return f"A: table {p.table(0)}"
    p.free(0)
    if p.num_free() != 4 or p.num_evictable() != 2:
        return "A released: 4 free, 2 of them evictable expected"
    if p.add(1, [5, 6, 7, 8, 9]) != 0 or p.table(1) != [1, 0, 2]:
        return f"B: table {p.table(1)} (expected [1, 0, 2])"
    if p.add(2, [1, 2, 3, 4]) is not None:
        return "C should run out of blocks"
    if p.num_free() != 1 or p.refcount(3) != 0 or p.num_evictable() != 1:
        return "failed request changed the pool"
    p.free(1)
    got = p.add(2, [1, 2, 3, 4])
    if got != 2 or p.table(2) != [3, 2]:
        return f"C: reused {got}, table {p.table(2)} (expected 2, [3, 2])"
    return None


def pin_free_blocks_before_eviction(make):
    """A = [1,2] takes 3 and is released (3 evictable); B = [5,6] must take a
    free block (2), not evict 3; C = [1,2] then reuses 3."""
    p = make(4, 2, None)
    p.add(0, [1, 2])
    p.free(0)
    p.add(1, [5, 6])
    if p.table(1) != [2]:
        return f"B took {p.table(1)}, expected the free block 2"
    if p.add(2, [1, 2]) != 2 or p.table(2) != [3]:
        return "C did not reuse block 3"
    return None


def pin_reuse_revives(make):
    """A reused block at count 0 is no longer evictable: A = [1,2] released
    (3 evictable); B = [1,2,3] reuses 3 and takes 2; D needs 3 blocks but only
    1 and 0 are free: out of blocks (3 and 2 belong to B)."""
    p = make(4, 2, None)
    p.add(0, [1, 2])
    p.free(0)
    if p.add(1, [1, 2, 3]) != 2 or p.table(1) != [3, 2] or p.refcount(3) != 1:
        return f"B: table {p.table(1)}"
    if p.num_free() != 2 or p.num_evictable() != 0:
        return "reused block still counted as evictable"
    if p.add(2, [7, 8, 9, 10, 11, 12]) is not None:
        return "D should run out of blocks"
    return None


def pin_prefix_decides(make):
    """Self-test question 2: equal tokens in block 1 after different block 0s
    are different K/V.  A = [1,1,5,5], B = [2,2,5,5]; C = [2,2,5,5,7] reuses
    B's two blocks, never A's second."""
    p = make(16, 2, None)
    p.add(0, [1, 1, 5, 5])
    p.add(1, [2, 2, 5, 5])
    got = p.add(2, [2, 2, 5, 5, 7])
    if got != 4 or p.table(2)[:2] != p.table(1):
        return f"C reused {got} tokens, blocks {p.table(2)[:2]} (B holds {p.table(1)})"
    return None


def pin_salt_separates(make):
    p = make(16, 2, None)
    p.add(0, [1, 2, 3, 4], salt=7)
    if p.add(1, [1, 2, 3, 4], salt=8) != 0:
        return "a request with another salt reused blocks"
    if p.add(2, [1, 2, 3, 4], salt=7) != 4:
        return "a request with the same salt did not reuse"
    return None


def pin_full_blocks_only(make):
    """Only full blocks are reused: A = [1,2,3,4,5] (bs 4) and B = A reuse the
    first block only; B's tail is its own block."""
    p = make(16, 4, None)
    p.add(0, [1, 2, 3, 4, 5])
    if p.add(1, [1, 2, 3, 4, 5]) != 4:
        return "B should reuse exactly the full block"
    if p.table(1)[0] != p.table(0)[0] or p.table(1)[1] == p.table(0)[1]:
        return "B must share block 0 and own its tail"
    if p.refcount(p.table(0)[0]) != 2 or p.refcount(p.table(0)[1]) != 1:
        return "reference counts"
    return None


def pin_appended_block_enters_table(make):
    """A = [1,2,3] (bs 4) filled by appending 4 and 9: its first block enters
    the table when full; B = [1,2,3,4,6] reuses it.  A sequence that appended
    without tokens is not cached from there on."""
    p = make(16, 4, None)
    p.add(0, [1, 2, 3])
    p.append(0, [4, 9])
    if p.add(1, [1, 2, 3, 4, 6]) != 4 or p.table(1)[0] != p.table(0)[0]:
        return "block filled by an append was not reused"
    p.add(2, [8, 8, 8])
    p.append_plain(2, 1)
    if p.add(3, [8, 8, 8, 0]) != 0:
        return "a block filled without known tokens was reused"
    return None


def pin_all_released_keeps_cache(make):
    """Releasing everything frees every block for allocation while the
    entries stay reusable; a reset forgets them."""
    p = make(16, 2, None)
    p.add(0, [1, 2, 3, 4, 5])
    p.fork(0, 1)
    p.append(1, [6])
    p.free(0)
    p.free(1)
    if p.num_free() != 16 or p.num_cached() != 3:
        return f"{p.num_free()} free, {p.num_cached()} cached (16, 3 expected)"
    if any(p.refcount(b) != 0 for b in range(16)):
        return "nonzero count after releasing everything"
    p.reset()
    if p.num_free() != 16 or p.num_cached() != 0 or p.num_evictable() != 0:
        return "reset left entries"
    if p.add(2, [1, 2, 3, 4]) != 0:
        return "reused a block after reset"
    return None


SCENARIOS = [pin_lru_and_release_order, pin_free_blocks_before_eviction, pin_reuse_revives,
             pin_prefix_decides, pin_salt_separates, pin_full_blocks_only,
             pin_appended_block_enters_table, pin_all_released_keeps_cache]
ALL_PINS = SCENARIOS + [pin_content, pin_maximal_reuse]


def failures(make):
    out = []
    for pin in ALL_PINS:
        try:
            msg = pin(make)
        except Exception as e:  # a mutant may also crash a pin
            msg = f"raised {type(e).__name__}: {e}"
        if msg:
            out.append(f"{pin.__name__}: {msg}")
    return out
