"""The reference prefix-caching pool against its pins (tests/prefix_cache_pins),
and builds of it with one planted mistake each: every mutant must break at
least one pin."""
import pytest

from oracle.alloc_ref import PrefixCachingPool
from tests import prefix_cache_pins as P


def test_reference_meets_every_pin():
    assert P.failures(P.oracle_factory()) == []


def test_content_pin_with_plain_appends():
    import numpy as np
    for seed in (5, 6):
        sim = P.ContentSim(P.oracle_factory()(40, 4, None))
        assert P.random_ops(sim, np.random.default_rng(seed), 400, plain_append=True) is None


class BlockTokensOnly(PrefixCachingPool):
    """Key from the block's own tokens, without the prefix before it."""

    def key(self, salt, tokens, i):
        bs = self.block_size
        return (salt, tuple(tokens[i * bs:(i + 1) * bs]))


class SaltIgnored(PrefixCachingPool):
    def key(self, salt, tokens, i):
        return super().key(0, tokens, i)


class EvictNewest(PrefixCachingPool):
    def _take(self):
        if not self.free and self.evictable:
            b = self.evictable.pop()
            del self.cached[self.key_of.pop(b)]
            self.ref[b] = 1
            return b
        return super()._take()


class EvictBeforeFree(PrefixCachingPool):
    def _take(self):
        if self.evictable:
            b = self.evictable.pop(0)
            del self.cached[self.key_of.pop(b)]
            self.ref[b] = 1
            return b
        return super()._take()


class ReleaseForward(PrefixCachingPool):
    def free_seq(self, seq):
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]
        del self.tokens[seq]


class NoRevive(PrefixCachingPool):
    """Reuse forgets to take the entry off the evictable list."""

    def _revive(self, b):
        self.ref[b] += 1

    def _take(self):
        if not self.free:
            b = self.evictable.pop(0)
            self.cached.pop(self.key_of.pop(b), None)
            self.ref[b] = 1
            return b
        return super()._take()


class NoRetention(PrefixCachingPool):
    """A cached block at count 0 goes straight back to the free list while
    its entry stays in the table."""

    def _drop(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)


class CachePartialTail(PrefixCachingPool):
    """The partially filled last block of a prompt is cached and reused too
    (keyed by the tokens it holds so far)."""

    def add_seq_tokens(self, seq, tokens, salt=0):
        tokens = list(tokens)
        bs, n = self.block_size, len(tokens)
        full = super().add_seq_tokens(seq, tokens, salt)
        if n % bs == 0:
            return full
        key = (salt, tuple(tokens), "partial")
        table = self.tables[seq]
        if full == (n // bs) * bs and key in self.cached:
            mine = table[-1]
            table[-1] = self.cached[key]
            self._revive(table[-1])
            self._drop(mine)
            return n
        self._register(key, table[-1])
        return full


class NeverReuse(PrefixCachingPool):
    def add_seq_tokens(self, seq, tokens, salt=0):
        saved, self.cached = self.cached, {}
        try:
            super().add_seq_tokens(seq, tokens, salt)
        finally:
            saved.update(self.cached)
            self.cached = saved
        return 0


MUTANTS = [BlockTokensOnly, SaltIgnored, EvictNewest, EvictBeforeFree, ReleaseForward, NoRevive,
           NoRetention, CachePartialTail, NeverReuse]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutant):
    assert P.failures(P.oracle_factory(mutant)), f"{mutant.__name__} passed every pin"
