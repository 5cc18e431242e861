"""The reference block manager against the pages' worked examples and the
tail-waste bound."""
import numpy as np
import pytest

from oracle.alloc_ref import BlockPool, OutOfBlocks
from tests.conftest import load_golden

G = load_golden("alloc_worked_examples.txt")


def test_example1_blocks_and_slots():
    g = G["example1"]
    pool = BlockPool(64, g["block_size"], shuffle_seed=1)
    for i, L in enumerate(g["lens"]):
        pool.add_seq(i, L)
    assert [len(pool.tables[i]) for i in range(2)] == g["blocks"]
    total = sum(pool.slots_reserved(i) for i in range(2))
    used = sum(pool.lens[i] for i in range(2))
    assert total == g["slots_total"]
    assert used == g["slots_used"]
    assert total - used == g["slots_empty"]


def test_example1_reserving_max_per_request():
    g = G["example1_reserve"]
    # contiguous reservation of a fixed maximum per request, as the example
    # contrasts: a "block" the size of the reservation
    pool = BlockPool(8, g["reserve_per_request"])
    for i, L in enumerate(g["lens"]):
        pool.add_seq(i, L)
    total = sum(pool.slots_reserved(i) for i in range(2))
    assert total == g["slots_total"]
    assert total - sum(g["lens"]) == g["slots_empty"]


def test_example2_waste():
    g = G["example2"]
    pool = BlockPool(16, g["block_size"])
    for i, L in enumerate(g["lens"]):
        pool.add_seq(i, L)
    assert [pool.slots_reserved(i) for i in range(3)] == g["slots"]
    assert [pool.tail_waste(i) for i in range(3)] == g["waste"]
    assert sum(pool.tail_waste(i) for i in range(3)) == g["waste_total"]


@pytest.mark.parametrize("rec", ["example2_grow", "example2_cross"])
def test_example2_growth(rec):
    g = G[rec]
    pool = BlockPool(16, g["block_size"])
    pool.add_seq(0, g["start_len"])
    before = len(pool.tables[0])
    slots, pairs = pool.append(0, g["grow_by"])
    assert len(pool.tables[0]) - before == g["new_blocks"]
    assert pairs == [] and len(slots) == g["grow_by"]


def test_tail_waste_bound():
    """w(L) = B*ceil(L/B) - L and 0 <= w <= B-1 for every length."""
    rng = np.random.default_rng(0)
    for B in (1, 4, 8, 16, 32, 128):
        pool = BlockPool(100000, B)
        for i, L in enumerate(rng.integers(1, 5000, size=200)):
            pool.add_seq(i, int(L))
            w = pool.tail_waste(i)
            assert w == B * (-(-int(L) // B)) - int(L)
            assert 0 <= w <= B - 1
            pool.free_seq(i)


def test_slots_are_block_times_size_plus_offset():
    pool = BlockPool(10, 4, shuffle_seed=3)
    pool.add_seq(0, 0)
    slots, _ = pool.append(0, 9)
    t = pool.tables[0]
    assert slots == [t[p // 4] * 4 + p % 4 for p in range(9)]
    assert len(set(slots)) == 9


def test_fork_shares_and_cow_copies_only_shared_partial_tail():
    pool = BlockPool(20, 4, shuffle_seed=5)
    pool.add_seq(0, 6)  # blocks: one full, one holding 2 of 4
    pool.fork(0, 1)
    assert all(pool.ref[b] == 2 for b in pool.tables[0])
    full, tail = pool.tables[0]
    free0 = pool.num_free()
    slots, pairs = pool.append(1, 1)  # writes position 6 into the shared tail
    assert len(pairs) == 1 and pairs[0][0] == tail
    new = pairs[0][1]
    assert pool.tables[1] == [full, new] and pool.tables[0] == [full, tail]
    assert pool.ref[tail] == 1 and pool.ref[new] == 1 and pool.ref[full] == 2
    assert slots == [new * 4 + 2]
    assert pool.num_free() == free0 - 1
    # the parent now owns its tail alone: no copy on its next write
    _, pairs0 = pool.append(0, 1)
    assert pairs0 == []


def test_fork_at_block_boundary_needs_no_copy():
    pool = BlockPool(20, 4)
    pool.add_seq(0, 8)
    pool.fork(0, 1)
    slots, pairs = pool.append(1, 1)
    assert pairs == [] and len(pool.tables[1]) == 3
    assert pool.ref[pool.tables[1][2]] == 1


def test_free_reclaims_only_at_zero():
    pool = BlockPool(20, 4)
    pool.add_seq(0, 7)
    pool.fork(0, 1)
    n = pool.num_free()
    pool.free_seq(0)
    assert pool.num_free() == n  # child still references both blocks
    pool.free_seq(1)
    assert pool.num_free() == 20


def test_out_of_blocks_is_all_or_nothing():
    pool = BlockPool(5, 4)
    pool.add_seq(0, 12)
    with pytest.raises(OutOfBlocks):
        pool.add_seq(1, 9)  # needs 3, 2 free
    assert pool.num_free() == 2 and 1 not in pool.tables
    with pytest.raises(OutOfBlocks):
        pool.append(0, 9)  # needs 3 more
    assert pool.lens[0] == 12 and len(pool.tables[0]) == 3 and pool.num_free() == 2
