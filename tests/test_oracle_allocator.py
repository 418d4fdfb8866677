"""Pins of the allocator model (O2): the pages' fixtures, copy-on-write, and invariants."""
import json
import os

import pytest
from hypothesis import given, settings, strategies as st

from oracle.allocator import BlockAllocatorModel, OutOfBlocks

FIX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "block_tables.json")))


def test_vllm_post_block_tables():
    f = FIX["vllm_post_example"]
    head = f["head_of_free_order"]
    rest = [b for b in range(f["num_blocks"]) if b not in head]
    a = BlockAllocatorModel(f["num_blocks"], f["block_size"], head + rest)
    a.alloc("A", f["session_a"]["tokens"])
    a.alloc("B", f["session_b"]["tokens"])
    assert a.block_table("A") == f["session_a"]["table"]
    assert a.block_table("B") == f["session_b"]["table"]
    # logical position i of A lives in physical block table[i // 16], slot offset i % 16
    assert a.slot("A", 0) == 47 * 16
    assert a.slot("A", 17) == 12 * 16 + 1
    assert a.slot("A", 39) == 91 * 16 + 7


def test_simulator_demo_trace():
    f = FIX["simulator_demo"]
    a = BlockAllocatorModel(f["num_blocks"], f["block_size"])
    a.alloc("A", 48)
    a.fork("A", "B", 16)
    slots, pairs = a.alloc("B", 16)
    assert pairs == []
    assert a.block_table("A") == f["table_a"]
    assert a.block_table("B") == f["table_b"]
    assert a.ref[0] == f["ref_block0_after_b"]
    assert len(a.free) == f["free_after_allocs"]
    a.free_seq("A")
    assert len(a.free) == f["free_after_free_a"]
    a.free_seq("B")
    assert len(a.free) == f["free_after_free_b"]
    assert a.free[-4:] == f["free_tail_after_all"]
    assert all(r == 0 for r in a.ref)


def test_on_demand_append_and_slots():
    a = BlockAllocatorModel(8, 4, [5, 2, 7, 0, 1, 3, 4, 6])
    a.alloc(1, 0)
    assert a.block_table(1) == [] and a.seq_len(1) == 0     # starts owning zero blocks
    s, _ = a.alloc(1, 3)
    assert s == [20, 21, 22] and a.block_table(1) == [5]
    s, _ = a.alloc(1, 1)
    assert s == [23] and a.block_table(1) == [5]            # fills the block, no new one
    s, _ = a.alloc(1, 1)
    assert s == [8] and a.block_table(1) == [5, 2]          # slot B+1 takes a fresh block


def test_copy_on_write_on_shared_partial_block():
    a = BlockAllocatorModel(10, 4)
    a.alloc("p", 6)                   # blocks [0, 1]; block 1 holds 2 tokens
    a.fork("p", "c", 6)               # child shares both
    assert a.ref[0] == 2 and a.ref[1] == 2
    slots, pairs = a.alloc("c", 3)    # child writes into shared block 1 -> copy it
    assert pairs == [(1, 2)]
    assert a.block_table("c") == [0, 2, 3] and a.block_table("p") == [0, 1]
    assert slots == [2 * 4 + 2, 2 * 4 + 3, 3 * 4 + 0]
    assert a.ref[1] == 1 and a.ref[2] == 1 and a.ref[3] == 1 and a.ref[0] == 2
    # the parent's own next write no longer sees a shared block
    _, pairs = a.alloc("p", 1)
    assert pairs == []


def test_fork_aligned_prefix_needs_no_copy():
    a = BlockAllocatorModel(32, 16)
    a.alloc("P", 64)
    for i in range(3):
        a.fork("P", i, 64)
    a.free_seq("P")
    assert [a.ref[b] for b in range(4)] == [3, 3, 3, 3]
    for i in range(3):
        _, pairs = a.alloc(i, 5)
        assert pairs == []
    assert a.stats()["shared_blocks"] == 4


def test_out_of_blocks_changes_nothing():
    a = BlockAllocatorModel(4, 4)
    a.alloc("x", 10)                  # 3 blocks
    before = (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()}, dict(a.lens))
    with pytest.raises(OutOfBlocks):
        a.alloc("x", 7)               # needs 2 more blocks, 1 free
    with pytest.raises(OutOfBlocks):
        a.alloc("y", 5)
    after = (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()}, dict(a.lens))
    assert before == after
    assert "y" not in a.tables


def test_errors():
    a = BlockAllocatorModel(4, 4)
    with pytest.raises(KeyError):
        a.free_seq("nope")
    with pytest.raises(KeyError):
        a.fork("nope", "c", 1)
    a.alloc("p", 2)
    a.alloc("q", 1)
    with pytest.raises(ValueError):
        a.fork("p", "q", 1)
    with pytest.raises(ValueError):
        a.fork("p", "c", 3)
    with pytest.raises(ValueError):
        a.alloc("p", -1)
    with pytest.raises(ValueError):
        BlockAllocatorModel(4, 4, [0, 1, 1, 2])


def check_invariants(a: BlockAllocatorModel):
    N, B = a.num_blocks, a.B
    counts = [0] * N
    for seq, t in a.tables.items():
        assert len(t) == -(-a.lens[seq] // B)
        for b in t:
            counts[b] += 1
    assert counts == a.ref                                    # ref = number of tables holding b
    assert len(set(a.free)) == len(a.free)                    # no duplicates on the free list
    allocated = [b for b in range(N) if a.ref[b] > 0]
    assert sorted(a.free + allocated) == list(range(N))       # free + allocated = pool
    for seq, t in a.tables.items():                           # unused tail <= B - 1
        assert len(t) * B - a.lens[seq] <= B - 1


op_strategy = st.lists(
    st.tuples(st.sampled_from(["alloc", "alloc", "alloc", "fork", "free"]),
              st.integers(0, 5), st.integers(0, 5), st.integers(-1, 40)),
    max_size=60)


@settings(max_examples=300, deadline=None)
@given(ops=op_strategy, B=st.sampled_from([1, 2, 4, 16]), N=st.integers(1, 24),
       perm_seed=st.integers(0, 1000))
def test_invariants_under_random_ops(ops, B, N, perm_seed):
    import random
    order = list(range(N))
    random.Random(perm_seed).shuffle(order)
    a = BlockAllocatorModel(N, B, order)
    for kind, x, y, n in ops:
        try:
            if kind == "alloc":
                a.alloc(x, max(n, 0))
            elif kind == "fork":
                a.fork(x, y, n)
            else:
                a.free_seq(x)
        except (KeyError, ValueError, OutOfBlocks):
            pass
        check_invariants(a)
    for seq in list(a.tables):
        a.free_seq(seq)
    assert sorted(a.free) == list(range(N)) and all(r == 0 for r in a.ref)


def test_slots_are_distinct_and_follow_table():
    a = BlockAllocatorModel(64, 16, list(reversed(range(64))))
    seen = set()
    for seq, n in [(0, 100), (1, 17), (2, 33), (0, 5), (1, 1)]:
        start = a.lens.get(seq, 0)
        slots, _ = a.alloc(seq, n)
        for i, s in enumerate(slots):
            p = start + i
            assert s == a.block_table(seq)[p // 16] * 16 + p % 16
            assert s not in seen
            seen.add(s)
