"""Pins of swapping sequences to host memory (oracle.allocator swap_out / swap_in with
oracle.scatter.move_blocks).

"Reserve for the worst case, or page", section "What this model leaves out": a preempted sequence's
blocks can go to host memory instead of being dropped and recomputed.  What that must preserve is fixed
by the definition of a sequence: after any interleaving of appends, forks, swaps and frees -- with the
freed device blocks reused by other sequences in between -- every device-resident sequence reads back
its own token history through its table, and every swapped-out one holds it in its host slots.  Pools
are poisoned, so a missing, misdirected or partial copy shows up.
"""
import numpy as np
import pytest

from oracle import scatter as SC
from oracle.allocator import BlockAllocatorModel, OutOfBlocks

B, HK, D, N, H = 8, 2, 16, 24, 20
POISON = 0x7FC1


class World:
    def __init__(self, seed, copy=True):
        self.rng = np.random.default_rng(seed)
        self.a = BlockAllocatorModel(N, B, self.rng.permutation(N))
        self.a.set_swap_space(H)
        self.kp, self.vp = SC.empty_pools(N, HK, D, B, np.uint16, POISON)
        self.kh, self.vh = SC.empty_pools(H, HK, D, B, np.uint16, POISON)
        self.hist = {}
        self.copy = copy

    def append(self, seq, n):
        slots, pairs = self.a.alloc(seq, n)
        SC.copy_blocks(self.kp, self.vp, pairs)
        k = self.rng.integers(0, 0x7F00, size=(n, HK, D), dtype=np.uint16)
        v = self.rng.integers(0, 0x7F00, size=(n, HK, D), dtype=np.uint16)
        SC.reshape_and_cache(k, v, np.array(slots), self.kp, self.vp)
        hk, hv = self.hist.get(seq, (np.zeros((0, HK, D), np.uint16),) * 2)
        self.hist[seq] = (np.concatenate([hk, k]), np.concatenate([hv, v]))

    def swap_out(self, seq):
        pairs = self.a.swap_out(seq)
        if self.copy:
            SC.move_blocks(self.kp, self.vp, self.kh, self.vh, pairs)
        return pairs

    def swap_in(self, seq):
        pairs = self.a.swap_in(seq)
        if self.copy:
            SC.move_blocks(self.kh, self.vh, self.kp, self.vp, pairs)
        return pairs

    def check(self):
        a = self.a
        for seq, (hk, hv) in self.hist.items():
            if seq in a.swapped:
                slots, L = a.swapped[seq]
                assert L == len(hk)
                K, V = SC.gather_logical(self.kh, self.vh, slots, L)
            else:
                K, V = SC.gather_logical(self.kp, self.vp, a.block_table(seq), len(hk))
            assert np.array_equal(K, hk) and np.array_equal(V, hv), f"sequence {seq}"
        # invariants: reference counts are table membership; device and host slots are conserved
        refs = [0] * N
        for t in a.tables.values():
            for b in t:
                refs[b] += 1
        assert refs == a.ref
        assert len(a.free) + sum(1 for r in a.ref if r > 0) == N
        assert len(a.host_free) + sum(len(s) for s, _ in a.swapped.values()) == H
        assert len(set(a.host_free)) == len(a.host_free)


def test_swap_round_trip_with_the_blocks_reused_in_between():
    w = World(1)
    w.append(0, 21)
    w.append(1, 30)
    table0 = w.a.block_table(0)
    pairs = w.swap_out(0)
    assert [b for b, _ in pairs] == table0                  # every block, in logical order
    assert [h for _, h in pairs] == [0, 1, 2]               # host slots from the head of their list
    assert w.a.free[-3:] == table0                          # device blocks back at the tail
    w.append(2, 24)                                         # reuses freed blocks
    w.check()
    w.a.free_seq(2)
    del w.hist[2]
    back = w.swap_in(0)
    assert [h for h, _ in back] == [0, 1, 2]
    assert w.a.host_free[-3:] == [0, 1, 2]                  # returned to the tail
    w.append(0, 5)
    w.check()


def test_without_the_copy_the_swapped_sequence_loses_its_tokens():
    w = World(1, copy=False)
    w.append(0, 21)
    w.swap_out(0)
    with pytest.raises(AssertionError):
        w.check()


def test_swapping_a_forked_child_leaves_the_parent_alone():
    w = World(2)
    w.append(0, 20)                     # 2.5 blocks
    w.a.fork(0, 1, 20)
    w.hist[1] = tuple(x.copy() for x in w.hist[0])
    shared = w.a.block_table(0)
    w.swap_out(1)
    assert w.a.block_table(0) == shared and all(w.a.ref[b] == 1 for b in shared)
    w.append(0, 3)                      # the parent's last block is no longer shared: no copy
    back = w.swap_in(1)
    assert not set(b for _, b in back) & set(w.a.block_table(0))     # the child's blocks are private
    w.append(1, 4)
    w.check()


def _state(a):
    return (list(a.free), list(a.ref), list(a.host_free), {k: list(t) for k, t in a.tables.items()},
            {k: (list(sl), L) for k, (sl, L) in a.swapped.items()}, dict(a.lens))


def test_swaps_are_all_or_nothing():
    w = World(3)
    w.append(0, 8 * 18)                 # 18 of 24 blocks
    w.append(1, 8 * 5)
    w.swap_out(1)                       # 5 of 20 host slots
    snap = _state(w.a)
    with pytest.raises(OutOfBlocks):
        w.a.swap_out(0)                 # 18 host slots needed, 15 free
    assert _state(w.a) == snap
    w.append(2, 8 * 6)                  # the device pool is full now
    snap = _state(w.a)
    with pytest.raises(OutOfBlocks):
        w.a.swap_in(1)                  # 5 blocks needed, none free
    assert _state(w.a) == snap
    with pytest.raises(ValueError):
        w.a.alloc(1, 1)                 # a swapped-out sequence cannot append
    with pytest.raises(KeyError):
        w.a.fork(1, 9, 1)               # nor be forked
    w.check()
    w.a.free_seq(1)                     # freeing it returns its host slots
    del w.hist[1]
    assert len(w.a.host_free) == H
    w.check()


def test_random_scripts_of_appends_forks_swaps_and_frees():
    for seed in range(8):
        w = World(100 + seed)
        nxt = 0
        for _ in range(60):
            live = [s for s in w.hist if s not in w.a.swapped]
            out = list(w.a.swapped)
            r = w.rng.random()
            try:
                if r < 0.35 or not live:
                    s = int(w.rng.choice(live)) if live and w.rng.random() < 0.6 else nxt
                    if s == nxt:
                        nxt += 1
                    w.append(s, int(w.rng.integers(1, 20)))
                elif r < 0.5:
                    p = int(w.rng.choice(live))
                    n = int(w.rng.integers(0, len(w.hist[p][0]) + 1))
                    w.a.fork(p, nxt, n)
                    w.hist[nxt] = (w.hist[p][0][:n].copy(), w.hist[p][1][:n].copy())
                    nxt += 1
                elif r < 0.7:
                    w.swap_out(int(w.rng.choice(live)))
                elif r < 0.85 and out:
                    w.swap_in(int(w.rng.choice(out)))
                else:
                    s = int(w.rng.choice(list(w.hist)))
                    w.a.free_seq(s)
                    del w.hist[s]
            except OutOfBlocks:
                pass
            w.check()
