"""Pins of the copy-on-write oracle (oracle.scatter.copy_blocks) through its whole mechanism.

"PagedAttention -- Math + Memory Model", section "Copy-on-write: sharing blocks across samples":
forked samples share their parent's blocks by reference, and a sample about to write into a
shared block first gets a private copy.  What that must preserve is fixed by the definition of a
sequence: after any interleaving of forks and appends, every sequence's logical K/V (read back
through its own block table) is its own token history.  These tests check exactly that against
histories kept as plain arrays, with poisoned pools, so a missing, misdirected or partial copy
shows up as poison or as another sequence's tokens.
"""
import numpy as np
import pytest

from oracle import scatter as SC
from oracle.allocator import BlockAllocatorModel

B, HK, D, N = 16, 2, 64, 64
POISON = 0x7FC1


def _rows(rng, n):
    # raw 16-bit patterns (bf16 storage), never the poison pattern
    r = rng.integers(0, 0x7F00, size=(n, HK, D), dtype=np.uint16)
    return r, rng.integers(0, 0x7F00, size=(n, HK, D), dtype=np.uint16)


class World:
    """Allocator model + oracle pools + each sequence's expected history."""

    def __init__(self, seed, with_copy=True):
        self.rng = np.random.default_rng(seed)
        self.alloc = BlockAllocatorModel(N, B, self.rng.permutation(N))
        self.kp, self.vp = SC.empty_pools(N, HK, D, B, np.uint16, POISON)
        self.hist = {}
        self.with_copy = with_copy
        self.copies = 0

    def append(self, seq, n):
        slots, pairs = self.alloc.alloc(seq, n)
        if self.with_copy:
            SC.copy_blocks(self.kp, self.vp, pairs)
        self.copies += len(pairs)
        k, v = _rows(self.rng, n)
        SC.reshape_and_cache(k, v, np.array(slots), self.kp, self.vp)
        hk, hv = self.hist.get(seq, (np.zeros((0, HK, D), np.uint16),) * 2)
        self.hist[seq] = (np.concatenate([hk, k]), np.concatenate([hv, v]))

    def fork(self, parent, child, n):
        self.alloc.fork(parent, child, n)
        hk, hv = self.hist[parent]
        self.hist[child] = (hk[:n].copy(), hv[:n].copy())

    def check(self):
        for seq, (hk, hv) in self.hist.items():
            K, V = SC.gather_logical(self.kp, self.vp, self.alloc.block_table(seq), len(hk))
            assert np.array_equal(K, hk), f"keys of sequence {seq}"
            assert np.array_equal(V, hv), f"values of sequence {seq}"


def test_parallel_sampling_from_an_unaligned_prompt():
    w = World(1)
    w.append(0, 40)                 # 2.5 blocks: the last one is shared partially
    w.fork(0, 1, 40)
    w.fork(0, 2, 40)
    w.append(1, 3)                  # copies the shared partial block
    w.append(2, 1)                  # copies it again, for the second sample
    w.append(0, 2)                  # the parent now holds the original alone: no copy
    assert w.copies == 2
    w.check()
    # the children's tables differ from the parent's exactly in the last block
    t0, t1, t2 = (w.alloc.block_table(s) for s in (0, 1, 2))
    assert t0[:2] == t1[:2] == t2[:2] and len({t0[2], t1[2], t2[2]}) == 3


def test_without_the_copy_the_child_loses_its_prefix():
    # the same script with copy_blocks skipped: the child's private block holds only poison
    # before its own token, so its history is wrong -- the pin above depends on the copy
    w = World(1, with_copy=False)
    w.append(0, 40)
    w.fork(0, 1, 40)
    w.append(1, 3)
    with pytest.raises(AssertionError):
        w.check()


def test_aligned_fork_needs_no_copy():
    w = World(2)
    w.append(0, 48)                 # exactly 3 blocks
    w.fork(0, 1, 48)
    w.append(1, 5)
    assert w.copies == 0
    w.check()


def test_random_fork_and_append_scripts():
    for seed in range(6):
        w = World(100 + seed)
        w.append(0, int(w.rng.integers(1, 60)))
        nxt = 1
        for _ in range(40):
            live = list(w.hist)
            if w.rng.random() < 0.3 and len(w.alloc.free) > 8:
                p = int(w.rng.choice(live))
                n = int(w.rng.integers(0, len(w.hist[p][0]) + 1))
                w.fork(p, nxt, n)
                nxt += 1
            else:
                s = int(w.rng.choice(live))
                n = int(w.rng.integers(1, 20))
                need = -(-(len(w.hist[s][0]) + n) // B) - -(-len(w.hist[s][0]) // B) + 1
                if need > len(w.alloc.free):
                    continue
                w.append(s, n)
        assert w.copies > 0
        w.check()


def test_copy_blocks_copies_every_head_of_both_pools_and_skips_bad_ids():
    rng = np.random.default_rng(3)
    kp, vp = SC.empty_pools(8, HK, D, B, np.uint16, POISON)
    kp.view(np.uint16)[...] = rng.integers(0, 65535, size=kp.shape, dtype=np.uint16)
    vp.view(np.uint16)[...] = rng.integers(0, 65535, size=vp.shape, dtype=np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    SC.copy_blocks(kp, vp, [(1, 5), (2, 6), (-1, 3), (4, 8)])
    assert np.array_equal(kp[5], k0[1]) and np.array_equal(vp[5], v0[1])
    assert np.array_equal(kp[6], k0[2]) and np.array_equal(vp[6], v0[2])
    untouched = [0, 1, 2, 3, 4, 7]
    assert np.array_equal(kp[untouched], k0[untouched]) and np.array_equal(vp[untouched], v0[untouched])
