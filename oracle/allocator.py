"""O2: the block manager, as plain Python lists and dicts.

Test infrastructure only (see the package docstring).

What it follows:

* Fixed-size physical blocks in one pool, any free block serving any
  sequence; a per-sequence block table maps logical block i (tokens
  i*B .. (i+1)*B-1) to a physical block -- "PagedAttention -- Math + Memory
  Model", sections "PagedAttention: blocks and the block table" and "Why
  fragmentation nearly vanishes"; "KV-cache paging in vLLM", section
  "PagedAttention: Paging for KV-Caches".
* On-demand append: a sequence starts with zero blocks and takes one free
  block when it needs a slot past its last block (same section of
  "PagedAttention -- Math + Memory Model").
* Free list order: take from the head, return to the tail, as the
  simulator of "KV-Cache Optimization & PagedAttention for Long-Context
  Agents" does (section "Python Implementation: Paged KV-Cache Virtual
  Memory Simulator"); a freed sequence returns its blocks in logical order.
* Sharing and copy-on-write: sequences may point their early table entries
  at the same physical blocks, a per-block reference count tracks sharers,
  a write into a block others still share first copies that one block to a
  fresh one and decrements the original, and a block goes back to the pool
  when its count reaches zero -- "PagedAttention -- Math + Memory Model",
  section "Copy-on-write: sharing blocks across samples".

Readings where the pages leave the policy open (each one fixes a unique
result, so the C++ allocator can be compared bit for bit):

* sharing is an explicit ``fork(parent, child, n)``: the child points at the
  parent's first ceil(n/B) blocks (the simulator's hash lookup shares only
  a prompt's first block; a fork shares them all);
* running out of blocks changes nothing (the simulator raises after it has
  already taken some blocks);
* only a write into the partly filled last block can hit a shared block, so
  copy-on-write is checked on the first token an ``alloc`` appends.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(MemoryError):
    """The pool has fewer free blocks than the request needs; nothing was changed."""


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.B = block_size
        self.free: List[int] = order            # head = next block handed out
        self.ref: List[int] = [0] * num_blocks  # sequences whose table holds the block
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- queries -------------------------------------------------------------
    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def seq_len(self, seq: int) -> int:
        return self.lens[seq]

    def slot(self, seq: int, pos: int) -> int:
        """Physical slot of logical position pos: table[pos // B] * B + pos % B."""
        return self.tables[seq][pos // self.B] * self.B + pos % self.B

    def stats(self) -> dict:
        allocated = sum(1 for r in self.ref if r > 0)
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "allocated_blocks": allocated,
            "shared_blocks": sum(1 for r in self.ref if r > 1),
            "num_seqs": len(self.tables),
            "live_tokens": sum(self.lens.values()),
            "allocated_slots": allocated * self.B,
        }

    # -- operations ----------------------------------------------------------
    def alloc(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append n tokens to seq (created empty if unknown); returns (slots, copy pairs)."""
        if n < 0:
            raise ValueError("n must be >= 0")
        B = self.B
        table = self.tables.get(seq, [])
        L = self.lens.get(seq, 0)
        fresh = sum(1 for p in range(L, L + n) if p % B == 0)
        cow = n > 0 and L % B != 0 and self.ref[table[-1]] > 1
        if fresh + (1 if cow else 0) > len(self.free):
            raise OutOfBlocks(f"need {fresh + cow} blocks, {len(self.free)} free")
        if seq not in self.tables:
            self.tables[seq] = table
        slots: List[int] = []
        pairs: List[Tuple[int, int]] = []
        for p in range(L, L + n):
            if p % B == 0:
                b = self.free.pop(0)
                self.ref[b] = 1
                table.append(b)
            elif p == L and cow:
                old = table[-1]
                new = self.free.pop(0)
                self.ref[old] -= 1
                self.ref[new] = 1
                table[-1] = new
                pairs.append((old, new))
            slots.append(table[p // B] * B + p % B)
        self.lens[seq] = L + n
        return slots, pairs

    def fork(self, parent: int, child: int, n: int = -1) -> None:
        """Child shares the parent's first ceil(n/B) blocks (n = -1: the parent's whole length)."""
        if parent not in self.tables:
            raise KeyError(parent)
        if child in self.tables:
            raise ValueError(f"sequence {child} already exists")
        plen = self.lens[parent]
        if n < 0:
            n = plen
        if n > plen:
            raise ValueError("cannot share more tokens than the parent holds")
        nb = -(-n // self.B)
        shared = self.tables[parent][:nb]
        for b in shared:
            self.ref[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = n

    def free_seq(self, seq: int) -> None:
        """Drop seq: each of its blocks loses one reference, in logical order; at zero it rejoins
        the tail of the free list."""
        table = self.tables.pop(seq)
        del self.lens[seq]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- convenience -----------------------------------------------------------
    def run(self, ops) -> None:
        """Apply a workload's prompt script (dicts with op alloc / fork / free)."""
        for op in ops:
            kind = op["op"]
            if kind == "alloc":
                self.alloc(op["seq"], op["n"])
            elif kind == "fork":
                self.fork(op["parent"], op["child"], op["n"])
            elif kind == "free":
                self.free_seq(op["seq"])
            else:
                raise ValueError(kind)
