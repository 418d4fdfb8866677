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

Swapping to host memory: instead of evicting a sequence and recomputing its cache, an engine
can move its blocks to host memory and bring them back later ("Reserve for the worst case, or
page", section "What this model leaves out").  The pages give no policy; the readings are:

* host memory is a fixed number of host slots of one block each, handed out from the head of
  their own free list and returned to its tail (the device pool's discipline);
* ``swap_out(seq)`` moves every block of a device-resident sequence, in logical order: each takes
  the next host slot, gives a (device block, host slot) copy pair, and loses the sequence's
  reference exactly as ``free_seq`` drops it (a block still shared stays on the device for its
  other sequences; the host copy is this sequence's own);
* ``swap_in(seq)`` takes fresh device blocks in logical order, gives (host slot, device block)
  pairs and returns the host slots, in order, to the tail of their list; the sequence comes
  back with private blocks and its length;
* both are all or nothing (too few host slots, or too few device blocks, change nothing); a
  swapped-out sequence cannot append or be forked until it is back, and freeing it returns its
  host slots.
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
        self.host_free: List[int] = []                          # head = next host slot handed out
        self.num_host = 0
        self.swapped: Dict[int, Tuple[List[int], int]] = {}    # seq -> (host slots, length)

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
        if seq in self.swapped:
            raise ValueError(f"sequence {seq} is swapped out")
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
        if child in self.tables or child in self.swapped:
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
        the tail of the free list.  A swapped-out sequence returns its host slots instead."""
        if seq in self.swapped:
            slots, _ = self.swapped.pop(seq)
            self.host_free.extend(slots)
            return
        table = self.tables.pop(seq)
        del self.lens[seq]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- swapping to host memory ------------------------------------------------
    def set_swap_space(self, num_host: int) -> None:
        """num_host host slots, handed out in order 0, 1, ..."""
        if num_host < 0 or self.num_host:
            raise ValueError("swap space is set once, with a non-negative size")
        self.num_host = num_host
        self.host_free = list(range(num_host))

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """Move a device-resident sequence to host slots; returns (device block, host slot) pairs."""
        table = self.tables[seq]
        if len(table) > len(self.host_free):
            raise OutOfBlocks(f"need {len(table)} host slots, {len(self.host_free)} free")
        pairs = []
        for b in table:
            h = self.host_free.pop(0)
            pairs.append((b, h))
        L = self.lens[seq]
        self.free_seq(seq)
        self.swapped[seq] = ([h for _, h in pairs], L)
        return pairs

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """Bring a swapped-out sequence back into fresh device blocks; returns (host slot, device
        block) pairs."""
        slots, L = self.swapped[seq]
        if len(slots) > len(self.free):
            raise OutOfBlocks(f"need {len(slots)} blocks, {len(self.free)} free")
        del self.swapped[seq]
        table, pairs = [], []
        for h in slots:
            b = self.free.pop(0)
            self.ref[b] = 1
            table.append(b)
            pairs.append((h, b))
        self.host_free.extend(slots)
        self.tables[seq] = table
        self.lens[seq] = L
        return pairs

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
