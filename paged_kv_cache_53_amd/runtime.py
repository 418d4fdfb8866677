"""The decode-step runtime around the kernels: device pools + host allocator, and a batch.

PagedKVCache   one layer's key/value pools on the device and the host block allocator that
               hands out their slots (prompt writes go allocator -> scatter kernel).  With
               enable_swap(host_blocks) it also keeps pinned host swap space, and swap_out /
               swap_in move a sequence's blocks there and back (allocator pairs -> copy kernel).  With
               dtype torch.float8_e4m3fn the pools hold FP8 E4M3 codes under the per-tensor
               scales k_scale / v_scale (the scatter quantises, decode reads the scaled values).
DecodeBatch    a fixed set of sequences decoded together: device block tables and lengths,
               a workspace, and ``step()`` -- one decode step of the whole hot path:
                 1. host: the allocator appends one token to every sequence (C++, one call),
                    writing the new slots into a pinned, double-buffered stage
                 2. copy_blocks kernel, when an append hit a shared block (copy-on-write)
                 3. decode_step: a prologue kernel (append of the new block ids into the device
                    tables and lengths + 1, the plan of the attention's work, and the scatter of
                    the new tokens' K/V into their slots; the slots are read from the stage in
                    place), then the attention and merge kernels
               (``step(fused=False)`` copies the slots to the device and makes the separate
               append_slots, reshape_and_cache and paged_attention_decode calls instead.)
               Host work for step i+1 overlaps the GPU work of step i; the host waits only
               before reusing a staging buffer that a step may still be reading.
FlatKVCache    the flat-span alternative: one contiguous virtual span per sequence (SpanPool),
               physical memory mapped as the sequence grows, no block table.
FlatDecodeBatch  one decode step over flat spans: span backing grown on the host when a token
               starts an unmapped chunk, slots staged as above, the append kernel bumps the
               lengths, scatter, then decode that computes block ids from each row's span.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import (PKV_ERR_INVALID, Allocator, PKVError, SpanPool, append_slots, check_block_tables, copy_blocks,
               decode_step, key_pool_shape, paged_attention_decode, paged_attention_decode_flat, reshape_and_cache,
               reshape_and_cache_spans, swap_blocks, value_pool_shape, workspace_size)


class PagedKVCache:
    def __init__(self, num_blocks: int, block_size: int, n_kv_heads: int, head_dim: int, dtype,
                 device="cuda", free_order: Optional[Sequence[int]] = None, fill: str = "zero",
                 k_scale: Optional[float] = None, v_scale: Optional[float] = None):
        self.num_blocks, self.block_size = num_blocks, block_size
        self.n_kv_heads, self.head_dim, self.dtype, self.device = n_kv_heads, head_dim, dtype, device
        self.quantised = dtype == torch.float8_e4m3fn
        if self.quantised != (k_scale is not None and v_scale is not None):
            raise ValueError("k_scale and v_scale go with (and only with) an FP8 cache")
        self.scales = {"k_scale": k_scale, "v_scale": v_scale} if self.quantised else {}
        self.allocator = Allocator(num_blocks, block_size, free_order)
        ks = key_pool_shape(num_blocks, n_kv_heads, head_dim, block_size, dtype)
        vs = value_pool_shape(num_blocks, n_kv_heads, head_dim, block_size)
        if self.quantised:
            code = {"zero": 0x00, "nan": 0x7F}.get(fill)
            if fill == "randn":
                self.k_pool = torch.randint(0, 0x7F, ks, device=device, dtype=torch.uint8).view(dtype)
                self.v_pool = torch.randint(0, 0x7F, vs, device=device, dtype=torch.uint8).view(dtype)
            elif code is not None:
                self.k_pool = torch.full(ks, code, device=device, dtype=torch.uint8).view(dtype)
                self.v_pool = torch.full(vs, code, device=device, dtype=torch.uint8).view(dtype)
            else:
                raise ValueError(fill)
        elif fill == "randn":
            self.k_pool = torch.randn(ks, device=device, dtype=torch.float32).to(dtype)
            self.v_pool = torch.randn(vs, device=device, dtype=torch.float32).to(dtype)
        elif fill == "nan":
            self.k_pool = torch.full(ks, float("nan"), device=device, dtype=dtype)
            self.v_pool = torch.full(vs, float("nan"), device=device, dtype=dtype)
        elif fill == "zero":
            self.k_pool = torch.zeros(ks, device=device, dtype=dtype)
            self.v_pool = torch.zeros(vs, device=device, dtype=dtype)
        else:
            raise ValueError(fill)

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Appends len(k) tokens to seq: slots from the allocator, rows written by the scatter kernel."""
        slots, pairs = self.allocator.alloc(seq, int(k.shape[0]))
        self.apply_copies(pairs)
        if slots:
            reshape_and_cache(k, v, torch.tensor(slots, dtype=torch.int64, device=self.device),
                              self.k_pool, self.v_pool, **self.scales)

    def apply_copies(self, pairs) -> None:
        """Makes the private block copies a copy-on-write append asked for (before its scatter)."""
        if pairs:
            copy_blocks(torch.tensor(pairs, dtype=torch.int32, device=self.device), self.k_pool, self.v_pool)

    def has_shared_blocks(self) -> bool:
        """Whether some block is referenced by more than one sequence (decode then keeps blocks cacheable)."""
        return self.allocator.stats()["shared_blocks"] > 0

    def fork(self, parent: int, child: int, n_tokens: int = -1) -> None:
        self.allocator.fork(parent, child, n_tokens)

    def enable_swap(self, host_blocks: int) -> None:
        """Pinned host swap space of host_blocks blocks (both pools), managed by the allocator."""
        self.allocator.set_swap_space(host_blocks)
        ks = key_pool_shape(host_blocks, self.n_kv_heads, self.head_dim, self.block_size, self.dtype)
        vs = value_pool_shape(host_blocks, self.n_kv_heads, self.head_dim, self.block_size)
        self.k_host = torch.empty(ks, dtype=self.dtype, pin_memory=True)
        self.v_host = torch.empty(vs, dtype=self.dtype, pin_memory=True)

    def swap_out(self, seq: int) -> int:
        """Moves seq's blocks to host memory (copies issued on the current stream, before anything
        later can reuse the freed blocks); returns the number of blocks moved."""
        pairs = self.allocator.swap_out(seq)
        if pairs:
            swap_blocks(torch.tensor(pairs, dtype=torch.int32, device=self.device), self.k_pool, self.v_pool,
                        self.k_host, self.v_host)
        return len(pairs)

    def swap_in(self, seq: int) -> int:
        """Brings seq back into fresh device blocks (its block table changes)."""
        pairs = self.allocator.swap_in(seq)
        if pairs:
            swap_blocks(torch.tensor(pairs, dtype=torch.int32, device=self.device), self.k_host, self.v_host,
                        self.k_pool, self.v_pool)
        return len(pairs)

    def free(self, seq: int) -> None:
        self.allocator.free(seq)


class DecodeBatch:
    def __init__(self, cache: PagedKVCache, seq_ids: Sequence[int], n_q_heads: int, max_seq_len: int,
                 partition_size: int = 512, scale: Optional[float] = None):
        self.cache = cache
        self.seq_ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        self.S = len(self.seq_ids)
        self.n_q_heads = n_q_heads
        self.max_seq_len = max_seq_len
        self.partition_size = partition_size
        self.scale = 1.0 / math.sqrt(cache.head_dim) if scale is None else scale
        B = cache.block_size
        self.stride = max(1, -(-max_seq_len // B))
        cache.allocator.alloc_batch(self.seq_ids, 0)      # sequences with no prompt exist, empty
        tables, lens = cache.allocator.fill_block_tables(self.seq_ids, self.stride, pad=0)
        if int(lens.max(initial=0)) > max_seq_len:
            raise ValueError("a sequence is already longer than max_seq_len")
        dev = cache.device
        self.tables = torch.from_numpy(tables).to(dev)
        self.seq_lens = torch.from_numpy(lens.copy()).to(dev)
        self.host_lens = lens.astype(np.int64)
        self.workspace = torch.empty(max(256, workspace_size(self.S, n_q_heads, cache.head_dim, max_seq_len,
                                                               partition_size)), dtype=torch.uint8, device=dev)
        # A ring of pinned slot stages, and a completion event every STAGE_EVENT_EVERY steps: an event
        # record costs the stream a few microseconds, so one per step would be a measurable share of
        # a step.  Before a stage is rewritten, the step that last read it must have finished.
        self.slot_stage = [torch.empty(self.S, dtype=torch.int64, pin_memory=True) for _ in range(self.STAGES)]
        self.slot_stage_np = [t.numpy() for t in self.slot_stage]
        self.step_events = {}     # step index -> event recorded after that step
        self.slot_dev = torch.empty(self.S, dtype=torch.int64, device=dev)
        self.steps = 0
        self.load_policy = "auto"   # "auto", "streamed" or "cached": how decode reads the pools
        self.vector = False         # one head per KV head on the per-token vector path (decode_only)
        self.check_tables = False   # debug mode: check the device tables before each decode (synchronises)
        self.shared_prefix = self._find_shared_prefix()
        self._check_result = torch.empty(2, dtype=torch.int32, device=dev)

    STAGES = 8
    STAGE_EVENT_EVERY = 4

    def _find_shared_prefix(self) -> int:
        """Tokens at the start of the batch's rows that lie in blocks other rows also read: for each row,
        its leading blocks whose reference count exceeds one (a prompt the rows were forked from), the
        largest such prefix over the rows.  Appends can only shorten it (a row writes into private blocks
        only, copying a partly filled shared block first), so the value taken when the batch is set up or
        refreshed bounds it: tokens it covers that became private are merely read cacheable."""
        c = self.cache
        tables, lens = c.allocator.fill_block_tables(self.seq_ids, self.stride, pad=0)
        best = 0
        for r in range(self.S):
            n = 0
            nb = -(-int(lens[r]) // c.block_size)
            while n < nb and c.allocator.ref_count(int(tables[r, n])) > 1:
                n += 1
            best = max(best, min(int(lens[r]), n * c.block_size))
        return best

    def _load_args(self) -> dict:
        """How decode reads the pools: the shared prefix cacheable and the rest streamed when the rows
        share a prompt, else every tile cacheable when they share other blocks, else streamed.  Measured
        on MI355X, decode us warm / after a 1 GiB write: the shared-prompt swarm 83 / 105 with the prefix
        policy, 88 / 143 every tile cacheable, 116 / 119 streamed; without sharing, streamed loads were as
        fast or faster (bf16 Llama-70B-class 753 / 769 against 845 / 910 cacheable): cacheable loads
        evict dirty lines and pay their write-back."""
        if self.load_policy == "cached":
            return {"shared_kv": True}
        if self.load_policy == "streamed":
            return {}
        if self.load_policy == "prefix" or (self.load_policy == "auto" and self.shared_prefix > 0):
            return {"shared_prefix_tokens": max(1, self.shared_prefix)} if self.shared_prefix else {"shared_kv": True}
        return {"shared_kv": self.cache.has_shared_blocks()}

    def _stage_for(self, n: int) -> int:
        """The stage of step n, once the step that last read it (n - STAGES) has finished."""
        m = n - self.STAGES
        if m >= 0:
            e = m + (-(m + 1)) % self.STAGE_EVENT_EVERY     # the first event step >= m (several n share it)
            ev = self.step_events.get(e)
            if ev is None:
                torch.cuda.current_stream().synchronize()    # not expected: fall back to a full wait
            else:
                ev.synchronize()
            for k in [k for k in self.step_events if k < e]:
                del self.step_events[k]
        return n % self.STAGES

    def _verify_tables(self) -> None:
        """Debug mode: every table entry the next decode reads must name a block of the pool (decode
        clamps an out-of-pool id, which would give a wrong row silently)."""
        c = self.cache
        r = check_block_tables(self.tables, self.seq_lens, c.block_size, c.num_blocks, self.max_seq_len,
                               result=self._check_result)
        bad, first = (int(x) for x in r.cpu())
        if bad:
            raise PKVError(PKV_ERR_INVALID, f"block tables hold {bad} out-of-pool entries (first in batch row {first})")

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, out: torch.Tensor,
             fused: bool = True) -> None:
        """One decode step for every row: append the new token, write its K/V, attend over all tokens.

        fused: one decode_step call, which reads the slots from their pinned staging buffer in place;
        otherwise the slots are copied to the device and append_slots, reshape_and_cache and
        paged_attention_decode run as separate calls.  The results are the same."""
        if int(self.host_lens.max(initial=0)) + 1 > self.max_seq_len:
            raise ValueError("decode step would exceed max_seq_len")
        if self.check_tables:
            self._verify_tables()
        i = self._stage_for(self.steps)
        _, pairs = self.cache.allocator.alloc_batch(self.seq_ids, 1, slots_out=self.slot_stage_np[i])
        self.host_lens += 1
        c = self.cache
        c.apply_copies(pairs)   # a forked row writing into a shared block gets its private copy first
        if fused:
            decode_step(out, q, k_new, v_new, self.slot_stage[i], c.k_pool, c.v_pool, self.tables, self.seq_lens,
                        self.scale, self.max_seq_len, self.partition_size, workspace=self.workspace,
                        **self._load_args(), **c.scales)
        else:
            self.slot_dev.copy_(self.slot_stage[i], non_blocking=True)
            append_slots(self.slot_dev, self.tables, self.seq_lens, c.block_size)
            reshape_and_cache(k_new, v_new, self.slot_dev, c.k_pool, c.v_pool, **c.scales)
            paged_attention_decode(out, q, c.k_pool, c.v_pool, self.tables, self.seq_lens, self.scale,
                                   self.max_seq_len, self.partition_size, workspace=self.workspace,
                                   **self._load_args(), **c.scales)
        if (self.steps + 1) % self.STAGE_EVENT_EVERY == 0:
            ev = torch.cuda.Event()
            ev.record()
            self.step_events[self.steps] = ev
        self.steps += 1

    def refresh(self) -> None:
        """Reloads the device tables and lengths from the allocator (after a row was swapped back in,
        its blocks differ)."""
        tables, lens = self.cache.allocator.fill_block_tables(self.seq_ids, self.stride, pad=0)
        self.tables.copy_(torch.from_numpy(tables))
        self.seq_lens.copy_(torch.from_numpy(lens.copy()))
        self.host_lens = lens.astype(np.int64)
        self.shared_prefix = self._find_shared_prefix()

    def decode_only(self, q: torch.Tensor, out: torch.Tensor) -> None:
        """Attention over the current tokens without appending (no host work, no scatter)."""
        if self.check_tables:
            self._verify_tables()
        c = self.cache
        paged_attention_decode(out, q, c.k_pool, c.v_pool, self.tables, self.seq_lens, self.scale,
                               self.max_seq_len, self.partition_size, workspace=self.workspace,
                               vector=self.vector, **self._load_args(), **c.scales)


class FlatKVCache:
    """Sequences in flat spans of a SpanPool: a sequence takes a free span when it first appends and
    gives it back (unmapped) when freed."""

    def __init__(self, max_seqs: int, max_tokens: int, block_size: int, n_kv_heads: int, head_dim: int, dtype,
                 device="cuda", chunk_bytes: int = 0):
        self.pool = SpanPool(max_seqs, max_tokens, n_kv_heads, head_dim, block_size, dtype, chunk_bytes)
        self.block_size, self.n_kv_heads, self.head_dim, self.dtype = block_size, n_kv_heads, head_dim, dtype
        self.device = device
        self.free_spans = list(range(max_seqs))
        self.span_of = {}
        self.span_len = np.zeros(max_seqs, dtype=np.int64)   # tokens held per span
        self.mapped = np.zeros(max_seqs, dtype=np.int64)     # tokens backed per span, mirrored on the host

    def span(self, seq: int) -> int:
        if seq not in self.span_of:
            if not self.free_spans:
                raise MemoryError("no free span")
            sp = self.free_spans.pop(0)
            self.span_of[seq] = sp
            self.span_len[sp] = 0
        return self.span_of[seq]

    def length(self, seq: int) -> int:
        return int(self.span_len[self.span_of[seq]])

    def ensure(self, span: int, n_tokens: int) -> None:
        """Backs tokens [0, n_tokens) of a span; a host call only when a new chunk is needed."""
        if n_tokens > self.mapped[span]:
            self.pool.reserve(span, n_tokens)
            self.mapped[span] = self.pool.mapped_tokens(span)

    def slots(self, seq: int, n: int):
        sp = self.span(seq)
        L = int(self.span_len[sp])
        self.ensure(sp, L + n)
        return [self.pool.slot(sp, L + i) for i in range(n)]

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor) -> None:
        n = int(k.shape[0])
        sl = self.slots(seq, n)
        self.span_len[self.span_of[seq]] += n
        if n:
            reshape_and_cache_spans(k, v, torch.tensor(sl, dtype=torch.int64, device=self.device), self.pool)

    def free(self, seq: int) -> None:
        sp = self.span_of.pop(seq)
        self.span_len[sp] = 0
        torch.cuda.current_stream().synchronize()   # nothing on the device may still touch the span
        self.pool.release(sp)
        self.mapped[sp] = 0
        self.free_spans.append(sp)


class FlatDecodeBatch:
    def __init__(self, cache: FlatKVCache, seq_ids: Sequence[int], n_q_heads: int, max_seq_len: int,
                 partition_size: int = 512, scale: Optional[float] = None):
        self.cache = cache
        self.seq_ids = [int(x) for x in seq_ids]
        self.S = len(self.seq_ids)
        self.n_q_heads, self.max_seq_len, self.partition_size = n_q_heads, max_seq_len, partition_size
        self.scale = 1.0 / math.sqrt(cache.head_dim) if scale is None else scale
        spans = [cache.span(s) for s in self.seq_ids]
        lens = cache.span_len[spans].astype(np.int32)
        if int(lens.max(initial=0)) > max_seq_len:
            raise ValueError("a sequence is already longer than max_seq_len")
        dev = cache.device
        self.spans = np.array(spans, dtype=np.int64)
        self.span_ids = torch.tensor(spans, dtype=torch.int32, device=dev)
        self.seq_lens = torch.from_numpy(lens).to(dev)
        self.host_lens = lens.astype(np.int64)
        # the append kernel bumps the lengths; the table it also writes is scratch (flat spans have none),
        # wide enough that no row's position falls outside it (the kernel skips such rows entirely)
        self.scratch_table = torch.zeros((self.S, max(1, -(-max_seq_len // cache.block_size))), dtype=torch.int32,
                                         device=dev)
        self.workspace = torch.empty(max(256, workspace_size(self.S, n_q_heads, cache.head_dim, max_seq_len,
                                                               partition_size)), dtype=torch.uint8, device=dev)
        self.slot_stage = [torch.empty(self.S, dtype=torch.int64, pin_memory=True) for _ in range(2)]
        self.slot_stage_np = [t.numpy() for t in self.slot_stage]
        self.stage_done = [None, None]
        self.slot_dev = torch.empty(self.S, dtype=torch.int64, device=dev)
        self.steps = 0

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, out: torch.Tensor) -> None:
        """One decode step for every row: back the new token, write its K/V, attend over all tokens."""
        c = self.cache
        if int(self.host_lens.max(initial=0)) + 1 > self.max_seq_len:
            raise ValueError("decode step would exceed max_seq_len")
        i = self.steps & 1
        if self.stage_done[i] is not None:
            self.stage_done[i].synchronize()
        pos = self.host_lens
        for r in np.nonzero(pos + 1 > c.mapped[self.spans])[0].tolist():
            c.ensure(int(self.spans[r]), int(pos[r]) + 1)     # a token that starts an unmapped chunk
        B, bps = c.block_size, c.pool.blocks_per_span
        self.slot_stage_np[i][:] = (self.spans * bps + pos // B) * B + pos % B
        self.host_lens += 1
        c.span_len[self.spans] = self.host_lens
        self.slot_dev.copy_(self.slot_stage[i], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.stage_done[i] = ev
        append_slots(self.slot_dev, self.scratch_table, self.seq_lens, B)
        reshape_and_cache_spans(k_new, v_new, self.slot_dev, c.pool)
        paged_attention_decode_flat(out, q, c.pool, self.span_ids, self.seq_lens, self.scale, self.max_seq_len,
                                    self.partition_size, workspace=self.workspace)
        self.steps += 1

    def decode_only(self, q: torch.Tensor, out: torch.Tensor) -> None:
        c = self.cache
        paged_attention_decode_flat(out, q, c.pool, self.span_ids, self.seq_lens, self.scale, self.max_seq_len,
                                    self.partition_size, workspace=self.workspace)
