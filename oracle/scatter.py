"""O3: writing token K/V rows into physical slots, and reading a sequence back.

Test infrastructure only (see the package docstring).

A physical block holds the keys and values of B consecutive tokens of one
sequence for every KV head ("PagedAttention -- Math + Memory Model", section
"PagedAttention: blocks and the block table"; "KV-cache paging in vLLM",
section "PagedAttention: Paging for KV-Caches").  The element order inside a
block is the library's documented storage layout, restated here from its
definition (x = 16 bytes / element size, so a 16-byte chunk of a key row is
x elements):

    key   pool  [num_blocks][n_kv_heads][head_dim / x][B][x]
          element (blk, h, c, off, e) = key of token (blk, off), head h, dim c*x + e
    value pool  [num_blocks][n_kv_heads][head_dim][B]
          element (blk, h, d, off)    = value of token (blk, off), head h, dim d

Slot s names token position s % B of physical block s // B.  Everything
here moves raw bits (uint8 / uint16 / uint32 / float32 arrays are copied, never
converted), so -0.0 and NaN payloads survive.  A quantised cache stores one-byte
FP8 E4M3 codes (x = 16) that ``reshape_and_cache_fp8`` computes from the new
rows before the same bit copy.
"""
from __future__ import annotations

import numpy as np

from . import fp8


def chunk_elems(esize: int) -> int:
    return 16 // esize


def empty_pools(num_blocks: int, n_kv_heads: int, head_dim: int, block_size: int,
                storage_dtype, fill_bits: int):
    """Key and value pools filled with one bit pattern (a NaN poison in parity runs)."""
    esize = np.dtype(storage_dtype).itemsize
    x = chunk_elems(esize)
    k = np.empty((num_blocks, n_kv_heads, head_dim // x, block_size, x), dtype=storage_dtype)
    v = np.empty((num_blocks, n_kv_heads, head_dim, block_size), dtype=storage_dtype)
    ui = {1: np.uint8, 2: np.uint16, 4: np.uint32}[esize]
    k.view(ui)[...] = fill_bits
    v.view(ui)[...] = fill_bits
    return k, v


def reshape_and_cache(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                      k_pool: np.ndarray, v_pool: np.ndarray) -> None:
    """pool[slot // B, :, slot % B, :] = row[t] for every token t whose slot is in range.

    Negative slots (padding tokens) and slots past the pool are skipped.
    k, v: [T, Hk, D] in the pool's storage dtype.
    """
    N, Hk, C, B, x = k_pool.shape
    T = k.shape[0]
    assert k.shape == (T, Hk, C * x) and v.shape == (T, Hk, C * x)
    # bits, not values: rows and pools must hold the same element type
    assert k.dtype == k_pool.dtype and v.dtype == v_pool.dtype
    for t in range(T):
        s = int(slot_mapping[t])
        if s < 0 or s >= N * B:
            continue
        blk, off = divmod(s, B)
        k_pool[blk, :, :, off, :] = k[t].reshape(Hk, C, x)
        v_pool[blk, :, :, off] = v[t]


def reshape_and_cache_fp8(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                          k_pool: np.ndarray, v_pool: np.ndarray, k_scale: float, v_scale: float) -> None:
    """The scatter into a quantised cache: every element of the new rows is stored as its E4M3
    code under the pool's per-tensor scale (``fp8.quantize``), then placed like any other row.
    k, v: [T, Hk, D] float32 (the exact values of the source rows); pools: uint8 codes."""
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    reshape_and_cache(fp8.quantize(k, k_scale), fp8.quantize(v, v_scale), slot_mapping, k_pool, v_pool)


def gather_logical(k_pool: np.ndarray, v_pool: np.ndarray, table, L: int):
    """A sequence's logical K and V, [L, Hk, D] each: position i is token i % B of block
    table[i // B] ("PagedAttention -- Math + Memory Model", section "PagedAttention: blocks and
    the block table").  Table entries past ceil(L/B) are never read."""
    N, Hk, C, B, x = k_pool.shape
    D = C * x
    nb = -(-L // B)
    ids = np.asarray(table[:nb], dtype=np.int64)
    if nb and (ids.min() < 0 or ids.max() >= N):
        raise IndexError("block table entry outside the pool")
    kb = k_pool[ids]                       # [nb, Hk, C, B, x]
    vb = v_pool[ids]                       # [nb, Hk, D, B]
    K = kb.transpose(0, 3, 1, 2, 4).reshape(nb * B, Hk, D)[:L]
    V = vb.transpose(0, 3, 1, 2).reshape(nb * B, Hk, D)[:L]
    return np.ascontiguousarray(K), np.ascontiguousarray(V)


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, pairs) -> None:
    """Copy-on-write: for each (src, dst) pair, block dst of both pools becomes a bit copy of
    block src, every KV head ("PagedAttention -- Math + Memory Model", section "Copy-on-write:
    sharing blocks across samples": a sequence about to write into a block it shares gets a
    private copy of it, and the write lands in the copy).  Pairs are applied in order; ids
    outside the pool are skipped."""
    N = k_pool.shape[0]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not (0 <= src < N and 0 <= dst < N):
            continue
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


def flat_span_table(span: int, blocks_per_span: int, L: int, B: int):
    """The blocks a flat span gives a sequence of L tokens: logical block i is block
    span * blocks_per_span + i of one virtual pool ("Contiguous vs Paged KV Cache on RDNA4", sections
    "Is paging the only way to fix KV cache fragmentation?" and "Why the single-user verdict flipped": a
    sequence gets one contiguous virtual range reserved up front and physical memory committed into it on
    demand, so reading it needs no block table).  Cut into blocks of the pools' layout, that range is the
    consecutive blocks of the sequence's span; token p then sits at slot
    (span * blocks_per_span + p // B) * B + p % B."""
    nb = -(-L // B)
    if nb > blocks_per_span:
        raise ValueError("sequence longer than its span")
    return [span * blocks_per_span + i for i in range(nb)]


def move_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray, pairs) -> None:
    """Block copies between two block arrays of the pools' layout (a device pool and host swap
    space): for each (src, dst) pair, block dst of dst_k / dst_v becomes a bit copy of block src
    of src_k / src_v ("Reserve for the worst case, or page", section "What this model leaves out":
    a preempted sequence's blocks go to host memory and come back).  Pairs with an id outside
    either array are skipped."""
    ns, nd = src_k.shape[0], dst_k.shape[0]
    for s, d in pairs:
        s, d = int(s), int(d)
        if not (0 <= s < ns and 0 <= d < nd):
            continue
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]
