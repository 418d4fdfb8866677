"""O1: the byte and utilisation arithmetic the pages state.

Test infrastructure only (see the package docstring).

Each function is the formula as written on the cited page; the tests pin
them to the numbers those pages print.
"""
from __future__ import annotations

import math


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K plus V cached per token over all layers.

    "PagedAttention -- Math + Memory Model", section "The KV cache is big, and
    it grows": two tensors (key and value) per layer, each n_kv_heads x
    head_dim elements of dtype_bytes.
    """
    return 2 * n_layers * n_kv_heads * head_dim * dtype_bytes


def blocks_needed(L: int, B: int) -> int:
    """Blocks a sequence of L tokens occupies: ceil(L / B).

    "PagedAttention -- Math + Memory Model", section "Why fragmentation nearly
    vanishes"; logical block i holds tokens i*B .. (i+1)*B - 1 (section
    "PagedAttention: blocks and the block table").
    """
    if L < 0 or B <= 0:
        raise ValueError("L must be >= 0 and B > 0")
    return -(-L // B)


def slots_paged(L: int, B: int) -> int:
    """KV slots a paged sequence holds: ceil(L/B) * B (same section)."""
    return blocks_needed(L, B) * B


def utilisation_contiguous(L: int, L_max: int) -> float:
    """U_contig = L / L_max for one request that reserved L_max slots.

    "PagedAttention -- Math + Memory Model", section "The fragmentation math".
    """
    return L / L_max


def utilisation_paged(L: int, B: int) -> float:
    """U_paged = L / (ceil(L/B) * B).

    "PagedAttention -- Math + Memory Model", section "Why fragmentation nearly
    vanishes".
    """
    return L / slots_paged(L, B)


def waste_paged(L: int, B: int) -> int:
    """Unused slots of a paged sequence: only the tail of its last block, at most B-1 (same section)."""
    return slots_paged(L, B) - L


def mean_waste_paged(B: int) -> float:
    """Average tail waste the page quotes for uniformly distributed lengths: (B-1)/2 (same section)."""
    return (B - 1) / 2


def idle_slots_contiguous(L: int, L_max: int) -> int:
    """Reserved but unused slots of a contiguous reservation (section "Naive allocation: one
    contiguous slab per request" of "PagedAttention -- Math + Memory Model")."""
    return L_max - L


def requests_that_fit(budget_bytes: float, per_request_bytes: float) -> int:
    """Whole requests a KV budget holds: floor(budget / per-request bytes).

    The worked example of "PagedAttention -- Math + Memory Model" (section "A
    worked example") and the admission count of "Contiguous vs Paged KV Cache
    on RDNA4" (section "The reservation you have to make before the first
    token") both divide a budget by a per-request footprint and keep whole
    requests.
    """
    return int(math.floor(budget_bytes / per_request_bytes))


def wasted_fraction(reserved_bytes: float, live_bytes: float) -> float:
    """Share of reserved KV memory that holds no token: 1 - live / reserved.

    "Contiguous vs Paged KV Cache on RDNA4", section "The same three numbers,
    three ways" (waste column).
    """
    return 1.0 - live_bytes / reserved_bytes
