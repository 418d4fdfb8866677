"""O4: decode attention through the block table, in fp64.

Test infrastructure only (see the package docstring).

The pages say what the paged kernel does and leave the arithmetic to the
standard definition: it follows the block table and collects keys and values
from their scattered physical blocks for the score product and the weighted
sum of values ("PagedAttention -- Math + Memory Model", section
"PagedAttention: blocks and the block table"; "KV-cache paging in vLLM", section "The Attention Kernel
Change": the kernel takes the block table as an extra input and gathers
blocks during the attention computation).  So the oracle is that plain
definition, written out:

1. decode the stored (already rounded) q, K, V to fp64 exactly;
2. materialise each sequence's logical K_s, V_s by following its block table
   (``scatter.gather_logical``);
3. for query head h, with G = n_q_heads / n_kv_heads and kv head h // G
   (consecutive grouping):
       x_j = scale * <K_s[j, kv], q[s, h]>     j = 0 .. L_s-1
       m   = max_j x_j
       p_j = exp(x_j - m)
       o[s, h] = sum_j p_j V_s[j, kv] / sum_j p_j
   (subtracting m is the numerically stable form; it changes nothing in
   exact arithmetic);
4. a sequence with L_s = 0 returns zeros.

Readings: the decode token attends to itself (seq_lens count it and the
scatter runs first); scale is a parameter (1/sqrt(head_dim) in every
workload); no partitioning -- the split-context merge is exact in real
arithmetic, so the oracle never splits.  A quantised cache (FP8 E4M3 codes with
per-tensor scales, ``fp8``) is read as the values it represents, and the same
definition applies to them (``paged_attention_decode_fp8``).
"""
from __future__ import annotations

import numpy as np

from . import fp8
from .scatter import gather_logical


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored elements: float32 / float16 widen; bf16 bits are the top half
    of an fp32."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def attention_logical(q_s: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one sequence's query heads over its logical K/V (all fp64).

    q_s: [Hq, D]; K, V: [L, Hk, D]; returns [Hq, D].
    """
    Hq, D = q_s.shape
    L, Hk, _ = K.shape
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    G = Hq // Hk
    for kv in range(Hk):
        heads = slice(kv * G, (kv + 1) * G)
        x = scale * (q_s[heads] @ K[:, kv, :].T)          # [G, L]
        m = x.max(axis=1, keepdims=True)
        p = np.exp(x - m)
        out[heads] = (p @ V[:, kv, :]) / p.sum(axis=1, keepdims=True)
    return out


def paged_attention_decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                           block_tables: np.ndarray, seq_lens: np.ndarray, scale: float,
                           dtype: str, rows=None) -> np.ndarray:
    """Decode attention for every batch row (or the listed ``rows``): [S, Hq, D] fp64.

    q: [S, Hq, D] storage; pools in the layout of ``scatter``; block_tables: [S, max_blocks].
    Rows not listed are left as NaN.
    """
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    for s in (range(S) if rows is None else rows):
        L = int(seq_lens[s])
        K, V = gather_logical(k_pool, v_pool, block_tables[s], L)
        out[s] = attention_logical(to_f64(q[s], dtype), to_f64(K, dtype), to_f64(V, dtype), scale)
    return out


def paged_attention_decode_fp8(q: np.ndarray, q_dtype: str, k_pool: np.ndarray, v_pool: np.ndarray,
                               k_scale: float, v_scale: float, block_tables: np.ndarray,
                               seq_lens: np.ndarray, scale: float, rows=None) -> np.ndarray:
    """Decode attention over a quantised cache: the same attention as ``paged_attention_decode``,
    on the values the cache holds, k_scale * value(code) and v_scale * value(code)
    (``fp8.dequantize``).  q: [S, Hq, D] storage of q_dtype; pools: uint8 E4M3 codes."""
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    for s in (range(S) if rows is None else rows):
        L = int(seq_lens[s])
        K, V = gather_logical(k_pool, v_pool, block_tables[s], L)
        out[s] = attention_logical(to_f64(q[s], q_dtype), fp8.dequantize(K, k_scale),
                                   fp8.dequantize(V, v_scale), scale)
    return out
