"""libpagedkv: paged KV cache for decode on MI355X -- Python binding.

Thin wrappers over the C ABI (include/pkv.h) that take torch tensors for
device memory and torch's current stream; every step of the hot path runs in
the HIP kernels of libpagedkv.so.  Nothing here computes on the CPU, and
nothing falls back if the library is missing.

    k_pool, v_pool = torch.empty(key_pool_shape(...)), torch.empty(value_pool_shape(...))
    reshape_and_cache(k, v, slot_mapping, k_pool, v_pool)
    paged_attention_decode(out, q, k_pool, v_pool, block_tables, seq_lens, scale, max_seq_len)

A quantised cache has pools of torch.float8_e4m3fn (or uint8) holding FP8 E4M3 codes, one
per-tensor scale per pool: pass k_scale / v_scale to reshape_and_cache and
paged_attention_decode.

decode_step(out, q, k, v, slot_mapping, k_pool, v_pool, block_tables, seq_lens, ...) is one decode
step (the device append, the scatter and the attention) in fewer launches, with the same results.
"""
from __future__ import annotations

import ctypes as C
from typing import List, Optional, Sequence, Tuple

from . import _lib
from ._lib import (PKV_BF16, PKV_ERR_HIP, PKV_ERR_INVALID, PKV_ERR_NOT_FOUND, PKV_ERR_OOM,  # noqa: F401
                   PKV_ERR_SCRATCH, PKV_ERR_UNSUPPORTED, PKV_F16, PKV_F32, PKV_FP8_E4M3, PKV_OK,
                   PKV_STATIC_SCRATCH_BYTES, KERNEL_NAMES, LibraryNotBuilt)

__all__ = [
    "PKVError", "Allocator", "reshape_and_cache", "append_slots", "paged_attention_decode",
    "workspace_size", "key_pool_shape", "value_pool_shape", "pool_bytes", "dtype_code",
    "timing_enable", "timing_select", "timing_collect", "lib", "copy_blocks", "SpanPool",
    "reshape_and_cache_spans", "paged_attention_decode_flat", "swap_blocks", "decode_step",
    "paged_attention_decode_noalloc", "read_probe", "validate_block_tables", "check_block_tables",
]


def lib():
    return _lib.load()


class PKVError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = lib().pkv_status_string(status).decode()
        super().__init__(f"{what}: {msg} ({status})" if what else f"{msg} ({status})")


class OutOfBlocks(PKVError, MemoryError):
    pass


def _check(status: int, what: str) -> None:
    if status == PKV_OK:
        return
    if status == PKV_ERR_OOM:
        raise OutOfBlocks(status, what)
    raise PKVError(status, what)


def dtype_code(t) -> int:
    """Element type code of a tensor or dtype: float32, float16, bfloat16, and for pools of a
    quantised cache float8_e4m3fn or uint8 (E4M3 codes)."""
    import torch
    dt = t if isinstance(t, torch.dtype) else t.dtype
    return {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
            torch.float8_e4m3fn: PKV_FP8_E4M3, torch.uint8: PKV_FP8_E4M3}[dt]


def _is_fp8_pool(t) -> bool:
    return dtype_code(t) == PKV_FP8_E4M3


def _x(dtype) -> int:
    import torch
    return 16 // torch.empty((), dtype=dtype).element_size()


def key_pool_shape(num_blocks: int, n_kv_heads: int, head_dim: int, block_size: int, dtype) -> Tuple[int, ...]:
    """[num_blocks][n_kv_heads][head_dim / X][block_size][X], X = 16 bytes / element size."""
    x = _x(dtype)
    return (num_blocks, n_kv_heads, head_dim // x, block_size, x)


def value_pool_shape(num_blocks: int, n_kv_heads: int, head_dim: int, block_size: int) -> Tuple[int, ...]:
    """[num_blocks][n_kv_heads][head_dim][block_size]."""
    return (num_blocks, n_kv_heads, head_dim, block_size)


def pool_bytes(num_blocks, n_kv_heads, head_dim, block_size, dtype) -> int:
    return int(lib().pkv_pool_bytes(num_blocks, n_kv_heads, head_dim, block_size, dtype_code(dtype)))


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _pool_dims(k_pool, v_pool):
    if k_pool.dim() != 5 or v_pool.dim() != 4:
        raise ValueError("k_pool must be [N, Hk, D/X, B, X] and v_pool [N, Hk, D, B]")
    N, Hk, Cx, B, X = k_pool.shape
    D = Cx * X
    if tuple(v_pool.shape) != (N, Hk, D, B):
        raise ValueError(f"value pool shape {tuple(v_pool.shape)} does not match key pool {tuple(k_pool.shape)}")
    if not (k_pool.is_contiguous() and v_pool.is_contiguous()) or k_pool.dtype != v_pool.dtype:
        raise ValueError("pools must be contiguous and of one dtype")
    return N, Hk, D, B


def reshape_and_cache(k, v, slot_mapping, k_pool, v_pool, stream=None, k_scale=None, v_scale=None) -> None:
    """Writes k[t], v[t] ([T, Hk, D], token rows may be strided) into slot slot_mapping[t].

    FP8 pools (float8_e4m3fn / uint8) store the E4M3 codes of k / k_scale and v / v_scale
    (both scales required); other pools take rows of their own dtype, copied bit for bit."""
    N, Hk, D, B = _pool_dims(k_pool, v_pool)
    T = k.shape[0]
    if k.shape != (T, Hk, D) or v.shape != (T, Hk, D) or slot_mapping.shape != (T,):
        raise ValueError("k, v must be [T, Hk, D] and slot_mapping [T]")
    for t in (k, v):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError("k/v rows must be contiguous within a token")
    if _is_fp8_pool(k_pool):
        if k_scale is None or v_scale is None:
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        if k.dtype != v.dtype:
            raise ValueError("k and v must have one dtype")
        _check(lib().pkv_reshape_and_cache_fp8(_ptr(k), _ptr(v), _ptr(slot_mapping), T, k.stride(0), v.stride(0),
                                               _ptr(k_pool), _ptr(v_pool), N, Hk, D, B, dtype_code(k),
                                               float(k_scale), float(v_scale), _stream(stream)),
               "pkv_reshape_and_cache_fp8")
        return
    if k_scale is not None or v_scale is not None:
        raise ValueError("scales apply to FP8 pools only")
    _check(lib().pkv_reshape_and_cache(_ptr(k), _ptr(v), _ptr(slot_mapping), T, k.stride(0), v.stride(0),
                                       _ptr(k_pool), _ptr(v_pool), N, Hk, D, B, dtype_code(k_pool),
                                       _stream(stream)), "pkv_reshape_and_cache")


def copy_blocks(pairs, k_pool, v_pool, stream=None) -> None:
    """Copy-on-write: block pairs[i, 1] of both pools becomes a copy of block pairs[i, 0].

    pairs: device int32 [n, 2] (the allocator's (src, dst) pairs)."""
    import torch
    N, Hk, D, B = _pool_dims(k_pool, v_pool)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n, 2] tensor")
    _check(lib().pkv_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(pairs), pairs.shape[0], N, Hk, D, B,
                                 dtype_code(k_pool), _stream(stream)), "pkv_copy_blocks")


def swap_blocks(pairs, src_k, src_v, dst_k, dst_v, stream=None) -> None:
    """Block dst of (dst_k, dst_v) becomes a copy of block src of (src_k, src_v) for each (src, dst)
    in pairs.  Each array is a device pool or pinned host swap space of the pool layout with its own
    block count in dim 0; pairs: int32 [n, 2], device or pinned."""
    import torch
    Ns, Hk, D, B = _pool_dims(src_k, src_v)
    Nd, Hk2, D2, B2 = _pool_dims(dst_k, dst_v)
    if (Hk, D, B) != (Hk2, D2, B2) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination must hold blocks of one shape and dtype")
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n, 2] tensor")
    _check(lib().pkv_swap_blocks(_ptr(src_k), _ptr(src_v), Ns, _ptr(dst_k), _ptr(dst_v), Nd, _ptr(pairs),
                                 pairs.shape[0], Hk, D, B, dtype_code(src_k), _stream(stream)), "pkv_swap_blocks")


def append_slots(slot_mapping, block_tables, seq_lens, block_size: int, stream=None) -> None:
    """Device half of a decode step's append: table[i][seq_lens[i] / B] = slot[i] / B; seq_lens[i] += 1."""
    S = slot_mapping.shape[0]
    _check(lib().pkv_append_slots(_ptr(slot_mapping), S, _ptr(block_tables), block_tables.stride(0),
                                  _ptr(seq_lens), block_size, _stream(stream)), "pkv_append_slots")


def workspace_size(num_seqs, n_q_heads, head_dim, max_seq_len, partition_size=512) -> int:
    return int(lib().pkv_paged_attention_workspace_size(num_seqs, n_q_heads, head_dim, max_seq_len,
                                                          partition_size))


PKV_DECODE_SHARED_KV = 1
PKV_DECODE_VECTOR = 2


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float, max_seq_len: int,
                           partition_size: int = 512, workspace=None, stream=None, shared_kv: bool = False,
                           k_scale=None, v_scale=None, vector: bool = False, shared_prefix_tokens: int = 0) -> None:
    """out[s, h] = softmax attention of q[s, h] over the row's paged K/V (see include/pkv.h).

    shared_kv: some blocks are read by more than one row (forks, a shared prompt); keeps them
    cacheable instead of streaming them.  Results are the same either way.
    shared_prefix_tokens: n > 0 reads tiles before token n of each row cacheable and streams the rest
    (pkv_paged_attention_decode_v2); overrides shared_kv.
    vector: 16-bit KV with one query head per KV head on the per-token vector path instead of MFMA.
    FP8 pools (float8_e4m3fn / uint8): attention over k_scale * value(code) and
    v_scale * value(code), with q in bf16 or f16."""
    import torch
    N, Hk, D, B = _pool_dims(k_pool, v_pool)
    S, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (S, Hq, D) or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [S, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [S, stride] with unit column stride")
    need = workspace_size(S, Hq, D, max_seq_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    flags = (PKV_DECODE_SHARED_KV if shared_kv else 0) | (PKV_DECODE_VECTOR if vector else 0)
    if shared_prefix_tokens:
        fp8 = _is_fp8_pool(k_pool)
        if fp8 and (k_scale is None or v_scale is None):
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        args = _lib.pkv_decode_args(
            out=_ptr(out), out_dtype=dtype_code(out), q=_ptr(q), q_dtype=dtype_code(q), k_pool=_ptr(k_pool),
            v_pool=_ptr(v_pool), kv_fp8=1 if fp8 else 0, k_scale=float(k_scale) if fp8 else 1.0,
            v_scale=float(v_scale) if fp8 else 1.0, block_tables=_ptr(block_tables),
            block_table_stride=block_tables.stride(0), seq_lens=_ptr(seq_lens), num_seqs=S, n_q_heads=Hq,
            n_kv_heads=Hk, head_dim=D, block_size=B, num_blocks=N, scale=float(scale), max_seq_len=int(max_seq_len),
            partition_size=int(partition_size), workspace=_ptr(workspace),
            workspace_bytes=workspace.numel() * workspace.element_size(), flags=flags,
            shared_prefix_tokens=int(shared_prefix_tokens))
        _check(lib().pkv_paged_attention_decode_v2(C.byref(args), _stream(stream)), "pkv_paged_attention_decode_v2")
        return
    if _is_fp8_pool(k_pool):
        if k_scale is None or v_scale is None:
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        _check(lib().pkv_paged_attention_decode_fp8(
            _ptr(out), dtype_code(out), _ptr(q), dtype_code(q), _ptr(k_pool), _ptr(v_pool), float(k_scale),
            float(v_scale), _ptr(block_tables), block_tables.stride(0), _ptr(seq_lens), S, Hq, Hk, D, B, N,
            float(scale), int(max_seq_len), int(partition_size), _ptr(workspace),
            workspace.numel() * workspace.element_size(), flags, _stream(stream)),
            "pkv_paged_attention_decode_fp8")
        return
    if k_scale is not None or v_scale is not None:
        raise ValueError("scales apply to FP8 pools only")
    _check(lib().pkv_paged_attention_decode_ex(
        _ptr(out), dtype_code(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.stride(0), _ptr(seq_lens), S, Hq, Hk, D, B, N, float(scale), int(max_seq_len),
        int(partition_size), _ptr(workspace), workspace.numel() * workspace.element_size(),
        dtype_code(k_pool), flags, _stream(stream)),
        "pkv_paged_attention_decode_ex")


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                                   max_seq_len: int, partition_size: int = 512, stream=None,
                                   shared_kv: bool = False) -> None:
    """paged_attention_decode on 16-bit or fp32 pools with no workspace: the library's static device
    scratch (PKV_STATIC_SCRATCH_BYTES per GPU) holds the plan and the partial results, and the call
    allocates nothing (pkv_paged_attention_decode_noalloc).  Calls in flight at once on one GPU share
    that scratch and must be ordered by the caller."""
    N, Hk, D, B = _pool_dims(k_pool, v_pool)
    S, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (S, Hq, D) or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [S, Hq, D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [S, stride] with unit column stride")
    if _is_fp8_pool(k_pool):
        raise ValueError("FP8 pools take paged_attention_decode with a workspace")
    _check(lib().pkv_paged_attention_decode_noalloc(
        _ptr(out), dtype_code(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.stride(0), _ptr(seq_lens), S, Hq, Hk, D, B, N, float(scale), int(max_seq_len),
        int(partition_size), dtype_code(k_pool), PKV_DECODE_SHARED_KV if shared_kv else 0, _stream(stream)),
        "pkv_paged_attention_decode_noalloc")


def decode_step(out, q, k, v, slot_mapping, k_pool, v_pool, block_tables, seq_lens, scale: float,
                max_seq_len: int, partition_size: int = 512, workspace=None, stream=None, shared_kv: bool = False,
                k_scale=None, v_scale=None, shared_prefix_tokens: int = 0) -> None:
    """One decode step: append_slots, reshape_and_cache and paged_attention_decode with the same
    results, in fewer launches (pkv_decode_step).  Row s appends token s of k / v ([S, Hk, D], token
    rows may be strided) at slot_mapping[s]; slot_mapping is int64 [S] on the device or in pinned
    host memory (read by the kernel in place).  Other arguments as for paged_attention_decode."""
    import torch
    N, Hk, D, B = _pool_dims(k_pool, v_pool)
    S, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != (S, Hq, D) or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [S, Hq, D]")
    if k.shape != (S, Hk, D) or v.shape != (S, Hk, D) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [S, Hk, D] of q's dtype")
    for t in (k, v):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError("k/v rows must be contiguous within a token")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (S,) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 [S] tensor")
    if not slot_mapping.is_cuda and not slot_mapping.is_pinned():
        raise ValueError("a host slot_mapping must be in pinned memory")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be [S, stride] with unit column stride")
    fp8 = _is_fp8_pool(k_pool)
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("an FP8 cache needs k_scale and v_scale")
    if not fp8 and (k_scale is not None or v_scale is not None):
        raise ValueError("scales apply to FP8 pools only")
    if not fp8 and k_pool.dtype != q.dtype:
        raise ValueError("the pools must hold q's dtype (or FP8 codes)")
    need = workspace_size(S, Hq, D, max_seq_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    a = _lib.pkv_decode_step_args(
        k=_ptr(k), v=_ptr(v), k_token_stride=k.stride(0), v_token_stride=v.stride(0),
        slot_mapping=_ptr(slot_mapping), k_pool=_ptr(k_pool), v_pool=_ptr(v_pool), num_blocks=N,
        kv_fp8=1 if fp8 else 0, k_scale=float(k_scale) if fp8 else 1.0, v_scale=float(v_scale) if fp8 else 1.0,
        block_tables=_ptr(block_tables), seq_lens=_ptr(seq_lens), block_table_stride=block_tables.stride(0),
        num_seqs=S, n_q_heads=Hq, n_kv_heads=Hk, head_dim=D, block_size=B, out=_ptr(out),
        out_dtype=dtype_code(out), dtype=dtype_code(q), q=_ptr(q), scale=float(scale), max_seq_len=int(max_seq_len),
        partition_size=int(partition_size), flags=PKV_DECODE_SHARED_KV if shared_kv else 0,
        workspace=_ptr(workspace), workspace_bytes=workspace.numel() * workspace.element_size(),
        shared_prefix_tokens=int(shared_prefix_tokens))
    _check(lib().pkv_decode_step(C.byref(a), _stream(stream)), "pkv_decode_step")


class SpanPool:
    """Flat spans (pkv_span_pool): one contiguous virtual range per sequence, physical memory mapped
    on demand in chunks.  Span s holds blocks s * blocks_per_span .. of a virtual pool in the
    documented layout; token p of span s has slot (s * blocks_per_span + p // B) * B + p % B."""

    def __init__(self, max_spans: int, max_tokens: int, n_kv_heads: int, head_dim: int, block_size: int, dtype,
                 chunk_bytes: int = 0):
        self._h = C.c_void_p()
        _check(lib().pkv_span_pool_create(max_spans, max_tokens, n_kv_heads, head_dim, block_size,
                                          dtype_code(dtype), chunk_bytes, C.byref(self._h)), "pkv_span_pool_create")
        self.max_spans, self.block_size, self.n_kv_heads, self.head_dim = max_spans, block_size, n_kv_heads, head_dim
        self.dtype = dtype
        inf = self.info()
        self.k_base, self.v_base = inf["k_base"], inf["v_base"]
        self.blocks_per_span, self.num_blocks = inf["blocks_per_span"], inf["num_blocks"]
        self.chunk_bytes = inf["chunk_bytes"]

    def info(self) -> dict:
        st = _lib.pkv_span_info()
        _check(lib().pkv_span_pool_info(self._h, C.byref(st)), "pkv_span_pool_info")
        return {name: getattr(st, name) for name, _ in st._fields_}

    def reserve(self, span: int, n_tokens: int) -> None:
        _check(lib().pkv_span_reserve(self._h, span, n_tokens), "pkv_span_reserve")

    def release(self, span: int) -> None:
        _check(lib().pkv_span_release(self._h, span), "pkv_span_release")

    def trim(self) -> None:
        _check(lib().pkv_span_pool_trim(self._h), "pkv_span_pool_trim")

    def mapped_tokens(self, span: int) -> int:
        return int(lib().pkv_span_mapped_tokens(self._h, span))

    def slot(self, span: int, pos: int) -> int:
        B = self.block_size
        return (span * self.blocks_per_span + pos // B) * B + pos % B

    def close(self) -> None:
        if self._h:
            lib().pkv_span_pool_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def reshape_and_cache_spans(k, v, slot_mapping, pool: SpanPool, stream=None) -> None:
    """pkv_reshape_and_cache into a span pool's virtual pools (the slots must be reserved)."""
    T = k.shape[0]
    Hk, D = pool.n_kv_heads, pool.head_dim
    if k.shape != (T, Hk, D) or v.shape != (T, Hk, D) or slot_mapping.shape != (T,):
        raise ValueError("k, v must be [T, Hk, D] and slot_mapping [T]")
    if dtype_code(k) != dtype_code(pool.dtype):
        raise ValueError("rows must have the pool's dtype")
    for t in (k, v):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError("k/v rows must be contiguous within a token")
    _check(lib().pkv_reshape_and_cache(_ptr(k), _ptr(v), _ptr(slot_mapping), T, k.stride(0), v.stride(0),
                                       pool.k_base, pool.v_base, pool.num_blocks, Hk, D, pool.block_size,
                                       dtype_code(pool.dtype), _stream(stream)), "pkv_reshape_and_cache")


def paged_attention_decode_flat(out, q, pool: SpanPool, span_ids, seq_lens, scale: float, max_seq_len: int,
                                partition_size: int = 512, workspace=None, stream=None) -> None:
    """Decode attention over flat spans (no block table): row s reads span span_ids[s]."""
    import torch
    S, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != (S, Hq, D) or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous [S, Hq, D] with the pool's head_dim")
    if span_ids.dtype != torch.int32 or span_ids.shape != (S,):
        raise ValueError("span_ids must be int32 [S]")
    need = workspace_size(S, Hq, D, max_seq_len, partition_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().pkv_paged_attention_decode_flat(
        _ptr(out), dtype_code(out), _ptr(q), pool.k_base, pool.v_base, _ptr(span_ids), pool.blocks_per_span,
        _ptr(seq_lens), S, Hq, pool.n_kv_heads, D, pool.block_size, pool.num_blocks, float(scale),
        int(max_seq_len), int(partition_size), _ptr(workspace), workspace.numel() * workspace.element_size(),
        dtype_code(q), 0, _stream(stream)), "pkv_paged_attention_decode_flat")


def timing_enable(on: bool = True) -> None:
    _check(lib().pkv_timing_enable(1 if on else 0), "pkv_timing_enable")


def timing_select(names=None) -> None:
    """Time only the named kernels (KERNEL_NAMES values); None restores all."""
    if names is None:
        mask = 0xFFFFFFFF
    else:
        ids = {v: k for k, v in KERNEL_NAMES.items()}
        mask = 0
        for nm in names:
            mask |= 1 << ids[nm]
    _check(lib().pkv_timing_select(mask), "pkv_timing_select")


def timing_collect() -> dict:
    """{kernel name: (launches, total ms)} for launches since the last collect (waits for them)."""
    recs = (_lib.pkv_kernel_time * 8)()
    n = C.c_int32(0)
    _check(lib().pkv_timing_collect(recs, 8, C.byref(n)), "pkv_timing_collect")
    return {KERNEL_NAMES[recs[i].kernel]: (recs[i].launches, recs[i].total_ms) for i in range(n.value)}


class Allocator:
    """Host block allocator (pkv_allocator): FIFO free list, ref counts, fork, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order: Optional[Sequence[int]] = None):
        self._h = C.c_void_p()
        order = None
        if initial_free_order is not None:
            order = (C.c_int32 * num_blocks)(*[int(b) for b in initial_free_order])
        _check(lib().pkv_allocator_create(num_blocks, block_size, order, C.byref(self._h)),
               "pkv_allocator_create")
        self.num_blocks, self.block_size = num_blocks, block_size

    def close(self) -> None:
        if self._h:
            lib().pkv_allocator_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots = (C.c_int64 * max(n, 1))()
        pair = (C.c_int32 * 2)()
        ncow = C.c_int32(0)
        _check(lib().pkv_alloc(self._h, seq, n, slots, pair, C.byref(ncow)), "pkv_alloc")
        return list(slots[:n]), ([(pair[0], pair[1])] if ncow.value else [])

    def alloc_batch(self, seqs: Sequence[int], n_each: int, slots_out=None):
        """Appends n_each tokens to every sequence; slots_out: optional int64 numpy array [S*n_each]."""
        import numpy as np
        S = len(seqs)
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        if slots_out is None:
            slots_out = np.empty(S * n_each, dtype=np.int64)
        pairs = np.empty(2 * max(S, 1), dtype=np.int32)
        ncow = C.c_int32(0)
        _check(lib().pkv_alloc_batch(self._h, ids.ctypes.data_as(_lib.PI64), S, n_each,
                                     slots_out.ctypes.data_as(_lib.PI64), pairs.ctypes.data_as(_lib.PI32),
                                     C.byref(ncow)), "pkv_alloc_batch")
        return slots_out, [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(ncow.value)]

    def fork(self, parent: int, child: int, n: int = -1) -> None:
        _check(lib().pkv_fork(self._h, parent, child, n), "pkv_fork")

    def free(self, seq: int) -> None:
        _check(lib().pkv_free(self._h, seq), "pkv_free")

    def block_table(self, seq: int) -> List[int]:
        nb, L = C.c_int32(0), C.c_int32(0)
        _check(lib().pkv_get_block_table(self._h, seq, None, 0, C.byref(nb), C.byref(L)), "pkv_get_block_table")
        buf = (C.c_int32 * max(nb.value, 1))()
        _check(lib().pkv_get_block_table(self._h, seq, buf, nb.value, None, None), "pkv_get_block_table")
        return list(buf[:nb.value])

    def seq_len(self, seq: int) -> int:
        nb, L = C.c_int32(0), C.c_int32(0)
        _check(lib().pkv_get_block_table(self._h, seq, None, 0, C.byref(nb), C.byref(L)), "pkv_get_block_table")
        return L.value

    def fill_block_tables(self, seqs: Sequence[int], stride: int, pad: int = 0):
        """(tables int32 [S, stride], seq_lens int32 [S]) as numpy arrays."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        tables = np.empty((len(seqs), stride), dtype=np.int32)
        lens = np.empty(len(seqs), dtype=np.int32)
        _check(lib().pkv_fill_block_tables(self._h, ids.ctypes.data_as(_lib.PI64), len(seqs),
                                           tables.ctypes.data_as(_lib.PI32), stride, pad,
                                           lens.ctypes.data_as(_lib.PI32)), "pkv_fill_block_tables")
        return tables, lens

    def stats(self) -> dict:
        st = _lib.pkv_stats()
        _check(lib().pkv_allocator_stats(self._h, C.byref(st)), "pkv_allocator_stats")
        return {name: getattr(st, name) for name, _ in st._fields_ if name != "reserved"}

    def set_swap_space(self, host_blocks: int) -> None:
        _check(lib().pkv_allocator_set_swap_space(self._h, host_blocks), "pkv_allocator_set_swap_space")

    def _swap(self, fn, seq: int, what: str):
        n = C.c_int32(0)
        st = fn(self._h, seq, None, 0, C.byref(n))   # a query: reports the block count, changes nothing
        if st == PKV_ERR_NOT_FOUND:
            _check(st, what)
        buf = (C.c_int32 * max(2 * n.value, 2))()
        _check(fn(self._h, seq, buf, n.value, C.byref(n)), what)
        return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]

    def swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """Moves seq to host slots; returns the (device block, host slot) copy pairs."""
        return self._swap(lib().pkv_swap_out, seq, "pkv_swap_out")

    def swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """Brings seq back into fresh device blocks; returns the (host slot, device block) copy pairs."""
        return self._swap(lib().pkv_swap_in, seq, "pkv_swap_in")

    def swap_stats(self) -> dict:
        hb, hf, ns = C.c_int32(0), C.c_int32(0), C.c_int64(0)
        _check(lib().pkv_swap_stats(self._h, C.byref(hb), C.byref(hf), C.byref(ns)), "pkv_swap_stats")
        return {"host_blocks": hb.value, "host_free": hf.value, "swapped_seqs": ns.value}

    def ref_count(self, block: int) -> int:
        return int(lib().pkv_block_ref_count(self._h, block))

    def free_list(self) -> List[int]:
        n = C.c_int32(0)
        _check(lib().pkv_free_list(self._h, None, 0, C.byref(n)), "pkv_free_list")
        buf = (C.c_int32 * max(n.value, 1))()
        _check(lib().pkv_free_list(self._h, buf, n.value, None), "pkv_free_list")
        return list(buf[:n.value])


def read_probe(buf, waves_per_cu: int, loads_per_batch: int, nontemporal: bool = True, random_chunks: bool = False,
               sink=None, stream=None) -> int:
    """Launches the streaming-read probe over the device tensor buf (pkv_read_probe); returns the bytes
    the launch reads.  sink: a device uint32 tensor of at least 1024 elements (allocated if None)."""
    import torch
    if sink is None:
        sink = torch.zeros(1024, dtype=torch.int32, device=buf.device)
    n = C.c_size_t(0)
    mode = (1 if nontemporal else 0) | (2 if random_chunks else 0)
    _check(lib().pkv_read_probe(_ptr(buf), buf.numel() * buf.element_size(), int(waves_per_cu),
                                int(loads_per_batch), mode, _ptr(sink), C.byref(n), _stream(stream)),
           "pkv_read_probe")
    return int(n.value)


def validate_block_tables(tables, seq_lens, block_size: int, num_blocks: int, max_seq_len: int):
    """Host check of the entries decode would read (pkv_validate_block_tables): returns (number of
    out-of-pool entries, first row holding one or -1).  tables: int32 [S, stride], seq_lens: int32 [S]
    (numpy arrays or CPU tensors)."""
    import numpy as np
    t = np.ascontiguousarray(np.asarray(tables, dtype=np.int32))
    L = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if t.ndim != 2 or L.shape != (t.shape[0],):
        raise ValueError("tables must be [S, stride] and seq_lens [S]")
    bad, first = C.c_int64(0), C.c_int32(-1)
    st = lib().pkv_validate_block_tables(t.ctypes.data_as(C.POINTER(C.c_int32)), t.shape[1],
                                         L.ctypes.data_as(C.POINTER(C.c_int32)), t.shape[0], int(block_size),
                                         int(num_blocks), int(max_seq_len), C.byref(bad), C.byref(first))
    if st not in (PKV_OK, PKV_ERR_INVALID):
        _check(st, "pkv_validate_block_tables")
    if st == PKV_ERR_INVALID and bad.value == 0:
        raise PKVError(st, "pkv_validate_block_tables")
    return int(bad.value), int(first.value)


def check_block_tables(tables, seq_lens, block_size: int, num_blocks: int, max_seq_len: int, result=None,
                       stream=None):
    """Device check of the entries decode would read (pkv_check_block_tables), queued on the stream:
    returns the device int32 [2] tensor {out-of-pool entries, first row holding one (INT32_MAX if
    none)}; read it after the stream has run the check."""
    import torch
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=tables.device)
    if tables.dim() != 2 or tables.stride(1) != 1 or tuple(seq_lens.shape) != (tables.shape[0],):
        raise ValueError("tables must be [S, stride] with unit column stride and seq_lens [S]")
    _check(lib().pkv_check_block_tables(_ptr(tables), tables.stride(0), _ptr(seq_lens), tables.shape[0],
                                        int(block_size), int(num_blocks), int(max_seq_len), _ptr(result),
                                        _stream(stream)), "pkv_check_block_tables")
    return result
