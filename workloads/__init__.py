"""Seeded synthetic workloads for the paged KV cache.

This module holds data only: the five workload shapes, their sequence
lengths, the order in which the physical pool hands out blocks, the
allocator operation script that builds each batch, and the q/K/V values.
Nothing here allocates blocks, scatters rows or computes attention; the
oracle and the HIP path each do that with their own code, and this module
is the one thing they share.

Values are "N(0,1) rounded to the storage dtype", drawn from a counter-based
generator so that any row of any sequence can be produced on its own, on
the CPU or on the GPU, with identical bits:

* a 32-bit key per (seed, tensor kind, source) from the lowbias32 integer
  hash (Chris Wellons, "Prospecting for Hash Functions", 2018:
  x ^= x>>16; x *= 0x7feb352d; x ^= x>>15; x *= 0x846ca68b; x ^= x>>16);
* element e of a source hashes (key + e * 0x9E3779B1) mod 2^32 with the same
  function; the top 16 bits index a 65,536-entry table of standard-normal
  quantiles Phi^-1((i + 0.5) / 65536) (scipy.special.ndtri in fp64, rounded
  to fp32 and then round-to-nearest-even to the storage dtype).

On a GPU the integer arithmetic runs in int64 torch operations that stay below
2^49, so every device computes the same bits; on the host the same values come
from wrapping uint32 numpy arithmetic on a thread pool, which is checked
against the int64 form.  Sequence lengths and block placement permutations come
from numpy.random.default_rng seeded with [seed, stream].
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "build", "quantised", "CONFIG_NAMES", "DTYPE_BYTES", "kv_rows", "q_values",
    "logical_kv", "storage_to_numpy", "normal_table", "poison_value",
]

CONFIG_NAMES = {
    1: "tiny",
    2: "opt13b_mha",
    3: "llama70b_gqa",
    4: "swarm_shared_prefix",
    5: "long_context",
}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

_M32 = 0xFFFFFFFF
_GOLDEN = 0x9E3779B1
_KIND_Q, _KIND_K, _KIND_V = 1, 2, 3
PREFIX_SOURCE = 1 << 20  # value source id of config 4's shared prompt


# ----------------------------------------------------------------------------
# workload description
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """One decode batch: the prompt-building allocator script plus one decode token per sequence.

    ``prompt_ops`` entries are dicts:
      {"op": "alloc", "seq": id, "n": n, "pos": p}  append n tokens; their values
                                                    are logical positions p..p+n-1
      {"op": "fork", "parent": id, "child": id, "n": n}
      {"op": "free", "seq": id}
    After the script, every sequence in ``batch`` appends one more token (the
    decode step's new token, logical position seq_lens[i]-1), whose K/V the
    scatter writes before attention reads all seq_lens[i] tokens.
    """
    name: str
    config_id: int
    seed: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    num_blocks: int
    free_order: np.ndarray          # int32 [num_blocks], the pool's initial free-list order
    prompt_ops: List[dict]
    batch: np.ndarray               # int64 [S] sequence ids, row order of the decode batch
    seq_lens: np.ndarray            # int32 [S] lengths including the decode token
    segments: Dict[int, List[Tuple[int, int, int]]]  # seq -> [(source, src_start, n)] covering 0..L-1
    partition_size: int = 512
    placement: str = "random"
    variant: str = "full"
    kv_format: str = "native"       # "native": pools of ``dtype``; "fp8": E4M3 codes of the rows
    k_scale: float = 1.0            # per-tensor scales of an "fp8" cache (code of x / scale)
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.batch.shape[0])

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def esize(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def kv_esize(self) -> int:
        """Bytes of one cached element (1 for an FP8 cache)."""
        return 1 if self.kv_format == "fp8" else self.esize

    def describe(self) -> dict:
        return {
            "workload": self.name, "variant": self.variant, "seqs": self.num_seqs,
            "n_q_heads": self.n_q_heads, "n_kv_heads": self.n_kv_heads,
            "head_dim": self.head_dim, "block_size": self.block_size, "dtype": self.dtype,
            "num_blocks": self.num_blocks, "placement": self.placement,
            "partition_size": self.partition_size, "seed": self.seed, "kv_format": self.kv_format,
            **({"k_scale": self.k_scale, "v_scale": self.v_scale} if self.kv_format == "fp8" else {}),
            "total_tokens": int(self.seq_lens.sum()), "max_seq_len": self.max_seq_len,
        }


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _pool_size(block_counts, slack: float) -> int:
    return int(math.ceil(slack * int(sum(block_counts))))


def _free_order(rng: np.random.Generator, n: int, placement: str) -> np.ndarray:
    if placement == "identity":
        return np.arange(n, dtype=np.int32)
    if placement == "random":
        return rng.permutation(n).astype(np.int32)
    raise ValueError(f"unknown placement {placement!r}")


def _independent(cid, name, seed, hq, hk, d, bsz, dtype, lens, free_order, n_blocks,
                 placement, variant, partition_size=512) -> Workload:
    """Each sequence is its own prompt of L-1 tokens followed by one decode token."""
    lens = np.asarray(lens, dtype=np.int32)
    ops, segs = [], {}
    for i, L in enumerate(lens.tolist()):
        if L - 1 > 0:
            ops.append({"op": "alloc", "seq": i, "n": L - 1, "pos": 0})
        segs[i] = [(i, 0, L)]
    return Workload(name=name, config_id=cid, seed=seed, n_q_heads=hq, n_kv_heads=hk,
                    head_dim=d, block_size=bsz, dtype=dtype, num_blocks=n_blocks,
                    free_order=free_order, prompt_ops=ops,
                    batch=np.arange(len(lens), dtype=np.int64), seq_lens=lens,
                    segments=segs, partition_size=partition_size, placement=placement,
                    variant=variant)


def build(config_id: int, *, small: bool = False, block_size: Optional[int] = None,
          placement: str = "random", copied_prefix: bool = False,
          partition_size: Optional[int] = None, seed: Optional[int] = None) -> Workload:
    """The seeded workload for config 1..5 (seed = config_id - 1 unless given: another seed draws
    another instance of the same distributions, for checks that a choice holds beyond one draw).

    ``small`` keeps the config's heads, head_dim, dtype, block size and length
    distribution shape but fewer/shorter sequences, so the fp64 oracle runs
    in seconds while still spanning several tiles, partitions and a ragged tail.
    """
    seed = config_id - 1 if seed is None else int(seed)
    rng_len = np.random.default_rng([seed, 0])
    rng_place = np.random.default_rng([seed, 1])
    variant = "small" if small else "full"
    name = CONFIG_NAMES[config_id]

    if config_id == 1:
        # 4 sequences {1,17,33,100}, 4 q = 4 kv heads, D=64, fp32, B=16, 64-block pool.
        bsz = block_size or 16
        return _independent(1, name, seed, 4, 4, 64, bsz, "f32", [1, 17, 33, 100],
                            _free_order(rng_place, 64, placement), 64, placement, variant,
                            partition_size or 512)

    if config_id == 2:
        # OPT-13B-class layer: 40 MHA heads x 128, fp16, B=16, lengths U[128, 2048], 8192 blocks.
        bsz = block_size or 16
        if small:
            lens = rng_len.integers(1, 700, size=8, endpoint=True)
            n_blocks = 512
        else:
            lens = rng_len.integers(128, 2048, size=32, endpoint=True)
            n_blocks = 8192
        return _independent(2, name, seed, 40, 40, 128, bsz, "f16", lens,
                            _free_order(rng_place, n_blocks, placement), n_blocks,
                            placement, variant, partition_size or 512)

    if config_id == 3:
        # Llama-3-70B-class layer: 64 q / 8 kv heads, D=128, bf16, B=16, 256 sequences with
        # log-normal lengths (median 3000, sigma 1.0) clipped to [16, 32768], pool = need + 10 %.
        bsz = block_size or 16
        if small:
            raw = rng_len.lognormal(mean=math.log(300.0), sigma=1.0, size=8)
            lens = np.clip(np.rint(raw), 16, 1500).astype(np.int32)
        else:
            raw = rng_len.lognormal(mean=math.log(3000.0), sigma=1.0, size=256)
            lens = np.clip(np.rint(raw), 16, 32768).astype(np.int32)
        n_blocks = _pool_size([_ceil_div(int(L), bsz) for L in lens], 1.1)
        # 3072-token partitions (a launch choice, not part of the workload): each partition ends in
        # a store of its partial result and rows of several partitions need the merge.  On MI355X,
        # 512, 1024 and 2048 took 1019, 862 and 795 us per decode; over four draws of this length
        # mix (seeds 2, 7, 11, 23), a call took on average 0.791 / 0.776 / 0.779 / 0.785 ms at
        # 2048 / 3072 / 3584 / 4096 with bf16 KV and 0.457 / 0.453 / 0.448 / 0.456 ms with FP8 KV.
        return _independent(3, name, seed, 64, 8, 128, bsz, "bf16", lens,
                            _free_order(rng_place, n_blocks, placement), n_blocks,
                            placement, variant, 3072 if partition_size is None else partition_size)

    if config_id == 4:
        # Agent swarm: 20 sequences share one 4000-token prompt (250 blocks), then private
        # suffixes U[0, 12000]; 32 q / 8 kv heads, fp16, B=16.  768-token partitions (a launch
        # choice): over two draws (seeds 3 and 9) a decode call took 0.140 / 0.134 / 0.148 ms and
        # 0.183 / 0.177 / 0.174 ms at 512 / 768 / 1024 on MI355X.
        bsz = block_size or 16
        if small:
            n_children, prefix, suffixes = 5, 400, rng_len.integers(0, 600, size=5, endpoint=True)
        else:
            n_children, prefix, suffixes = 20, 4000, rng_len.integers(0, 12000, size=20, endpoint=True)
        lens = (prefix + suffixes + 1).astype(np.int32)
        parent = n_children  # sequence id of the prompt owner; children are 0..n-1
        segs = {i: [(PREFIX_SOURCE, 0, prefix), (i, 0, int(L) - prefix)] for i, L in enumerate(lens)}
        ops: List[dict] = []
        if copied_prefix:
            need = [_ceil_div(int(L), bsz) for L in lens]
            for i, L in enumerate(lens.tolist()):
                ops.append({"op": "alloc", "seq": i, "n": L - 1, "pos": 0})
        else:
            need = [_ceil_div(prefix, bsz)] + [_ceil_div(int(L), bsz) - prefix // bsz for L in lens]
            ops.append({"op": "alloc", "seq": parent, "n": prefix, "pos": 0})
            for i in range(n_children):
                ops.append({"op": "fork", "parent": parent, "child": i, "n": prefix})
            ops.append({"op": "free", "seq": parent})
            for i, L in enumerate(lens.tolist()):
                if L - 1 - prefix > 0:
                    ops.append({"op": "alloc", "seq": i, "n": L - 1 - prefix, "pos": prefix})
        segs[parent] = [(PREFIX_SOURCE, 0, prefix)]
        n_blocks = _pool_size(need, 1.1)
        return Workload(name=name, config_id=4, seed=seed, n_q_heads=32, n_kv_heads=8,
                        head_dim=128, block_size=bsz, dtype="f16", num_blocks=n_blocks,
                        free_order=_free_order(rng_place, n_blocks, placement),
                        prompt_ops=ops, batch=np.arange(n_children, dtype=np.int64),
                        seq_lens=lens, segments=segs, partition_size=partition_size or 768,
                        placement=placement,
                        variant=variant + ("-copied" if copied_prefix else "-shared"))

    if config_id == 5:
        # Long context: 8 x 65536 tokens, 64 q / 8 kv heads, bf16, B in {8, 16, 32}; 2048-token
        # partitions (one work unit per wave of the persistent grid; 512 measured 10 % slower).
        bsz = block_size or 16
        n_seqs, L = (2, 2048) if small else (8, 65536)
        lens = np.full(n_seqs, L, dtype=np.int32)
        n_blocks = _pool_size([_ceil_div(L, bsz)] * n_seqs, 1.1)
        return _independent(5, name, seed, 64, 8, 128, bsz, "bf16", lens,
                            _free_order(rng_place, n_blocks, placement), n_blocks,
                            placement, variant, partition_size or 2048)

    raise ValueError(f"unknown config {config_id}")


# Scales of the quantised variants: the rows are N(0, 1) draws whose largest magnitude is 4.32
# (the table's extreme quantile), so x / 0.01 stays below the format's 448 and no element
# saturates (tests that need saturation pick smaller scales); the two pools get different scales.
FP8_K_SCALE, FP8_V_SCALE = 0.01, 0.0125


def quantised(w: Workload, k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE) -> Workload:
    """The same workload with an FP8 E4M3 cache: rows of ``w.dtype`` (which q and the results
    keep) are stored as the codes of x / k_scale and x / v_scale."""
    return dataclasses.replace(w, kv_format="fp8", k_scale=float(k_scale), v_scale=float(v_scale),
                               variant=w.variant + "-fp8")


def custom(*, seed: int, lens, n_q_heads: int, n_kv_heads: int, head_dim: int,
           block_size: int, dtype: str, num_blocks: Optional[int] = None,
           placement: str = "random", partition_size: int = 512, name: str = "custom") -> Workload:
    """An ad-hoc independent-sequence workload (edge cases, sweeps of shapes)."""
    lens = np.asarray(lens, dtype=np.int32)
    if num_blocks is None:
        num_blocks = max(1, _pool_size([_ceil_div(int(L), block_size) for L in lens], 1.1))
    rng_place = np.random.default_rng([seed, 1])
    return _independent(0, name, seed, n_q_heads, n_kv_heads, head_dim, block_size, dtype,
                        lens, _free_order(rng_place, num_blocks, placement), num_blocks,
                        placement, "custom", partition_size)


# ----------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------
_TABLES: Dict[str, np.ndarray] = {}


def _round_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    u = x32.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def normal_table(dtype: str) -> np.ndarray:
    """65,536 standard-normal quantiles in storage form (float32 / float16 / uint16 bf16 bits)."""
    if dtype not in _TABLES:
        from scipy.special import ndtri
        z = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
        if dtype == "f32":
            t = z
        elif dtype == "f16":
            t = z.astype(np.float16)
        elif dtype == "bf16":
            t = _round_f32_to_bf16_bits(z)
        else:
            raise ValueError(dtype)
        _TABLES[dtype] = t
    return _TABLES[dtype]


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def _mul32(x, c: int):
    """(x * c) mod 2^32 for int64 tensors x in [0, 2^32), without leaving 49 bits."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _hash32(x):
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _hash32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _key(seed: int, kind: int, source: int) -> int:
    k = _hash32_int(seed ^ 0x5EED5EED)
    k = _hash32_int(k ^ kind)
    return _hash32_int(k ^ (source & _M32))


_CHUNK = 1 << 25
_CPU_CHUNK = 1 << 18


def _hash32_u32(x: np.ndarray) -> np.ndarray:
    """lowbias32 on a uint32 array in place (numpy's uint32 products wrap mod 2^32)."""
    x ^= x >> np.uint32(16)
    x *= np.uint32(0x7FEB352D)
    x ^= x >> np.uint32(15)
    x *= np.uint32(0x846CA68B)
    x ^= x >> np.uint32(16)
    return x


def _draw_cpu(key: int, start: int, count: int, dtype: str) -> np.ndarray:
    """``_draw`` on the host in storage form: the same elements from uint32 arithmetic, in
    cache-sized chunks on a thread pool (numpy releases the GIL inside each operation)."""
    from concurrent.futures import ThreadPoolExecutor
    table = normal_table(dtype)
    out = np.empty(count, dtype=table.dtype)

    def fill(c0: int) -> None:
        n = min(_CPU_CHUNK, count - c0)
        e = np.arange(start + c0, start + c0 + n, dtype=np.uint64).astype(np.uint32)   # e mod 2^32
        e *= np.uint32(_GOLDEN)
        e += np.uint32(key)
        out[c0:c0 + n] = table[_hash32_u32(e) >> np.uint32(16)]

    starts = range(0, count, _CPU_CHUNK)
    if count <= 4 * _CPU_CHUNK:
        for c0 in starts:
            fill(c0)
    else:
        with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
            list(ex.map(fill, starts))
    return out


def _draw(key: int, start: int, count: int, dtype: str, device):
    """Elements start..start+count-1 of the stream with this key, as a flat torch tensor."""
    import torch
    if str(device) == "cpu":
        host = _draw_cpu(key, start, count, dtype)
        t = torch.from_numpy(host.view(np.int16) if dtype == "bf16" else host)
        return t.view(torch.bfloat16) if dtype == "bf16" else t
    return _draw_torch(key, start, count, dtype, device)


def _draw_torch(key: int, start: int, count: int, dtype: str, device):
    """``_draw`` in int64 torch arithmetic on any device (the GPU path of the generator)."""
    import torch
    table_np = normal_table(dtype)
    if dtype == "bf16":
        table = torch.from_numpy(table_np.view(np.int16).copy()).to(device).view(torch.bfloat16)
    else:
        table = torch.from_numpy(table_np.copy()).to(device)
    out = torch.empty(count, dtype=_torch_dtype(dtype), device=device)
    for c0 in range(0, count, _CHUNK):
        n = min(_CHUNK, count - c0)
        e = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=device)
        x = (_mul32(e & _M32, _GOLDEN) + key) & _M32
        idx = _hash32(x) >> 16
        out[c0:c0 + n] = table[idx]
        del e, x, idx
    return out


def _source_rows(w: Workload, kind: int, source: int, start: int, n: int, device):
    row = w.n_kv_heads * w.head_dim
    flat = _draw(_key(w.seed, kind, source), start * row, n * row, w.dtype, device)
    return flat.view(n, w.n_kv_heads, w.head_dim)


def kv_rows(w: Workload, seq: int, start: int, n: int, device="cpu"):
    """K and V of logical positions start..start+n-1 of sequence ``seq``: two [n, Hk, D] tensors."""
    import torch
    ks, vs = [], []
    pos = 0
    for (src, s0, cnt) in w.segments[seq]:
        lo, hi = max(start, pos), min(start + n, pos + cnt)
        if lo < hi:
            ks.append(_source_rows(w, _KIND_K, src, s0 + lo - pos, hi - lo, device))
            vs.append(_source_rows(w, _KIND_V, src, s0 + lo - pos, hi - lo, device))
        pos += cnt
    if pos < start + n:
        raise ValueError(f"sequence {seq} has only {pos} logical positions")
    if not ks:
        shape = (0, w.n_kv_heads, w.head_dim)
        return (torch.empty(shape, dtype=_torch_dtype(w.dtype), device=device),
                torch.empty(shape, dtype=_torch_dtype(w.dtype), device=device))
    return torch.cat(ks), torch.cat(vs)


def logical_kv(w: Workload, row: int, device="cpu"):
    """The whole logical K/V of batch row ``row`` (seq_lens[row] positions)."""
    return kv_rows(w, int(w.batch[row]), 0, int(w.seq_lens[row]), device)


def q_values(w: Workload, device="cpu"):
    """Decode queries [S, Hq, D] in the storage dtype."""
    S, per = w.num_seqs, w.n_q_heads * w.head_dim
    flat = _draw(_key(w.seed, _KIND_Q, 0), 0, S * per, w.dtype, device)
    return flat.view(S, w.n_q_heads, w.head_dim)


def new_token_kv(w: Workload, device="cpu"):
    """K and V of each batch row's decode token (logical position seq_lens-1): [S, Hk, D] each."""
    import torch
    ks, vs = [], []
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        k, v = kv_rows(w, int(w.batch[r]), L - 1, 1, device)
        ks.append(k)
        vs.append(v)
    return torch.cat(ks), torch.cat(vs)


def storage_to_numpy(t) -> np.ndarray:
    """A CPU numpy view of a storage tensor: float32, float16, or uint16 bit patterns for bf16."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def poison_value(dtype: str):
    """The bit pattern (as a python int) of a quiet NaN in the storage dtype, for pool poisoning."""
    return {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}[dtype]
