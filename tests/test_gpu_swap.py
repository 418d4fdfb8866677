"""GPU parity of swapping to host memory (pkv_swap_blocks with the allocator's swap pairs).

Block moves between a device pool and pinned host swap space are compared with the oracle's
move_blocks bit for bit, both ways.  Through the runtime, rows swapped out, overwritten in the device
pool by other sequences and swapped back in decode to the very same bits as before (the summation
order depends only on logical positions), and within tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import TOL, TORCH_DTYPE, log, max_abs_err, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt,B", [(torch.bfloat16, 16), (torch.float16, 8), (torch.float8_e4m3fn, 32)])
def test_swap_blocks_bit_exact_vs_oracle(dt, B):
    from oracle import scatter as SC
    N, H, Hk, D = 64, 40, 4, 128
    ks = pkv.key_pool_shape(N, Hk, D, B, dt)
    vs = pkv.value_pool_shape(N, Hk, D, B)
    hks = pkv.key_pool_shape(H, Hk, D, B, dt)
    hvs = pkv.value_pool_shape(H, Hk, D, B)
    ib = torch.uint8 if dt == torch.float8_e4m3fn else torch.int16
    gen = torch.Generator().manual_seed(5)
    rnd = lambda shape: torch.randint(0, 120 if ib == torch.uint8 else 30000, shape, generator=gen).to(ib)
    kp, vp = rnd(ks).cuda().view(dt), rnd(vs).cuda().view(dt)
    kh = torch.full(hks, 0x7F if ib == torch.uint8 else 0x7FC1, dtype=ib).pin_memory().view(dt)
    vh = torch.full(hvs, 0x7F if ib == torch.uint8 else 0x7FC1, dtype=ib).pin_memory().view(dt)
    np_ = lambda t: t.view(ib).cpu().numpy().copy()
    okp, ovp, okh, ovh = np_(kp), np_(vp), np_(kh), np_(vh)
    rng = np.random.default_rng(B)
    out_pairs = np.stack([rng.permutation(N)[:30], rng.permutation(H)[:30]], 1).astype(np.int32)
    out_pairs[4] = (N + 3, 0)                       # out of range: skipped
    pk = torch.from_numpy(out_pairs).cuda()
    pkv.swap_blocks(pk, kp, vp, kh, vh)             # pool -> host
    torch.cuda.synchronize()
    SC.move_blocks(okp, ovp, okh, ovh, out_pairs)
    assert np.array_equal(np_(kh), okh) and np.array_equal(np_(vh), ovh)
    in_pairs = np.stack([rng.permutation(H)[:25], rng.permutation(N)[:25]], 1).astype(np.int32)
    pin = torch.from_numpy(in_pairs).pin_memory()   # pairs in pinned host memory work too
    pkv.swap_blocks(pin, kh, vh, kp, vp)            # host -> pool
    torch.cuda.synchronize()
    SC.move_blocks(okh, ovh, okp, ovp, in_pairs)
    assert np.array_equal(np_(kp), okp) and np.array_equal(np_(vp), ovp)


def test_swap_rejects_pageable_host_memory():
    N, Hk, D, B, dt = 8, 2, 64, 16, torch.bfloat16
    kp = torch.zeros(pkv.key_pool_shape(N, Hk, D, B, dt), dtype=dt, device="cuda")
    vp = torch.zeros(pkv.value_pool_shape(N, Hk, D, B), dtype=dt, device="cuda")
    kh = torch.zeros(pkv.key_pool_shape(N, Hk, D, B, dt), dtype=dt)     # pageable: not reachable by a kernel
    vh = torch.zeros(pkv.value_pool_shape(N, Hk, D, B), dtype=dt)
    pairs = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PKVError) as e:
        pkv.swap_blocks(pairs, kp, vp, kh, vh)
    assert e.value.status == pkv.PKV_ERR_INVALID


def _runtime_batch(w, slack_blocks):
    from paged_kv_cache_53_amd.runtime import DecodeBatch, PagedKVCache
    dt = TORCH_DTYPE[w.dtype]
    cache = PagedKVCache(w.num_blocks + slack_blocks, w.block_size, w.n_kv_heads, w.head_dim, dt,
                         free_order=list(range(w.num_blocks + slack_blocks)), fill="nan")
    for op in w.prompt_ops:
        if op["op"] == "alloc":
            k, v = wl.kv_rows(w, op["seq"], op["pos"], op["n"], device="cuda")
            cache.append(op["seq"], k, v)
        elif op["op"] == "fork":
            cache.fork(op["parent"], op["child"], op["n"])
        else:
            cache.free(op["seq"])
    kn, vn = wl.new_token_kv(w, device="cuda")
    for r, seq in enumerate(w.batch.tolist()):
        cache.append(seq, kn[r:r + 1], vn[r:r + 1])
    batch = DecodeBatch(cache, w.batch.tolist(), w.n_q_heads, w.max_seq_len, partition_size=w.partition_size,
                        scale=w.scale)
    return cache, batch


@pytest.mark.parametrize("cid", [3, 4])
def test_swapped_rows_decode_to_the_same_bits(cid):
    w = wl.build(cid, small=True)
    # rows of the shared-prefix workload come back with private copies of the prefix: room for them
    cache, batch = _runtime_batch(w, slack_blocks=80)
    cache.enable_swap(2 * w.num_blocks)
    q = wl.q_values(w, device="cuda").contiguous()
    out0 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    batch.decode_only(q, out0)
    rows = [1, 3]
    moved = sum(cache.swap_out(int(w.batch[r])) for r in rows)
    st = cache.allocator.swap_stats()
    assert st["swapped_seqs"] == 2 and st["host_free"] == 2 * w.num_blocks - moved
    # other sequences take the freed blocks and overwrite them
    free = cache.allocator.stats()["free_blocks"]
    junk = torch.full((free * w.block_size, w.n_kv_heads, w.head_dim), float("nan"), dtype=TORCH_DTYPE[w.dtype],
                      device="cuda")
    cache.append(10 ** 6, junk, junk)
    assert cache.allocator.stats()["free_blocks"] == 0
    cache.free(10 ** 6)
    for r in rows:
        cache.swap_in(int(w.batch[r]))
    batch.refresh()
    out1 = torch.empty_like(out0)
    batch.decode_only(q, out1)
    torch.cuda.synchronize()
    assert torch.equal(out0.view(torch.int32), out1.view(torch.int32))
    ref = oracle_rows(w, range(w.num_seqs))
    err = max_abs_err(out1, ref, rows=range(w.num_seqs))
    log(f"config {cid} small: swapped rows {rows} ({moved} blocks) decode identically; err {err:.3e}")
    assert err <= TOL[w.dtype]
