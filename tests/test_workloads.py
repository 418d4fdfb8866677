"""The seeded input generator: determinism, shapes, distributions, random access."""
import math

import numpy as np
import pytest
import torch

import workloads as wl


def test_hash_reference_values():
    # lowbias32 of a few inputs, computed with exact python integers from its published steps
    def lowbias32(x):
        x &= 0xFFFFFFFF
        x ^= x >> 16
        x = (x * 0x7FEB352D) & 0xFFFFFFFF
        x ^= x >> 15
        x = (x * 0x846CA68B) & 0xFFFFFFFF
        x ^= x >> 16
        return x
    xs = torch.tensor([0, 1, 2, 0xDEADBEEF, 0xFFFFFFFF, 123456789], dtype=torch.int64)
    got = wl._hash32(xs).tolist()
    assert got == [lowbias32(int(x)) for x in xs]
    assert got[0] == 0  # zero is the fixed point of the xor-shift-multiply chain


def test_normal_table():
    t32 = wl.normal_table("f32")
    assert t32.shape == (65536,) and np.all(np.diff(t32) >= 0)
    assert np.allclose(t32, -t32[::-1], atol=1e-6)          # symmetric quantiles
    assert abs(float(t32.astype(np.float64).mean())) < 1e-6
    assert abs(float(t32.astype(np.float64).var()) - 1.0) < 2e-3
    bf = wl.normal_table("bf16")
    back = (bf.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - t32) <= np.abs(t32) * 2 ** -8 + 1e-30)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_build_is_deterministic(cid):
    a, b = wl.build(cid), wl.build(cid)
    assert np.array_equal(a.seq_lens, b.seq_lens)
    assert np.array_equal(a.free_order, b.free_order)
    assert a.prompt_ops == b.prompt_ops
    assert sorted(a.free_order.tolist()) == list(range(a.num_blocks))


def test_config_shapes():
    c1 = wl.build(1)
    assert c1.seq_lens.tolist() == [1, 17, 33, 100] and c1.num_blocks == 64
    assert (c1.n_q_heads, c1.n_kv_heads, c1.head_dim, c1.dtype, c1.block_size) == (4, 4, 64, "f32", 16)
    assert c1.scale == 1 / 8
    c2 = wl.build(2)
    assert c2.num_seqs == 32 and c2.num_blocks == 8192 and c2.dtype == "f16"
    assert c2.seq_lens.min() >= 128 and c2.seq_lens.max() <= 2048
    c3 = wl.build(3)
    assert c3.num_seqs == 256 and (c3.n_q_heads, c3.n_kv_heads) == (64, 8) and c3.dtype == "bf16"
    assert c3.seq_lens.min() >= 16 and c3.seq_lens.max() <= 32768
    need = sum(math.ceil(int(L) / 16) for L in c3.seq_lens)
    assert c3.num_blocks == math.ceil(1.1 * need)
    med = float(np.median(c3.seq_lens))
    assert 2000 < med < 4500                       # median 3000 log-normal
    c4 = wl.build(4)
    assert c4.num_seqs == 20 and (c4.seq_lens >= 4001).all() and (c4.seq_lens <= 16001).all()
    forks = [op for op in c4.prompt_ops if op["op"] == "fork"]
    assert len(forks) == 20 and all(op["n"] == 4000 for op in forks)
    for B in (8, 16, 32):
        c5 = wl.build(5, block_size=B)
        assert c5.seq_lens.tolist() == [65536] * 8 and c5.block_size == B
    ident = wl.build(5, placement="identity")
    assert np.array_equal(ident.free_order, np.arange(ident.num_blocks))


def test_values_random_access_and_segments():
    w = wl.build(4, small=True)
    K, V = wl.logical_kv(w, 2)
    L = int(w.seq_lens[2])
    assert K.shape == (L, 8, 128) and K.dtype == torch.float16
    n = L - 100
    k2, v2 = wl.kv_rows(w, 2, 100, n)
    assert n > 300 and torch.equal(k2, K[100:]) and torch.equal(v2, V[100:])
    with pytest.raises(ValueError):
        wl.kv_rows(w, 2, 0, L + 1)
    # the shared prompt is the same values in every child
    K0, _ = wl.logical_kv(w, 0)
    assert torch.equal(K0[:400], K[:400])
    assert not torch.equal(K0[400:401], K[400:401])
    # K and V streams differ; q is [S, Hq, D]
    assert not torch.equal(K, V)
    assert wl.q_values(w).shape == (w.num_seqs, 32, 128)


def test_values_are_standard_normal():
    w = wl.build(3, small=True)
    K, V = wl.logical_kv(w, 0)
    x = K.float().reshape(-1)
    assert abs(x.mean().item()) < 0.05 and abs(x.std().item() - 1) < 0.05
    assert x.abs().max().item() < 4.4


def test_bf16_storage_view_round_trip():
    t = torch.tensor([1.0, -0.0, 3.140625], dtype=torch.bfloat16)
    n = wl.storage_to_numpy(t)
    assert n.dtype == np.uint16 and n.tolist() == [0x3F80, 0x8000, 0x4049]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_host_draw_equals_int64_draw(dtype):
    # the host's uint32 generator and the int64 form the GPU runs give the same elements, across
    # chunk boundaries, at offsets past 2^32 (element counters wrap mod 2^32) and in the threaded case
    key = wl._key(7, 2, 3)
    for start, count in ((0, 1), (123, 1000), ((1 << 32) - 700, 2000), (5, 5 * wl._CPU_CHUNK + 17)):
        a = wl._draw(key, start, count, dtype, "cpu")
        b = wl._draw_torch(key, start, count, dtype, "cpu")
        assert a.dtype == b.dtype and a.shape == b.shape
        bits = torch.int32 if dtype == "f32" else torch.int16
        assert torch.equal(a.view(bits), b.view(bits)), (start, count)
