"""Pins of the scatter (O3) and decode attention (O4) oracles.

They are checked against things other than themselves: hand-computed flat offsets of the
documented pool layout, a per-token brute force that follows the block table with math.fsum,
torch's scaled_dot_product_attention in fp64, closed forms (L = 1, constant V, uniform
weights, a dominant key), placement and sharing invariance, and overflow stability.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as O
from oracle import scatter as SC
from oracle.allocator import BlockAllocatorModel


def _np_storage(dtype):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def build_oracle_pools(w, poison=True):
    """Run the workload's prompt script and decode step through the oracle: pools, tables, q."""
    a = BlockAllocatorModel(w.num_blocks, w.block_size, w.free_order)
    kp, vp = SC.empty_pools(w.num_blocks, w.n_kv_heads, w.head_dim, w.block_size,
                            _np_storage(w.dtype), wl.poison_value(w.dtype) if poison else 0)
    lens = {}
    for op in w.prompt_ops:
        if op["op"] == "alloc":
            slots, pairs = a.alloc(op["seq"], op["n"])
            assert not pairs
            k, v = wl.kv_rows(w, op["seq"], op["pos"], op["n"])
            SC.reshape_and_cache(wl.storage_to_numpy(k), wl.storage_to_numpy(v), np.array(slots), kp, vp)
        elif op["op"] == "fork":
            a.fork(op["parent"], op["child"], op["n"])
        else:
            a.free_seq(op["seq"])
    new_slots = []
    for seq in w.batch.tolist():
        s, pairs = a.alloc(seq, 1)
        assert not pairs
        new_slots += s
    kn, vn = wl.new_token_kv(w)
    SC.reshape_and_cache(wl.storage_to_numpy(kn), wl.storage_to_numpy(vn), np.array(new_slots), kp, vp)
    maxb = max(1, max(len(a.block_table(int(s))) for s in w.batch))
    tables = np.full((w.num_seqs, maxb), -7, dtype=np.int64)   # entries past ceil(L/B): garbage
    for r, seq in enumerate(w.batch.tolist()):
        t = a.block_table(seq)
        tables[r, :len(t)] = t
        assert a.seq_len(seq) == int(w.seq_lens[r])
    q = wl.storage_to_numpy(wl.q_values(w))
    return a, kp, vp, tables, q


# ---------------------------------------------------------------------------- scatter
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f16", 128), ("bf16", 128)])
def test_layout_flat_offsets(dtype, D):
    """The documented layouts, by hand: element (blk,h,c,off,e) of K and (blk,h,d,off) of V."""
    N, Hk, B = 5, 3, 8
    esize = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    x = 16 // esize
    kp, vp = SC.empty_pools(N, Hk, D, B, _np_storage(dtype), 0)
    rng = np.random.default_rng(0)
    ui = {2: np.uint16, 4: np.uint32}[esize]
    k = rng.integers(1, 2 ** (8 * esize) - 1, size=(2, Hk, D), dtype=np.uint64).astype(ui)
    v = rng.integers(1, 2 ** (8 * esize) - 1, size=(2, Hk, D), dtype=np.uint64).astype(ui)
    slots = np.array([3 * B + 5, 0 * B + 7])
    SC.reshape_and_cache(k.view(kp.dtype), v.view(vp.dtype), slots, kp, vp)
    kflat, vflat = kp.view(ui).reshape(-1), vp.view(ui).reshape(-1)
    for t, s in enumerate(slots):
        blk, off = divmod(int(s), B)
        for h in range(Hk):
            for d in range(D):
                c, e = divmod(d, x)
                kidx = (((blk * Hk + h) * (D // x) + c) * B + off) * x + e
                vidx = ((blk * Hk + h) * D + d) * B + off
                assert kflat[kidx] == k[t, h, d]
                assert vflat[vidx] == v[t, h, d]
    assert np.count_nonzero(kflat) == 2 * Hk * D and np.count_nonzero(vflat) == 2 * Hk * D


def test_scatter_bit_exact_specials_and_skips():
    N, Hk, D, B = 4, 2, 16, 4
    kp, vp = SC.empty_pools(N, Hk, D, B, np.uint16, 0x7E00)
    k = np.zeros((3, Hk, D), np.uint16)
    v = np.zeros((3, Hk, D), np.uint16)
    k[0, 0, 0] = 0x8000          # -0.0
    k[1, 1, 3] = 0x7D01          # signalling NaN payload
    v[1, 0, 5] = 0xFC00          # -inf
    SC.reshape_and_cache(k, v, np.array([5, 14, -1]), kp, vp)
    Kl, Vl = SC.gather_logical(kp, vp, [1, 3], 8)
    assert Kl[1, 0, 0] == 0x8000 and Kl[6, 1, 3] == 0x7D01 and Vl[6, 0, 5] == 0xFC00
    untouched = [b for b in range(N) if b not in (1, 3)]
    assert np.all(kp[untouched].view(np.uint16) == 0x7E00)
    # slot 13 (block 3, token 1) was never written: still poison
    assert np.all(kp[3, :, :, 1, :] == 0x7E00)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_scatter_round_trip_through_tables(cid):
    w = wl.build(cid, small=True)
    a, kp, vp, tables, q = build_oracle_pools(w)
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        K, V = SC.gather_logical(kp, vp, tables[r], L)
        Kw, Vw = wl.logical_kv(w, r)
        Kw, Vw = wl.storage_to_numpy(Kw), wl.storage_to_numpy(Vw)
        assert np.array_equal(K.view(np.uint8), Kw.view(np.uint8))
        assert np.array_equal(V.view(np.uint8), Vw.view(np.uint8))


# ---------------------------------------------------------------------------- attention
def brute_force(q, kp, vp, tables, seq_lens, scale, dtype):
    """Per-token loops with math.exp / math.fsum, reading pool elements through the table."""
    N, Hk, C, B, x = kp.shape
    D = C * x
    S, Hq, _ = q.shape
    G = Hq // Hk
    dec = lambda a: O.to_f64(np.asarray(a), dtype).reshape(-1).tolist()
    out = np.zeros((S, Hq, D))
    for s in range(S):
        L = int(seq_lens[s])
        for h in range(Hq):
            kv = h // G
            qv = dec(q[s, h])
            xs, vrows = [], []
            for j in range(L):
                blk, off = int(tables[s][j // B]), j % B
                krow = dec(kp[blk, kv, :, off, :])
                xs.append(scale * math.fsum(a * b for a, b in zip(qv, krow)))
                vrows.append(dec(vp[blk, kv, :, off]))
            if L == 0:
                continue
            m = max(xs)
            p = [math.exp(t - m) for t in xs]
            den = math.fsum(p)
            for d in range(D):
                out[s, h, d] = math.fsum(p[j] * vrows[j][d] for j in range(L)) / den
    return out


def test_brute_force_tiny_config():
    w = wl.build(1)
    a, kp, vp, tables, q = build_oracle_pools(w)
    got = O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    ref = brute_force(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_brute_force_gqa_bf16_ragged():
    w = wl.custom(seed=11, lens=[1, 9, 31, 40], n_q_heads=4, n_kv_heads=2, head_dim=16,
                  block_size=8, dtype="bf16")
    a, kp, vp, tables, q = build_oracle_pools(w)
    got = O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    ref = brute_force(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_length_one_returns_v0_exactly():
    w = wl.build(1)
    a, kp, vp, tables, q = build_oracle_pools(w)
    got = O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    assert w.seq_lens[0] == 1
    K, V = SC.gather_logical(kp, vp, tables[0], 1)
    assert np.array_equal(got[0], O.to_f64(V[0], "f32"))


def _sdpa(q64, K64, V64, scale):
    """torch's SDPA in fp64 on CPU with GQA (kv head h // G) as the independent reference."""
    qt = torch.from_numpy(q64)[None, :, None, :]            # [1, Hq, 1, D]
    kt = torch.from_numpy(K64).permute(1, 0, 2)[None]       # [1, Hk, L, D]
    vt = torch.from_numpy(V64).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_matches_sdpa_fp64(cid):
    w = wl.build(cid, small=True)
    a, kp, vp, tables, q = build_oracle_pools(w)
    got = O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    for r in range(w.num_seqs):
        Kw, Vw = wl.logical_kv(w, r)
        ref = _sdpa(O.to_f64(q[r], w.dtype), O.to_f64(wl.storage_to_numpy(Kw), w.dtype),
                    O.to_f64(wl.storage_to_numpy(Vw), w.dtype), w.scale)
        assert np.max(np.abs(got[r] - ref)) <= 1e-12


def test_closed_forms():
    rng = np.random.default_rng(3)
    Hq, Hk, D, L = 4, 2, 8, 37
    K = rng.standard_normal((L, Hk, D))
    V = rng.standard_normal((L, Hk, D))
    q = rng.standard_normal((Hq, D))
    # q = 0: every weight equal -> mean of V's rows
    o = O.attention_logical(np.zeros_like(q), K, V, 0.3)
    assert np.allclose(o, np.repeat(V.mean(axis=0), 2, axis=0), atol=1e-14)
    # all K rows equal -> uniform weights too
    Keq = np.broadcast_to(K[:1], K.shape).copy()
    o = O.attention_logical(q, Keq, V, 0.3)
    assert np.allclose(o, np.repeat(V.mean(axis=0), 2, axis=0), atol=1e-14)
    # V constant c -> c
    Vc = np.full_like(V, 1.75)
    o = O.attention_logical(q, K, Vc, 0.3)
    assert np.allclose(o, 1.75, atol=1e-14, rtol=0)
    # one key aligned with q and 100x longer dominates: output = its V row up to exp(-gap)
    K2 = K.copy()
    j = 20
    K2[j, 0, :] = 100 * q[0] / np.linalg.norm(q[0])
    o = O.attention_logical(q[:1].repeat(2, axis=0), K2, V, 1.0)
    assert np.allclose(o[0], V[j, 0], atol=1e-20 + 1e-6)
    # GQA grouping: head h reads kv head h // G (consecutive)
    o = O.attention_logical(q, K, V, 0.5)
    for h in range(Hq):
        solo = O.attention_logical(q[h:h + 1], K[:, h // 2: h // 2 + 1], V[:, h // 2: h // 2 + 1], 0.5)
        assert np.allclose(o[h], solo[0], atol=1e-15, rtol=0)
    # L = 0 -> zeros
    assert np.array_equal(O.attention_logical(q, K[:0], V[:0], 0.5), np.zeros((Hq, D)))


def test_overflow_stable():
    w = wl.build(3, small=True)
    a, kp, vp, tables, q = build_oracle_pools(w)
    q64 = O.to_f64(q, w.dtype) * 1000.0
    for r in range(w.num_seqs):
        K, V = SC.gather_logical(kp, vp, tables[r], int(w.seq_lens[r]))
        o = O.attention_logical(q64[r], O.to_f64(K, w.dtype), O.to_f64(V, w.dtype), w.scale)
        assert np.all(np.isfinite(o))
        # a convex combination of V rows stays inside their range
        Vf = O.to_f64(V, w.dtype)
        assert np.all(o <= Vf.max() + 1e-12) and np.all(o >= Vf.min() - 1e-12)


def test_placement_invariance_and_shared_prefix():
    ws = [wl.build(3, small=True, placement="random"), wl.build(3, small=True, placement="identity")]
    outs = []
    for w in ws:
        a, kp, vp, tables, q = build_oracle_pools(w)
        outs.append(O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype))
    assert np.array_equal(outs[0], outs[1])
    shared, copied = wl.build(4, small=True), wl.build(4, small=True, copied_prefix=True)
    outs = []
    for w in (shared, copied):
        a, kp, vp, tables, q = build_oracle_pools(w)
        outs.append(O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype))
    assert np.array_equal(outs[0], outs[1])
    a, *_ = build_oracle_pools(shared)
    prefix_blocks = 400 // 16
    assert a.stats()["shared_blocks"] == prefix_blocks


def test_poisoned_table_tail_and_slots_never_read():
    w = wl.build(2, small=True)
    a, kp, vp, tables, q = build_oracle_pools(w, poison=True)
    got = O.paged_attention_decode(q, kp, vp, tables, w.seq_lens, w.scale, w.dtype)
    assert np.all(np.isfinite(got))
